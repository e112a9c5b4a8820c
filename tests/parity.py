"""Run the HIP path through the C ABI and compare every stage with the CPU oracle.

Used by the GPU parity tests and by the smoke check.  Inputs come from moe_synth (shared by both
sides); expected values come only from the oracle.

Bars: bit-exact for indices, counts, offsets, positions, metadata and payload bytes; router
weights within 1 fp32 ulp of the fp64 oracle; combine output bit-exact against the oracle's
fp32 fused-multiply-add chain (same operations in the same order) wherever the two sides' weights
agree bit for bit, and within 1 bf16 ulp of the oracle's fp64 sum everywhere (identity and
tagged experts: all terms of a sum share a sign).
"""
from __future__ import annotations

import numpy as np
import torch

import moe_synth as ms
import oracle


def _np(t):
    if t.dtype == torch.int16:
        return t.cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def upload_inputs(b, inp):
    b.logits.copy_(torch.from_numpy(inp["logits"]))
    if inp["bias"] is not None:
        b.bias.copy_(torch.from_numpy(inp["bias"]))
    x = inp["x"]
    b.x.copy_(torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x))
    if inp["x_scale"] is not None:
        b.x_scale.copy_(torch.from_numpy(inp["x_scale"]))


def gpu_run(N, T, H, E, R, fp8, inp, expert_mode=0, capacity=0, y=None, topk_idx=None,
            poison=True, split_combine=False, quant=False, tokens=None):
    """The whole path on the GPU.  Returns (buffers, host copies of every valid output).
    quant: inp["x"] holds bf16 tokens that the send pack quantises to e4m3 rows; tokens: the
    per-rank token counts (int array of N), or None."""
    import combine_moe_route_top_amd as moe
    b = moe.alloc_buffers(N, T, H, E, R, fp8, capacity, quant=quant, tokens=tokens is not None)
    if poison:  # garbage in every output so that stale values cannot pass for results
        for k, t in b.t.items():
            if t is not None and k not in ("status", "tokens"):
                t.view(torch.uint8).fill_(0xA5)
        b.status.zero_()
    if tokens is not None:
        b.tokens.copy_(torch.from_numpy(np.ascontiguousarray(tokens, np.int32)))
    upload_inputs(b, inp)
    if topk_idx is None:
        moe.moe_route(b.shape, b.logits, b.bias if inp["bias"] is not None else None,
                      b.topk_idx, b.topk_w)
    else:
        b.topk_idx.copy_(torch.from_numpy(np.ascontiguousarray(topk_idx, np.int32).reshape(N, -1)))
        b.topk_w.fill_(1.0 / R)
    moe.moe_dispatch_send(b.shape, b.x, b.x_scale, b.topk_idx, b.counts, b.send_off, b.send_pos,
                          b.send_buf, b.send_meta, b.workspace)
    moe.moe_net_dispatch(b.shape, b.send_off, b.send_buf, b.send_meta, b.recv_buf, b.recv_meta,
                         b.recv_off)
    moe.moe_dispatch_recv(b.shape, b.counts, b.recv_off, b.recv_buf, b.recv_meta, b.expert_x,
                          b.expert_scale, b.expert_cnt, b.expert_off, b.expert_src, b.expert_rpos)
    if y is None:
        moe.moe_expert_stub(b.shape, expert_mode, b.expert_x, b.expert_scale, b.expert_off,
                            b.expert_y)
    else:
        b.expert_y.copy_(torch.from_numpy(y.view(np.int16)))
    if split_combine:  # the two halves, with a second stream between them
        moe.moe_combine_send(b.shape, b.expert_y, b.expert_rpos, b.recv_off, b.send_off, b.cs_buf,
                             b.cr_buf)
        ev = torch.cuda.Event()
        ev.record()
        side = torch.cuda.Stream()
        side.wait_event(ev)
        moe.moe_combine_recv(b.shape, b.cr_buf, b.send_pos, b.topk_w, b.out, side)
        torch.cuda.current_stream().wait_stream(side)
    else:
        moe.run_combine(b)
    torch.cuda.synchronize()
    g = fetch(b, N, T, R)
    g["poisoned"] = poison
    return b, g


def fetch(b, N, T, R):
    """Host copies of the valid part of every output (rows past a rank's totals are undefined)."""
    g = {k: _np(getattr(b, k)) for k in ("topk_idx", "topk_w", "counts", "send_off", "send_pos",
                                          "recv_off", "expert_cnt", "expert_off", "out", "status")}
    so, ro = g["send_off"], g["recv_off"]
    g["send_rows"] = [_np(b.send_buf[s, :so[s, N]]) for s in range(N)]
    g["send_meta"] = [_np(b.send_meta[s, :so[s, N]]) for s in range(N)]
    g["recv_rows"] = [_np(b.recv_buf[d, :ro[d, N]]) for d in range(N)]
    g["recv_meta"] = [_np(b.recv_meta[d, :ro[d, N]]) for d in range(N)]
    g["expert_x"] = [_np(b.expert_x[d, :ro[d, N]]) for d in range(N)]
    if b.expert_scale is not None:
        g["expert_scale"] = [_np(b.expert_scale[d, :ro[d, N]]) for d in range(N)]
    g["expert_src"] = [_np(b.expert_src[d, :ro[d, N]]) for d in range(N)]
    g["expert_rpos"] = [_np(b.expert_rpos[d, :ro[d, N]]) for d in range(N)]
    g["expert_y"] = [_np(b.expert_y[d, :ro[d, N]]) for d in range(N)]
    g["cs_buf"] = [_np(b.cs_buf[d, :ro[d, N]]) for d in range(N)]
    g["cr_buf"] = [_np(b.cr_buf[s, :so[s, N]]) for s in range(N)]
    return g


def oracle_run(N, T, H, E, R, fp8, inp, expert_mode=0, y=None, topk_idx=None, quant=False,
               tokens=None):
    """The oracle on the same inputs, packed receive layout (rank d holds exactly its rows).
    quant: the oracle's block quantiser turns the bf16 tokens into e4m3 codes and scales, then
    the e4m3 path runs on them."""
    if quant:
        q, sc = oracle.quantize_e4m3(inp["x"])
        inp = dict(inp, x=q, x_scale=sc)
        fp8 = True
    sh = oracle.shape(N, T, H, E, R, fp8, tokens=tokens)
    if topk_idx is None:
        idx, w = oracle.route(inp["logits"], inp["bias"], R)
    else:
        idx = np.ascontiguousarray(topk_idx, np.int32).reshape(N * T, R)
        w = np.full((N * T, R), np.float32(1.0 / R), np.float32)
    res = dict(topk_idx=idx, topk_w=w)
    res.update(oracle.dispatch_send(sh, inp["x"], inp["x_scale"], idx.reshape(N, T * R)))
    recv_rows = np.diff(res["send_off"], axis=1).sum(axis=0)
    sh = oracle.packed_shape(N, T, H, E, R, fp8, recv_rows, tokens)
    res.update(oracle.net_dispatch(sh, res["send_off"], res["send_buf"], res["send_meta"]))
    res.update(oracle.dispatch_recv(sh, res["counts"], res["recv_off"], res["recv_buf"],
                                    res["recv_meta"]))
    if y is None:
        res["expert_y"] = oracle.expert(sh, expert_mode, res["expert_x"], res["expert_scale"],
                                        res["expert_off"])
    else:
        res["expert_y"] = np.ascontiguousarray(
            np.concatenate([y[d, :recv_rows[d]] for d in range(N)]), np.uint16)
    for mode in (0, 1):
        c = oracle.combine(sh, mode, res["expert_y"], res["expert_rpos"], res["recv_off"],
                           res["send_off"], res["send_pos"], w)
        res[f"out{mode}"] = c["out"]
        if mode == 0:
            res["cs_buf"], res["cr_buf"] = c["cs_buf"], c["cr_buf"]
    res["shape"] = sh
    res["tokens"] = None if tokens is None else np.asarray(tokens)
    return res


def _bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 representable steps between two bf16 bit arrays (same-sign values)."""
    def key(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u & 0x7FFF)
    return np.abs(key(a) - key(b))


def compare(g: dict, o: dict, N, T, H, E, R, fp8, check_stub=True, check_ulp=True) -> dict:
    """Assert every stage's parity; returns a few statistics."""
    sh = o["shape"]
    TR = T * R
    stats = {}
    assert g["status"][0] == 0, f"device status word {g['status'][0]}"
    # tokens present on each rank (all T unless per-rank counts were given); rows of absent
    # tokens must keep the poison the outputs were filled with
    nt = np.full(N, T) if o.get("tokens") is None else np.asarray(o["tokens"])
    present = (np.arange(T)[None, :] < nt[:, None]).reshape(N * T)
    gi = g["topk_idx"].reshape(N * T, R)
    if not present.all() and g.get("poisoned"):
        assert np.all(gi[~present].view(np.uint32) == 0xA5A5A5A5), "route wrote absent tokens"
        assert np.all(g["out"].reshape(N * T, H)[~present] == 0xA5A5), "combine wrote absent tokens"
    assert np.array_equal(gi[present], o["topk_idx"][present]), "topk_idx"
    gw, ow = g["topk_w"].reshape(N * T, R)[present], o["topk_w"][present]
    ulp = np.abs(gw.view(np.int32).astype(np.int64) - ow.view(np.int32).astype(np.int64))
    assert ulp.max(initial=0) <= 1, f"topk_w differs by {ulp.max()} fp32 ulp"
    stats["w_exact"] = float((ulp == 0).mean()) if ulp.size else 1.0
    assert np.array_equal(g["counts"], o["counts"]), "counts"
    assert np.array_equal(g["send_off"], o["send_off"]), "send_off"
    assert np.array_equal(g["send_pos"], o["send_pos"]), "send_pos"
    for s in range(N):
        n = o["send_off"][s, N]
        assert np.array_equal(g["send_rows"][s], o["send_buf"][s, :n]), f"send_buf rank {s}"
        assert np.array_equal(g["send_meta"][s], o["send_meta"][s, :n]), f"send_meta rank {s}"
    assert np.array_equal(g["recv_off"], o["recv_off"]), "recv_off"
    assert np.array_equal(g["expert_cnt"], o["expert_cnt"]), "expert_cnt"
    assert np.array_equal(g["expert_off"], o["expert_off"]), "expert_off"
    for d in range(N):
        assert np.array_equal(g["recv_rows"][d], sh.rank_rows(o["recv_buf"], d)), f"recv_buf rank {d}"
        assert np.array_equal(g["recv_meta"][d], sh.rank_rows(o["recv_meta"], d)), f"recv_meta rank {d}"
        assert np.array_equal(g["expert_x"][d], sh.rank_rows(o["expert_x"], d)), f"expert_x rank {d}"
        if fp8:
            assert np.array_equal(g["expert_scale"][d], sh.rank_rows(o["expert_scale"], d)), \
                f"expert_scale rank {d}"
        assert np.array_equal(g["expert_src"][d], sh.rank_rows(o["expert_src"], d)), f"expert_src rank {d}"
        assert np.array_equal(g["expert_rpos"][d], sh.rank_rows(o["expert_rpos"], d)), f"expert_rpos rank {d}"
        if check_stub:
            assert np.array_equal(g["expert_y"][d], sh.rank_rows(o["expert_y"], d)), f"expert_y rank {d}"
        assert np.array_equal(g["cs_buf"][d], sh.rank_rows(o["cs_buf"], d)), f"cs_buf rank {d}"
    for s in range(N):
        n = o["send_off"][s, N]
        assert np.array_equal(g["cr_buf"][s], o["cr_buf"][s, :n]), f"cr_buf rank {s}"
    out = g["out"].reshape(N * T, H)[present]
    same_w = np.all(gw == ow, axis=1)
    o1 = o["out1"].reshape(N * T, H)[present]
    assert np.array_equal(out[same_w], o1[same_w]), "out vs the oracle's fp32 fma chain"
    stats["fma_chain_tokens"] = int(same_w.sum())
    if check_ulp:
        d0 = _bf16_ulp_diff(out, o["out0"].reshape(N * T, H)[present])
        assert d0.max(initial=0) <= 1, f"out differs from the fp64 oracle by {d0.max()} bf16 ulp"
        stats["out_exact_vs_fp64"] = float((d0 == 0).mean()) if d0.size else 1.0
    return stats


# ------------------------------------------------------------------ prefill (replicated tokens)


def prefill_inputs(T, H, E, R, fp8, bias, seed):
    """One replicated token set: moe_synth's inputs for a single rank, reshaped to [T][...]."""
    inp = ms.make_inputs(1, T, H, E, R, fp8, bias, seed)
    out = dict(logits=inp["logits"], bias=inp["bias"], x=inp["x"].reshape(T, H),
               x_scale=None if inp["x_scale"] is None else inp["x_scale"].reshape(T, H // 128))
    return out


def gpu_run_prefill(N, T, H, E, R, fp8, inp, expert_mode=0, capacity=0, y=None, split=False,
                    width=None):
    """The replicated-token path on the GPU; width: run every call once per range of `width`
    ranks (each step for all ranges before the next) instead of once for all ranks."""
    import combine_moe_route_top_amd as moe
    b = moe.alloc_prefill_buffers(N, T, H, E, R, fp8, capacity)
    for k, t in b.t.items():
        if t is not None and k != "status":
            t.view(torch.uint8).fill_(0xA5)
    b.status.zero_()
    upload_inputs(b, inp)
    shapes = [b.shape] if width is None else \
        [moe.for_ranks(b.shape, r0, min(width, N - r0)) for r0 in range(0, N, width)]
    use_bias = inp["bias"] is not None
    moe.moe_route(b.shape, b.logits, b.bias if use_bias else None, b.topk_idx, b.topk_w)
    for sh in shapes:
        moe.moe_prefill_dispatch(sh, b.x, b.x_scale, b.topk_idx, b.slot_pos, b.expert_x,
                                 b.expert_scale, b.expert_cnt, b.expert_off, b.expert_src,
                                 b.workspace)
    if y is None:
        for sh in shapes:
            moe.moe_expert_stub(sh, expert_mode, b.expert_x, b.expert_scale, b.expert_off,
                                b.expert_y)
    else:
        b.expert_y.copy_(torch.from_numpy(y.view(np.int16)))
    if split or width is not None:
        for sh in shapes:
            moe.moe_prefill_combine_local(sh, b.expert_y, b.topk_idx, b.slot_pos, b.topk_w,
                                          b.partial)
        moe.moe_prefill_allreduce(b.shape, b.partial, b.out)
    else:
        moe.moe_prefill_combine(b.shape, b.expert_y, b.topk_idx, b.slot_pos, b.topk_w, b.partial,
                                b.out)
    torch.cuda.synchronize()
    g = {k: _np(getattr(b, k)) for k in ("topk_idx", "topk_w", "slot_pos", "expert_cnt",
                                          "expert_off", "partial", "out", "status")}
    eo = g["expert_off"]
    for k in ("expert_x", "expert_src", "expert_y"):
        g[k] = [_np(getattr(b, k)[d, :eo[d, -1]]) for d in range(N)]
    if fp8:
        g["expert_scale"] = [_np(b.expert_scale[d, :eo[d, -1]]) for d in range(N)]
    return b, g


def oracle_run_prefill(N, T, H, E, R, fp8, inp, expert_mode=0, y=None):
    idx, w = oracle.route(inp["logits"], inp["bias"], R)
    B = T * min(R, E // N)          # the most any rank receives; keeps host arrays small
    sh = oracle.shape(N, T, H, E, R, fp8, B=B)
    res = dict(topk_idx=idx, topk_w=w, shape=sh)
    res.update(oracle.prefill_dispatch(sh, inp["x"], inp["x_scale"], idx))
    if y is None:
        res["expert_y"] = oracle.expert(sh, expert_mode, res["expert_x"], res["expert_scale"],
                                        res["expert_off"])
    else:
        res["expert_y"] = np.ascontiguousarray(y[:, :B], np.uint16)
    for mode in (0, 1):
        c = oracle.prefill_combine(sh, mode, res["expert_y"], res["slot_pos"], idx, w)
        res[f"out{mode}"] = c["out"]
        if mode == 1:
            res["partial"] = c["partial"]
    return res


def compare_prefill(g, o, N, T, H, E, R, fp8, check_stub=True, check_ulp=True):
    """Bit-exact layout and payload; partials and out bit-exact against the oracle's fp32 steps
    wherever the router weights agree bit for bit, and out within 1 bf16 ulp of the fp64 sum."""
    stats = {}
    assert g["status"][0] == 0, f"device status word {g['status'][0]}"
    assert np.array_equal(g["topk_idx"], o["topk_idx"]), "topk_idx"
    ulp = np.abs(g["topk_w"].view(np.int32).astype(np.int64) - o["topk_w"].view(np.int32).astype(np.int64))
    assert ulp.max() <= 1, f"topk_w differs by {ulp.max()} fp32 ulp"
    assert np.array_equal(g["slot_pos"], o["slot_pos"]), "slot_pos"
    assert np.array_equal(g["expert_cnt"], o["expert_cnt"]), "expert_cnt"
    assert np.array_equal(g["expert_off"], o["expert_off"]), "expert_off"
    for d in range(N):
        n = int(o["expert_off"][d, -1])
        assert np.array_equal(g["expert_x"][d], o["expert_x"][d, :n]), f"expert_x rank {d}"
        if fp8:
            assert np.array_equal(g["expert_scale"][d], o["expert_scale"][d, :n]), f"expert_scale {d}"
        assert np.array_equal(g["expert_src"][d], o["expert_src"][d, :n]), f"expert_src rank {d}"
        if check_stub:
            assert np.array_equal(g["expert_y"][d], o["expert_y"][d, :n]), f"expert_y rank {d}"
    same_w = np.all(g["topk_w"] == o["topk_w"], axis=1)
    assert np.array_equal(g["partial"][:, same_w].view(np.uint32),
                          o["partial"][:, same_w].view(np.uint32)), "partial vs fp32 steps"
    assert np.array_equal(g["out"][same_w], o["out1"][same_w]), "out vs the oracle's fp32 steps"
    stats["fp32_step_tokens"] = int(same_w.sum())
    if check_ulp:
        d0 = _bf16_ulp_diff(g["out"], o["out0"])
        assert d0.max() <= 1, f"out differs from the fp64 oracle by {d0.max()} bf16 ulp"
        stats["out_exact_vs_fp64"] = float((d0 == 0).mean())
    return stats
