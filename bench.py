"""Benchmark: MoE dispatch + combine on one MI355X (all N logical ranks in one GPU's HBM).

One step = one pass of the whole path over one batch: route -> dispatch send -> network ->
dispatch receive -> combine (shuffle, network back, weighted sum).  The stand-in expert between
dispatch and combine is not part of the metric: for bf16 identity experts it is no work at all
(combine reads the dispatched tensor), for fp8 it runs between the timed phases.

Prints ONE JSON line.  value = effective HBM GB/s of dispatch + combine = algorithmic bytes /
(dispatch + combine time), both phases timed with HIP events on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine µs/layer and effective HBM GB/s (fraction of MI355X peak)"
PEAK_HBM_GBS = 8000.0
HEADLINE = "deepseek_v3_decode"
# every workload the benchmark reports beside the headline: the other four target shapes (the
# Qwen3-shaped batch in the decode layout, 4 ranks x 4096 own tokens, as well as with replicated
# tokens), the e4m3 variants and the ragged token mix
EXTRA = ["tiny", "mixtral_8x7b_decode", "deepseek_v3_decode_fp8", "kimi_k2_worst",
         "qwen3_235b_prefill", "deepseek_v3_decode_fp8q", "deepseek_v3_decode_ragged",
         "qwen3_235b_prefill_ep"]
MALL_BYTES = 256 << 20


def exchange_fits_mall(c) -> bool:
    """The library keeps a layer's exchanged rows in the 256 MB memory-side cache between the
    network kernel and the unpack when all N*T*R rows fit (the same shape test it makes)."""
    P = (c.H + 4 * (c.H // 128)) if c.rows_fp8 else 2 * c.H
    return c.N * c.T * c.R * P <= MALL_BYTES


def alg_bytes(c) -> dict:
    """Compulsory bytes each ABI call reads and writes (every routed row is valid).  With token
    counts per rank only the present tokens count: absent ones are neither read nor written."""
    import moe_synth as ms
    N, T, H, E, R, L = c.N, c.T, c.H, c.E, c.R, c.L
    tok = ms.config_tokens(c)
    NT = N * T if tok is None else int(tok.sum())
    M = NT * R
    P = (H + 4 * (H // 128)) if c.rows_fp8 else 2 * H    # one dispatched row (codes + scales)
    xrow = 2 * H if c.quant else P                      # one input token (bf16, or codes + scales)
    Pc = 2 * H                                          # one combine row (bf16)
    bias = E * 4 if c.bias != "none" else 0
    b = {}
    b["route"] = NT * E * 4 + bias + M * 8
    b["dispatch_send"] = (M * 4 + NT * xrow) + (N * E * 4 + N * (N + 1) * 4 + M * 4 + M * 8 + M * P)
    b["net_dispatch"] = (M * (P + 8) + N * (N + 1) * 4) + (M * (P + 8) + N * (N + 1) * 4)
    b["dispatch_recv"] = (M * (P + 8) + N * E * 4 + N * (N + 1) * 4) + (M * P + M * 8 + N * (2 * L + 1) * 4)
    b["combine_pack"] = (M * Pc + M * 4 + N * (N + 1) * 4) + M * Pc
    b["combine_net"] = (M * Pc + 2 * N * (N + 1) * 4) + M * Pc
    b["combine_wsum"] = (M * Pc + M * 8) + NT * Pc
    b["combine"] = b["combine_pack"] + b["combine_net"] + b["combine_wsum"]
    b["mall_resident"] = M * (P + 8)   # the unpack's read of the exchanged rows
    b["dispatch"] = b["route"] + b["dispatch_send"] + b["net_dispatch"] + b["dispatch_recv"]
    b["total"] = b["dispatch"] + b["combine"]
    return b


def prefill_alg_bytes(c) -> dict:
    """Compulsory bytes of the replicated-token (prefill) calls: the T tokens are read once,
    every slot's row written once to its owner rank and read once by the local combine, every
    rank writes a partial of every token and the all-reduce reads them all."""
    N, T, H, E, R, L = c.N, c.T, c.H, c.E, c.R, c.L
    M = T * R
    P = (H + 4 * (H // 128)) if c.fp8 else 2 * H
    Pc = 2 * H
    bias = E * 4 if c.bias != "none" else 0
    b = {"route": T * E * 4 + bias + M * 8,
         "prefill_dispatch": M * 16 + T * P + M * P + M * 4 + N * (2 * L + 1) * 4,
         "combine_local": M * Pc + N * M * 12 + N * T * H * 4,
         "allreduce": N * T * H * 4 + T * Pc}
    b["dispatch"] = b["route"] + b["prefill_dispatch"]
    b["combine"] = b["combine_local"] + b["allreduce"]
    b["total"] = b["dispatch"] + b["combine"]
    return b


def run_prefill_workload(name, steps, warmup, check=True, flush_mall=True):
    """The replicated-token path: route -> prefill dispatch | (stand-in expert, outside the
    metric) | local combine -> all-reduce, per call timed with HIP events on the kernels' stream,
    medians over the steps, timed with the memory-side cache flushed between steps and back to
    back as the decode workloads are.  The dispatch's cached stores leave part of their write-back
    to the stand-in, so the layer is also reported with the stand-in counted."""
    import numpy as np
    import torch

    import combine_moe_route_top_amd as moe
    import moe_synth as ms

    c = ms.CONFIGS[name]
    inp = ms.make_inputs(1, c.T, c.H, c.E, c.R, c.fp8, c.bias, c.seed)
    b = moe.alloc_prefill_buffers(c.N, c.T, c.H, c.E, c.R, c.fp8)
    b.logits.copy_(torch.from_numpy(inp["logits"]))
    use_bias = inp["bias"] is not None
    if use_bias:
        b.bias.copy_(torch.from_numpy(inp["bias"]))
    x = inp["x"].reshape(c.T, c.H)
    b.x.copy_(torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x))
    if c.fp8:
        b.x_scale.copy_(torch.from_numpy(inp["x_scale"].reshape(c.T, -1)))
    st = torch.cuda.current_stream()
    sh = b.shape
    names = ["route", "prefill_dispatch", "stub", "combine_local", "allreduce"]
    calls = [
        lambda: moe.moe_route(sh, b.logits, b.bias if use_bias else None, b.topk_idx, b.topk_w, st),
        lambda: moe.moe_prefill_dispatch(sh, b.x, b.x_scale, b.topk_idx, b.slot_pos, b.expert_x,
                                         b.expert_scale, b.expert_cnt, b.expert_off, b.expert_src,
                                         b.workspace, st),
        lambda: moe.moe_expert_stub(sh, 0, b.expert_x, b.expert_scale, b.expert_off, b.expert_y, st),
        lambda: moe.moe_prefill_combine_local(sh, b.expert_y, b.topk_idx, b.slot_pos, b.topk_w,
                                              b.partial, st),
        lambda: moe.moe_prefill_allreduce(sh, b.partial, b.out, st),
    ]
    for _ in range(warmup):
        for f in calls:
            f()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
    ab = prefill_alg_bytes(c)

    def timed(flush):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
        for k in range(steps):
            if flush:
                scratch.sum()
            for i, f in enumerate(calls):
                evs[k][i].record(st)
                f()
            evs[k][len(calls)].record(st)
        torch.cuda.synchronize()
        per = {n: round(float(np.median([evs[k][i].elapsed_time(evs[k][i + 1]) * 1e3 for k in range(steps)])), 2)
               for i, n in enumerate(names)}
        dispatch_us = per["route"] + per["prefill_dispatch"]
        combine_us = per["combine_local"] + per["allreduce"]
        layer_us = dispatch_us + combine_us
        return dict(layer_us=round(layer_us, 2), layer_with_stub_us=round(layer_us + per["stub"], 2),
                    dispatch_us=round(dispatch_us, 2), combine_us=round(combine_us, 2), per_call_us=per,
                    gbs=round(ab["total"] / (layer_us * 1e-6) / 1e9, 1),
                    per_call_gbs={n: round(ab[n] / (per[n] * 1e-6) / 1e9, 1)
                                  for n in ["route", "prefill_dispatch", "combine_local", "allreduce"]})

    head = timed(flush_mall)
    other = timed(not flush_mall)
    del scratch
    res = dict(workload=name, dtype=c.dtype, mall_flushed_between_steps=bool(flush_mall), **head,
               alg_bytes=ab["total"])
    res["other_protocol"] = {"mall_flushed_between_steps": not flush_mall,
                             **{k: other[k] for k in ("layer_us", "layer_with_stub_us", "per_call_us", "gbs")}}
    if check:
        # identity experts: out == bf16(x * sum_k w_k) up to the torch reference's own double
        # rounding; every slot lands on exactly one rank
        sw = b.topk_w.double().sum(1, keepdim=True)
        if c.fp8:
            xv = (b.x.view(torch.float8_e4m3fn).double() *
                  b.x_scale.double().repeat_interleave(128, dim=1)).to(torch.bfloat16).double()
        else:
            xv = b.x.view(torch.bfloat16).double()
        want = (xv * sw).to(torch.float32).to(torch.bfloat16).view(torch.int16).int()
        got = b.out.int()
        key = lambda u: torch.where(u < 0, -(u & 0x7FFF), u & 0x7FFF)  # noqa: E731
        ulp = (key(want) - key(got)).abs().max().item()
        cnt_ok = int(b.expert_cnt.sum().item()) == c.T * c.R
        if ulp > 2 or not cnt_ok:
            raise RuntimeError(f"prefill closed-form check failed: {ulp} ulp, counts ok {cnt_ok}")
        res["check"] = f"ok (max {ulp} bf16 ulp vs identity closed form; every slot on one rank)"
    if int(b.status.item()) != 0:
        raise RuntimeError(f"device status word {int(b.status.item())}")
    del b
    torch.cuda.empty_cache()
    return res


def run_workload(name, steps, warmup, check=True, flush_mall=True):
    """One decode-layout workload: per-call HIP-event times (median and mean over the steps),
    graph replay time, and the closed-form check.  The steps are timed twice: with the 256 MB
    memory-side cache flushed between steps (a 1 GiB scratch buffer read outside every timed
    call, so the cache holds none of the previous step's data; a read, not a write, since written
    lines would stay dirty and be written back during the next step's first calls) and back to
    back.  flush_mall picks which of the two is the headline; the other is reported beside it."""
    import numpy as np
    import torch

    import combine_moe_route_top_amd as moe
    import moe_synth as ms

    c = ms.CONFIGS[name]
    inp = ms.config_inputs(c)
    tok = ms.config_tokens(c)
    b = moe.alloc_buffers(c.N, c.T, c.H, c.E, c.R, c.fp8, quant=c.quant, tokens=tok is not None)
    if tok is not None:
        b.tokens.copy_(torch.from_numpy(tok))
    b.logits.copy_(torch.from_numpy(inp["logits"]))
    use_bias = inp["bias"] is not None
    if use_bias:
        b.bias.copy_(torch.from_numpy(inp["bias"]))
    x = inp["x"]
    b.x.copy_(torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x))
    if c.fp8:
        b.x_scale.copy_(torch.from_numpy(inp["x_scale"]))
    stream = torch.cuda.current_stream()
    sh = b.shape
    y = b.expert_y if c.rows_fp8 else b.expert_x   # identity expert: bf16 combine reads expert_x

    names = ["route", "dispatch_send", "net_dispatch", "dispatch_recv", "stub", "combine"]

    def step(ev=None, st=None):
        st = stream if st is None else st

        def rec(i):
            if ev is not None:
                ev[i].record(st)
        rec(0)
        moe.moe_route(sh, b.logits, b.bias if use_bias else None, b.topk_idx, b.topk_w, st)
        rec(1)
        moe.moe_dispatch_send(sh, b.x, b.x_scale, b.topk_idx, b.counts, b.send_off, b.send_pos,
                              b.send_buf, b.send_meta, b.workspace, st)
        rec(2)
        moe.moe_net_dispatch(sh, b.send_off, b.send_buf, b.send_meta, b.recv_buf, b.recv_meta,
                             b.recv_off, st)
        rec(3)
        moe.moe_dispatch_recv(sh, b.counts, b.recv_off, b.recv_buf, b.recv_meta, b.expert_x,
                              b.expert_scale, b.expert_cnt, b.expert_off, b.expert_src,
                              b.expert_rpos, st)
        rec(4)
        if c.rows_fp8:
            moe.moe_expert_stub(sh, 0, b.expert_x, b.expert_scale, b.expert_off, b.expert_y, st)
        rec(5)
        moe.moe_combine(sh, y, b.expert_rpos, b.recv_off, b.send_off, b.send_pos, b.topk_w,
                        b.cs_buf, b.cr_buf, b.out, st)
        rec(6)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
    ab = alg_bytes(c)

    def timed(flush):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            if flush:
                scratch.sum()
            step(evs[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        samples = {n: [evs[k][i].elapsed_time(evs[k][i + 1]) * 1e3 for k in range(steps)]   # us
                   for i, n in enumerate(names)}
        med = {n: float(np.median(v)) for n, v in samples.items()}
        mean = {n: float(np.mean(v)) for n, v in samples.items()}
        layer = sum(v for n, v in med.items() if n != "stub")
        return dict(per_call_us={n: round(v, 2) for n, v in med.items()},
                    per_call_mean_us={n: round(v, 2) for n, v in mean.items()},
                    layer_us=layer, layer_mean_us=sum(v for n, v in mean.items() if n != "stub"),
                    dispatch_us=med["route"] + med["dispatch_send"] + med["net_dispatch"] + med["dispatch_recv"],
                    combine_us=med["combine"], wall_ms_per_step=wall * 1e3 / steps,
                    gbs=ab["total"] / (layer * 1e-6) / 1e9,
                    per_call_gbs={n: round(ab[n] / (med[n] * 1e-6) / 1e9, 1)
                                  for n in ["route", "dispatch_send", "net_dispatch", "dispatch_recv", "combine"]})

    head = timed(flush_mall)
    other = timed(not flush_mall)
    del scratch
    res = dict(workload=name, desc=c.desc, dtype=c.dtype, N=c.N, T=c.T, H=c.H, E=c.E, R=c.R,
               alg_bytes=ab, mall_flushed_between_steps=bool(flush_mall), **head)
    res["other_protocol"] = {"mall_flushed_between_steps": not flush_mall,
                             **{k: (round(v, 2) if isinstance(v, float) else v) for k, v in other.items()
                                if k in ("layer_us", "layer_mean_us", "per_call_us", "gbs", "wall_ms_per_step")}}
    if exchange_fits_mall(c):
        # the unpack reads the exchanged rows from the memory-side cache, where the network kernel
        # left them: those bytes are not HBM traffic
        hbm = ab["total"] - ab["mall_resident"]
        res["hbm_only"] = {"bytes": hbm, "excluded_bytes": ab["mall_resident"],
                           "excluded": "the unpack's read of the exchanged rows (served by the 256 MB "
                                       "memory-side cache)",
                           "gbs": round(hbm / (res["layer_us"] * 1e-6) / 1e9, 1),
                           "frac_of_peak": round(hbm / (res["layer_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    # the same step captured once in a HIP graph and replayed (no host work per step)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    step(st=side)                      # warm-up on a side stream, as graph capture expects
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(st=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    res["graph_replay_us_per_step"] = round(g0.elapsed_time(g1) * 1e3 / steps, 2)
    if check:
        res["check"] = closed_form_check(b, c)
    status = int(b.status.item())
    if status != 0:
        raise RuntimeError(f"device status word {status} ({moe.moe_strerror(status)})")
    del b
    torch.cuda.empty_cache()
    return res


def closed_form_check(b, c) -> str:
    """Identity experts: out == bf16(y * sum_k w_k) up to 1 bf16 ulp for every token (y the
    dispatched value), and each rank's counts sum to T_s*R.  A property check at full size; the
    element-wise oracle comparison lives in the GPU parity tests.  Tokens quantised by the send
    pack: out is within e4m3 rounding of x * sum_k w_k instead."""
    import torch

    import moe_synth as ms
    tok = ms.config_tokens(c)
    nt = torch.full((c.N,), c.T, dtype=torch.int64) if tok is None else torch.from_numpy(tok).long()
    present = (torch.arange(c.T)[None, :] < nt[:, None]).to(b.out.device)     # [N][T]
    counts_ok = bool((b.counts.sum(1).cpu() == nt * c.R).all().item())
    if c.quant:
        # |e4m3(v) - v| <= 2^-4 |v| (3 mantissa bits) above 2^-6, <= 2^-10 below, in units of
        # the block scale; then one bf16 rounding of the weighted sum (2^-8 relative)
        xv = b.x.view(torch.bfloat16).float()
        sc = xv.abs().view(c.N, c.T, c.H // 128, 128).amax(-1) / 448.0
        sc = sc.repeat_interleave(128, dim=2)
        sw = b.topk_w.float().sum(1).view(c.N, c.T, 1)
        got = b.out.view(torch.bfloat16).float()
        err = (got - xv * sw).abs()
        bound = (xv.abs() * (2.0 ** -4) + sc * (2.0 ** -10)) * sw * 1.01 + got.abs() * 2.0 ** -8
        bad = int(((err > bound) & present[..., None]).sum().item())
        if bad or not counts_ok:
            raise RuntimeError(f"closed-form check failed: {bad} values outside the e4m3 bound, "
                               f"counts ok {counts_ok}")
        return "ok (every value within e4m3 + bf16 rounding of x * sum w; counts sum to T_s*R)"
    sw = b.topk_w.double().sum(1).view(c.N, c.T, 1)
    if c.fp8:
        xv = b.x.view(torch.float8_e4m3fn).double() * b.x_scale.double().repeat_interleave(128, dim=2)
    else:
        xv = b.x.view(torch.bfloat16).double()
    want = (xv * sw).to(torch.float32).to(torch.bfloat16) if not c.fp8 else \
        (xv.to(torch.bfloat16).double() * sw).to(torch.float32).to(torch.bfloat16)
    got = b.out.view(torch.bfloat16)
    a = want.view(torch.int16).int()
    g = got.view(torch.int16).int()
    key = lambda u: torch.where(u < 0, -(u & 0x7FFF), u & 0x7FFF)  # noqa: E731
    ulp = ((key(a) - key(g)).abs() * present[..., None]).max().item()
    if ulp > 2 or not counts_ok:  # the torch reference itself rounds twice (fp64->fp32->bf16)
        raise RuntimeError(f"closed-form check failed: max {ulp} bf16 ulp, counts ok {counts_ok}")
    return f"ok (max {ulp} bf16 ulp vs identity closed form; counts sum to T_s*R)"


def kernel_text(src: str, name: str):
    """The definition of kernel (or device function) `name` in a source text: from its
    template/__global__/__device__ line to the brace that closes its body, or None."""
    import re
    m = re.search(r"^(template <[^\n]*>\n)?(__global__|__device__)[^\n]*\b" + re.escape(name) + r"\(",
                  src, re.M)
    if not m:
        return None
    i = src.index("{", m.end())
    depth = 0
    for j in range(i, len(src)):
        depth += {"{": 1, "}": -1}.get(src[j], 0)
        if depth == 0:
            return src[m.start():j + 1]
    return None


def source_digest(spec: str):
    """sha256 over the sources a kernel is built from: comma-separated files, where
    `file#kernel` stands for that kernel's own definition in the file."""
    import hashlib
    h = hashlib.sha256()
    for item in spec.split(","):
        rel, _, kern = item.partition("#")
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path):
            return None
        text = open(path).read()
        if kern:
            text = kernel_text(text, kern)
            if text is None:
                return None
        h.update(text.encode())
    return h.hexdigest()


def traffic_record(kernel, workload):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch from the committed counter summary, or
    None if there is none or the kernel's source changed since the counters were taken."""
    import glob
    import re
    for path in glob.glob(os.path.join(ROOT, "profiles", "counters_*.md")):
        for line in open(path):
            m = re.match(r"traffic-record: kernel=(\S+) workload=(\S+) bytes_per_launch=(\d+) "
                         r"source=(\S+) sha256=([0-9a-f]+)", line.strip())
            if not m or m.group(1) != kernel or m.group(2) != workload:
                continue
            digest = source_digest(m.group(4))
            if digest is None or digest != m.group(5):
                return None
            return int(m.group(3))
    return None


def dominant_kernel(res, calib=None) -> dict:
    """Roofline of the dominant kernel: the network stand-in, k_net_dispatch, the one kernel of
    moe_net_dispatch (its first blocks also write the recv_off table).  Beside the fraction of the
    8 TB/s peak, the fraction of the measured copy ceiling when the bench took it."""
    ab = res["alg_bytes"]
    us = res["per_call_us"]["net_dispatch"]
    achieved = ab["net_dispatch"] / (us * 1e-6) / 1e9
    out = {"kernel": "k_net_dispatch (the whole of moe_net_dispatch)", "bound": "hbm",
           "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": round(achieved / PEAK_HBM_GBS, 4),
           "traffic": traffic_record("k_net_dispatch", res["workload"]),
           "bytes_per_launch": ab["net_dispatch"], "us_per_launch": round(us, 2)}
    if calib is not None:
        out["frac_of_copy_ceiling"] = round(achieved / calib["stream_copy"]["gbs"], 4)
    return out


def cpu_baseline(name, budget_s=20.0) -> dict:
    """The oracle, as it stands, on one full layer of the workload on the host cores: the
    single-threaded calls (the baseline), and beside it the same oracle functions with each step's
    ranks split into one chunk per available core, run on that many threads (each chunk is one C
    call of the oracle's rank-range form; the steps run one after another)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import moe_synth as ms
    import oracle
    c = ms.CONFIGS[name]
    inp = ms.config_inputs(c)
    tok = ms.config_tokens(c)
    ab = alg_bytes(c)

    def layer_single():
        x, xs = inp["x"], inp["x_scale"]
        if c.quant:
            x, xs = oracle.quantize_e4m3(x)
        ts = [time.perf_counter()]
        sh = oracle.shape(c.N, c.T, c.H, c.E, c.R, c.rows_fp8, tokens=tok)
        idx, w = oracle.route(inp["logits"], inp["bias"], c.R)
        ts.append(time.perf_counter())
        r = oracle.dispatch_send(sh, x, xs, idx.reshape(c.N, -1))
        ts.append(time.perf_counter())
        sh = oracle.packed_shape(c.N, c.T, c.H, c.E, c.R, c.rows_fp8,
                                 np.diff(r["send_off"], axis=1).sum(axis=0), tok)
        r.update(oracle.net_dispatch(sh, r["send_off"], r["send_buf"], r["send_meta"]))
        ts.append(time.perf_counter())
        r.update(oracle.dispatch_recv(sh, r["counts"], r["recv_off"], r["recv_buf"], r["recv_meta"]))
        ts.append(time.perf_counter())
        y = oracle.expert(sh, 0, r["expert_x"], r["expert_scale"], r["expert_off"])
        t2 = time.perf_counter()
        out = oracle.combine(sh, 0, y, r["expert_rpos"], r["recv_off"], r["send_off"], r["send_pos"], w)
        t3 = time.perf_counter()
        stages = [b - a for a, b in zip(ts, ts[1:])] + [t3 - t2]
        return sum(stages), stages, y, out["out"]

    def layer_threaded(pool, parts, y):
        x, xs = inp["x"], inp["x_scale"]
        if c.quant:
            x, xs = oracle.quantize_e4m3(x)
        t0 = time.perf_counter()
        sh = oracle.shape(c.N, c.T, c.H, c.E, c.R, c.rows_fp8, tokens=tok)
        idx, w = oracle.route_chunked(inp["logits"], inp["bias"], c.R, pool, parts)
        r = oracle.dispatch_send_chunked(sh, x, xs, idx.reshape(c.N, -1), pool, parts)
        sh = oracle.packed_shape(c.N, c.T, c.H, c.E, c.R, c.rows_fp8,
                                 np.diff(r["send_off"], axis=1).sum(axis=0), tok)
        r.update(oracle.net_dispatch_chunked(sh, r["send_off"], r["send_buf"], r["send_meta"], pool, parts))
        r.update(oracle.dispatch_recv_chunked(sh, r["counts"], r["recv_off"], r["recv_buf"], r["recv_meta"],
                                              pool, parts))
        # (the stand-in expert's output y is the single run's; it is not part of the timing)
        out = oracle.combine_chunked(sh, 0, y, r["expert_rpos"], r["recv_off"], r["send_off"], r["send_pos"],
                                     w, pool, parts)
        return time.perf_counter() - t0, out["out"]

    times, stage_times, t_start = [], [], time.perf_counter()
    y = out1 = None
    while True:
        t, st_, y, out1 = layer_single()
        times.append(t)
        stage_times.append(st_)
        # about budget_s/2 .. budget_s of host work: at least 3 layers, at most 20
        if len(times) >= 20 or (len(times) >= 3 and time.perf_counter() - t_start > budget_s * 0.5):
            break
    t1core = float(np.median(times))
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    ttimes, outn = [], None
    with ThreadPoolExecutor(max_workers=cores) as pool:
        t_start = time.perf_counter()
        while True:
            t, outn = layer_threaded(pool, cores, y)
            ttimes.append(t)
            if len(ttimes) >= 20 or (len(ttimes) >= 3 and time.perf_counter() - t_start > budget_s * 0.25):
                break
    if not np.array_equal(outn, out1):
        raise RuntimeError("threaded oracle output differs from the single-threaded oracle")
    tn = float(np.median(ttimes))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(ab["total"] / t1core / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_share": cores, "cpu_model": model,
            "us_per_layer": round(t1core * 1e6, 1),
            "per_stage_us": {n: round(float(np.median([st_[i] for st_ in stage_times])) * 1e6, 1)
                             for i, n in enumerate(["route", "dispatch_send", "net_dispatch", "dispatch_recv",
                                                    "combine"])},
            "sample": f"one full {name} layer (all {c.N} ranks) through the single-threaded C oracle "
                      f"(route, dispatch, network, unpack, combine; stand-in expert excluded), "
                      f"median of {len(times)}",
            "threaded": {"value": round(ab["total"] / tn / 1e9, 3), "unit": "GB/s", "cores": cores,
                         "us_per_layer": round(tn * 1e6, 1), "speedup": round(t1core / tn, 2),
                         "sample": f"the same layer with each step's ranks split into {cores} chunks on "
                                   f"{cores} threads, median of {len(ttimes)}; output equal to the "
                                   f"single-threaded run"}}


def copy_calibration(nbytes=1 << 30, reps=10) -> dict:
    """Copies of known size timed with HIP events: moe_stream_copy (the library's row-streaming
    engine on a contiguous row map: the practical ceiling the row-copy kernels are measured
    against) and torch's copy_, each 1 GiB read + 1 GiB written, median of `reps`."""
    import numpy as np
    import torch

    import combine_moe_route_top_amd as moe
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    out = {"bytes_read": nbytes, "bytes_written": nbytes}
    for name, fn in (("stream_copy", lambda: moe.moe_stream_copy(src, dst, nbytes)),
                     ("torch_copy", lambda: dst.copy_(src))):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e3)
        us = float(np.median(t))
        out[name] = {"us": round(us, 2), "gbs": round(2 * nbytes / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(2 * nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    del src, dst
    torch.cuda.empty_cache()
    return out


def cu_masked_stream(n_cus: int):
    """A HIP stream (default priority) whose kernels run only on the first n_cus compute units
    (hipExtStreamCreateWithCUMask), wrapped for torch; returns (handle, torch stream)."""
    import ctypes

    import torch
    hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch has loaded (same SONAME)
    total = torch.cuda.get_device_properties(0).multi_processor_count
    words = (total + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for i in range(min(n_cus, total)):
        mask[i // 32] |= 1 << (i % 32)
    handle = ctypes.c_void_p()
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                ctypes.POINTER(ctypes.c_uint32)]
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), words, mask)
    if rc != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed: {rc}")
    return handle.value, torch.cuda.ExternalStream(handle.value)


def destroy_stream(handle):
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    hip.hipStreamDestroy(handle)


def overlap_leg(name, steps=10, warmup=2, inter=2048, cu_splits=(256, 224, 192, 160, 128)) -> dict:
    """Send/receive split in use: a stand-in shared expert (one MLP, hidden H -> inter -> H, bf16
    GEMMs through torch) runs on a second stream while (a) the dispatch transfer (network
    stand-in + receive) and (b) the combine send half run on the first.  Reports serial and
    overlapped time and the part of the shared expert hidden behind the transfer.  On one GPU the
    copy stand-ins are themselves CU kernels that fill the chip, so the transfer's stream is
    restricted to a subset of the compute units (a CU-masked stream, swept over cu_splits of the
    GPU's units; 'all' is the unmasked stream), standing in for a transfer that leaves CUs free;
    the shared expert's stream is never masked.  Serial references run on the same masked stream."""
    import numpy as np
    import torch
    import torch.nn.functional as F

    import combine_moe_route_top_amd as moe
    import moe_synth as ms

    c = ms.CONFIGS[name]
    assert not c.fp8, "the overlap leg runs on a bf16 workload"
    inp = ms.config_inputs(c)
    b = moe.alloc_buffers(c.N, c.T, c.H, c.E, c.R, c.fp8)
    b.logits.copy_(torch.from_numpy(inp["logits"]))
    use_bias = inp["bias"] is not None
    if use_bias:
        b.bias.copy_(torch.from_numpy(inp["bias"]))
    b.x.copy_(torch.from_numpy(inp["x"].view(np.int16)))
    gen = torch.Generator(device="cuda").manual_seed(0)
    wg = (torch.randn(c.H, inter, device="cuda", generator=gen) * c.H ** -0.5).to(torch.bfloat16)
    wu = (torch.randn(c.H, inter, device="cuda", generator=gen) * c.H ** -0.5).to(torch.bfloat16)
    wd = (torch.randn(inter, c.H, device="cuda", generator=gen) * inter ** -0.5).to(torch.bfloat16)
    xs = b.x.view(torch.bfloat16).view(c.N * c.T, c.H)
    ys = torch.empty_like(xs)
    s2 = torch.cuda.Stream()   # default priority, all compute units
    sh = b.shape
    total_cus = torch.cuda.get_device_properties(0).multi_processor_count

    def shared(st):
        with torch.cuda.stream(st):
            torch.matmul(F.silu(xs @ wg) * (xs @ wu), wd, out=ys)

    def measure(s1):
        def d_send():
            moe.moe_route(sh, b.logits, b.bias if use_bias else None, b.topk_idx, b.topk_w, s1)
            moe.moe_dispatch_send(sh, b.x, b.x_scale, b.topk_idx, b.counts, b.send_off, b.send_pos,
                                  b.send_buf, b.send_meta, b.workspace, s1)

        def d_transfer():
            moe.moe_net_dispatch(sh, b.send_off, b.send_buf, b.send_meta, b.recv_buf, b.recv_meta,
                                 b.recv_off, s1)
            moe.moe_dispatch_recv(sh, b.counts, b.recv_off, b.recv_buf, b.recv_meta, b.expert_x,
                                  b.expert_scale, b.expert_cnt, b.expert_off, b.expert_src,
                                  b.expert_rpos, s1)

        def c_send():
            moe.moe_combine_send(sh, b.expert_x, b.expert_rpos, b.recv_off, b.send_off, b.cs_buf,
                                 b.cr_buf, s1)

        def c_recv():
            moe.moe_combine_recv(sh, b.cr_buf, b.send_pos, b.topk_w, b.out, s1)

        def fork_join(first, second):
            """first() on s1, then the shared expert on s2 concurrently with second() on s1."""
            first()
            ev = torch.cuda.Event()
            ev.record(s1)
            s2.wait_event(ev)
            shared(s2)
            second()
            s1.wait_stream(s2)

        def serial(*fns):
            for fn in fns:
                fn()
            shared(s1)

        # dispatch: the shared expert runs while the transfer (network + receive) is in flight;
        # combine: while the combine send half (shuffle + network back) is, before the weighted sum
        variants = {
            "shared_alone": lambda: shared(s1),
            "dispatch_alone": lambda: (d_send(), d_transfer()),
            "dispatch_then_shared": lambda: serial(d_send, d_transfer),
            "dispatch_overlap": lambda: fork_join(d_send, d_transfer),
            "combine_alone": lambda: (c_send(), c_recv()),
            "combine_then_shared": lambda: (c_send(), shared(s1), c_recv()),
            "combine_overlap": lambda: (fork_join(lambda: None, c_send), c_recv()),
        }
        us = {}
        for k, fn in variants.items():
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s1)
            for _ in range(steps):
                fn()
            e1.record(s1)
            torch.cuda.synchronize()
            us[k] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
        out = {"us": us}
        for ph in ("dispatch", "combine"):
            hidden = us[f"{ph}_then_shared"] - us[f"{ph}_overlap"]
            out[f"{ph}_hidden_us"] = round(hidden, 2)
            out[f"{ph}_hidden_frac_of_shared"] = round(hidden / us["shared_alone"], 3)
        return out

    res = {"workload": name, "shared_expert": f"bf16 MLP {c.H}->{inter}->{c.H} on {c.N * c.T} tokens "
                                               f"(torch GEMMs on a second stream)",
           "total_cus": total_cus}
    torch.cuda.synchronize()
    res.update(measure(torch.cuda.current_stream()))
    sweep = {}
    for n in cu_splits:
        if n >= total_cus:
            continue
        handle, sm = cu_masked_stream(n)
        try:
            r = measure(sm)
        finally:
            torch.cuda.synchronize()
            destroy_stream(handle)
        base = res["us"]
        r["dispatch_overlap_vs_unmasked_serial_us"] = round(base["dispatch_then_shared"] - r["us"]["dispatch_overlap"], 2)
        r["combine_overlap_vs_unmasked_serial_us"] = round(base["combine_then_shared"] - r["us"]["combine_overlap"], 2)
        sweep[f"{n}_cus"] = r
    res["cu_masked_transfer"] = sweep
    if sweep:
        # the split that saves the most against everything run serially on all compute units
        best = max(sweep.items(), key=lambda kv: kv[1]["dispatch_overlap_vs_unmasked_serial_us"] +
                   kv[1]["combine_overlap_vs_unmasked_serial_us"])
        res["best_cu_split"] = {"transfer_cus": int(best[0].split("_")[0]),
                                "dispatch_saved_us": best[1]["dispatch_overlap_vs_unmasked_serial_us"],
                                "combine_saved_us": best[1]["combine_overlap_vs_unmasked_serial_us"],
                                "transfer_alone_us": best[1]["us"]["dispatch_alone"],
                                "transfer_alone_unmasked_us": res["us"]["dispatch_alone"]}
    if int(b.status.item()) != 0:
        raise RuntimeError("device status word set in the overlap leg")
    del b
    torch.cuda.empty_cache()
    return res


def microbatch_leg(name, steps=10, warmup=2, inter=2048) -> dict:
    """Two-micro-batch pipelining ([DSK] computation/communication overlap): the layer's tokens
    are split into two micro-batches of T/2 tokens per rank, each with its own buffers.  A
    stand-in compute stage (the shared-expert MLP of the overlap leg on the micro-batch's tokens)
    runs on a second stream.  Serial: dispatch A, compute A, combine A, then the same for B.
    Pipelined: dispatch A; compute A on stream 2 while dispatch B runs on stream 1; combine A
    (after compute A) on stream 1 while compute B (after dispatch B) runs on stream 2; combine B.
    Reports both times and the time hidden."""
    import numpy as np
    import torch
    import torch.nn.functional as F

    import combine_moe_route_top_amd as moe
    import moe_synth as ms

    c = ms.CONFIGS[name]
    assert not c.rows_fp8 and c.T % 2 == 0, "the micro-batch leg runs on a bf16 workload, T even"
    Th = c.T // 2
    inp = ms.config_inputs(c)
    # two streams taken from torch's pool one after the other (default priority): consecutive pool
    # streams sit on different hardware queues, whereas a stream taken late in a run can share a
    # queue with the one the path runs on and serialise behind it
    s1 = torch.cuda.Stream()
    s2 = torch.cuda.Stream()
    gen = torch.Generator(device="cuda").manual_seed(0)
    wg = (torch.randn(c.H, inter, device="cuda", generator=gen) * c.H ** -0.5).to(torch.bfloat16)
    wu = (torch.randn(c.H, inter, device="cuda", generator=gen) * c.H ** -0.5).to(torch.bfloat16)
    wd = (torch.randn(inter, c.H, device="cuda", generator=gen) * inter ** -0.5).to(torch.bfloat16)
    logits = inp["logits"].reshape(c.N, c.T, c.E)
    x = inp["x"].view(np.int16)
    use_bias = inp["bias"] is not None
    mbs = []
    for h in range(2):
        b = moe.alloc_buffers(c.N, Th, c.H, c.E, c.R)
        b.logits.copy_(torch.from_numpy(np.ascontiguousarray(logits[:, h * Th:(h + 1) * Th]).reshape(-1, c.E)))
        if use_bias:
            b.bias.copy_(torch.from_numpy(inp["bias"]))
        b.x.copy_(torch.from_numpy(np.ascontiguousarray(x[:, h * Th:(h + 1) * Th])))
        xs = b.x.view(torch.bfloat16).view(c.N * Th, c.H)
        mbs.append((b, xs, torch.empty_like(xs)))
    torch.cuda.synchronize()   # the uploads ran on the current stream, which s1 and s2 do not wait for

    def dispatch(mb, st):
        b = mb[0]
        moe.moe_route(b.shape, b.logits, b.bias if use_bias else None, b.topk_idx, b.topk_w, st)
        moe.moe_dispatch_send(b.shape, b.x, None, b.topk_idx, b.counts, b.send_off, b.send_pos,
                              b.send_buf, b.send_meta, b.workspace, st)
        moe.moe_net_dispatch(b.shape, b.send_off, b.send_buf, b.send_meta, b.recv_buf, b.recv_meta,
                             b.recv_off, st)
        moe.moe_dispatch_recv(b.shape, b.counts, b.recv_off, b.recv_buf, b.recv_meta, b.expert_x,
                              None, b.expert_cnt, b.expert_off, b.expert_src, b.expert_rpos,
                              st)

    def compute(mb, st):
        _, xs, ys = mb
        with torch.cuda.stream(st):
            torch.matmul(F.silu(xs @ wg) * (xs @ wu), wd, out=ys)

    def combine(mb, st):
        b = mb[0]
        moe.moe_combine(b.shape, b.expert_x, b.expert_rpos, b.recv_off, b.send_off, b.send_pos,
                        b.topk_w, b.cs_buf, b.cr_buf, b.out, st)

    def after(st_wait, st_done):
        ev = torch.cuda.Event()
        ev.record(st_done)
        st_wait.wait_event(ev)

    A, Bm = mbs

    def serial():
        for mb in (A, Bm):
            dispatch(mb, s1)
            compute(mb, s1)
            combine(mb, s1)

    def pipelined():
        dispatch(A, s1)
        after(s2, s1)
        compute(A, s2)         # compute A  ||  dispatch B
        dispatch(Bm, s1)
        after(s1, s2)          # combine A needs compute A
        after(s2, s1)          # compute B needs dispatch B
        combine(A, s1)
        compute(Bm, s2)        # compute B  ||  combine A
        after(s1, s2)
        combine(Bm, s1)

    us = {}
    for k, fn in (("serial", serial), ("pipelined", pipelined)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s1)
        for _ in range(steps):
            fn()
        e1.record(s1)
        torch.cuda.synchronize()
        us[k] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
    # the parts alone, for reference
    parts = {}
    for k, fn in (("dispatch", lambda: dispatch(A, s1)), ("compute", lambda: compute(A, s1)),
                  ("combine", lambda: combine(A, s1))):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s1)
        for _ in range(steps):
            fn()
        e1.record(s1)
        torch.cuda.synchronize()
        parts[k] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
    for mb in mbs:
        if int(mb[0].status.item()) != 0:
            raise RuntimeError("device status word set in the micro-batch leg")
    res = {"workload": name, "micro_batches": 2, "tokens_per_rank_each": Th,
           "compute": f"bf16 MLP {c.H}->{inter}->{c.H} on each micro-batch's {c.N * Th} tokens "
                      f"(torch GEMMs on a second stream)",
           "us": us, "one_micro_batch_us": parts,
           "hidden_us": round(us["serial"] - us["pipelined"], 2)}
    del mbs, A, Bm
    torch.cuda.empty_cache()
    return res


LAUNCH_REPS = 8
# kernels in one rank's decode layer: route; count and pack; network; unpack; combine pack and
# network back; weighted sum
KERNELS_PER_RANK_LAYER = 8


def graph_period(fn, reps) -> float:
    """Median µs per call of fn(stream) when LAUNCH_REPS calls are captured in one HIP graph and
    the graph is replayed (HIP events around each replay)."""
    import numpy as np
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(LAUNCH_REPS):
            fn(torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(LAUNCH_REPS):
            fn(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3 / LAUNCH_REPS)
    del g
    return round(float(np.median(t)), 2)


def rank_leg(name, steps=20, warmup=3) -> dict:
    """One rank's share at its real shape: every call restricted to a single rank (as each GPU of
    an expert-parallel deployment runs it), timed with HIP events, for the rank that receives the
    most rows and for the median rank (by rows received), and the rank's combine with the sum on
    the sending side in place of its combine.  The other ranks' data are in place from a full step
    first; the network time between GPUs is not part of this."""
    import numpy as np
    import torch

    import combine_moe_route_top_amd as moe
    import moe_synth as ms

    c = ms.CONFIGS[name]
    inp = ms.config_inputs(c)
    b = moe.alloc_buffers(c.N, c.T, c.H, c.E, c.R, c.fp8)
    b.logits.copy_(torch.from_numpy(inp["logits"]))
    use_bias = inp["bias"] is not None
    if use_bias:
        b.bias.copy_(torch.from_numpy(inp["bias"]))
    x = inp["x"]
    b.x.copy_(torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x))
    if c.fp8:
        b.x_scale.copy_(torch.from_numpy(inp["x_scale"]))
    st = torch.cuda.current_stream()
    moe.run_dispatch(b, bias=use_bias)
    moe.moe_expert_stub(b.shape, 0, b.expert_x, b.expert_scale, b.expert_off, b.expert_y)
    y = b.expert_y
    moe.run_combine(b, y)
    torch.cuda.synchronize()
    recv = b.recv_off[:, c.N].cpu().numpy()
    order = np.argsort(recv, kind="stable")
    picks = {"max_rank": int(order[-1]), "median_rank": int(order[len(order) // 2])}
    calls = ["route", "dispatch_send", "net_dispatch", "dispatch_recv", "combine_send", "combine_recv"]
    out = {"workload": name, "rows_received": {}}
    for label, r in picks.items():
        sh = moe.for_ranks(b.shape, r, 1)

        def calls_on(s_):
            return [
                lambda: moe.moe_route(sh, b.logits, b.bias if use_bias else None, b.topk_idx,
                                      b.topk_w, s_),
                lambda: moe.moe_dispatch_send(sh, b.x, b.x_scale, b.topk_idx, b.counts, b.send_off,
                                              b.send_pos, b.send_buf, b.send_meta, b.workspace, s_),
                lambda: moe.moe_net_dispatch(sh, b.send_off, b.send_buf, b.send_meta, b.recv_buf,
                                             b.recv_meta, b.recv_off, s_),
                lambda: moe.moe_dispatch_recv(sh, b.counts, b.recv_off, b.recv_buf, b.recv_meta,
                                              b.expert_x, b.expert_scale, b.expert_cnt, b.expert_off,
                                              b.expert_src, b.expert_rpos, s_),
                lambda: moe.moe_combine_send(sh, y, b.expert_rpos, b.recv_off, b.send_off, b.cs_buf,
                                             b.cr_buf, s_),
                lambda: moe.moe_combine_recv(sh, b.cr_buf, b.send_pos, b.topk_w, b.out, s_),
            ]
        fns = calls_on(st)
        for _ in range(warmup):
            for f in fns:
                f()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
        for k in range(steps):
            for i, f in enumerate(fns):
                evs[k][i].record(st)
                f()
            evs[k][len(fns)].record(st)
        torch.cuda.synchronize()
        per = {n: round(sum(evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)) * 1e3 / steps, 2)
               for i, n in enumerate(calls)}
        # the rank's layer captured once in a HIP graph and replayed: no host launch per call
        side = torch.cuda.Stream()
        side.wait_stream(st)
        for f in calls_on(side):
            f()
        st.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for f in calls_on(torch.cuda.current_stream()):
                f()
        torch.cuda.synchronize()
        for _ in range(warmup):
            graph.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(st)
        for _ in range(steps):
            graph.replay()
        g1.record(st)
        torch.cuda.synchronize()
        # the rank's combine with the sum on the sending side instead (its two halves)
        acc_fns = [lambda: moe.moe_combine_acc_send(sh, y, b.recv_meta, b.counts, b.recv_off, b.expert_off,
                                                    b.send_off, b.topk_w, b.cs_buf, b.cr_buf, st),
                   lambda: moe.moe_combine_acc_recv(sh, b.cr_buf, b.topk_idx, b.send_pos, b.out, st)]
        for _ in range(warmup):
            for f in acc_fns:
                f()
        torch.cuda.synchronize()
        aev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for k in range(steps):
            for i, f in enumerate(acc_fns):
                aev[k][i].record(st)
                f()
            aev[k][2].record(st)
        torch.cuda.synchronize()
        acc = {n: round(sum(aev[k][i].elapsed_time(aev[k][i + 1]) for k in range(steps)) * 1e3 / steps, 2)
               for i, n in enumerate(["combine_acc_send", "combine_acc_recv"])}
        out[label] = {"rank": r, "rows_received": int(recv[r]), "us_per_layer": round(sum(per.values()), 2),
                      "graph_replay_us_per_layer": round(g0.elapsed_time(g1) * 1e3 / steps, 2),
                      "per_call_us": per, "send_side_sum_combine_us": acc}
        if label == "median_rank":
            # each call alone: a graph of LAUNCH_REPS repeats of it (every call is idempotent once
            # the full step has run), replayed; beside it the same for a 16-byte stream copy, the
            # cost of one graph-launched kernel that does (almost) nothing
            fl_src = torch.zeros(16, dtype=torch.uint8, device="cuda")
            fl_dst = torch.zeros(16, dtype=torch.uint8, device="cuda")
            floor = graph_period(lambda s_: moe.moe_stream_copy(fl_src, fl_dst, 16, s_), steps)
            periods = {n: graph_period(lambda s_, i=i: calls_on(s_)[i](), steps) for i, n in enumerate(calls)}
            out[label]["graph_period_us"] = periods
            out[label]["launch_floor_us"] = floor
            out[label]["kernels_per_layer"] = KERNELS_PER_RANK_LAYER
            out[label]["launch_floor_us_per_layer"] = round(floor * KERNELS_PER_RANK_LAYER, 2)
        del graph
    status = int(b.status.item())
    if status != 0:
        raise RuntimeError(f"device status word {status}")
    del b
    torch.cuda.empty_cache()
    return out


def acc_combine_leg(name, steps=20, warmup=3) -> dict:
    """The combine with the sum taken on the sending side ([EFA] results: fewer bytes back, some
    accuracy lost) beside the receive-side combine, on one dispatched layer of the workload:
    per-call times (HIP events, means over the steps), rows sent back (one partial per token and
    owner rank vs one row per routed slot), algorithmic bytes, and the accuracy cost as the bf16
    ulp distance between the two outputs (identity experts)."""
    import numpy as np
    import torch

    import combine_moe_route_top_amd as moe
    import moe_synth as ms

    c = ms.CONFIGS[name]
    inp = ms.config_inputs(c)
    b = moe.alloc_buffers(c.N, c.T, c.H, c.E, c.R, c.fp8)
    b.logits.copy_(torch.from_numpy(inp["logits"]))
    use_bias = inp["bias"] is not None
    if use_bias:
        b.bias.copy_(torch.from_numpy(inp["bias"]))
    x = inp["x"]
    b.x.copy_(torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x))
    if c.fp8:
        b.x_scale.copy_(torch.from_numpy(inp["x_scale"]))
    st = torch.cuda.current_stream()
    moe.run_dispatch(b, bias=use_bias)
    if c.rows_fp8:
        moe.moe_expert_stub(b.shape, 0, b.expert_x, b.expert_scale, b.expert_off, b.expert_y)
    y = b.expert_y if c.rows_fp8 else b.expert_x   # identity expert: bf16 combine reads expert_x
    sh = b.shape
    calls = {
        "receive_side": [
            lambda: moe.moe_combine_send(sh, y, b.expert_rpos, b.recv_off, b.send_off, b.cs_buf, b.cr_buf),
            lambda: moe.moe_combine_recv(sh, b.cr_buf, b.send_pos, b.topk_w, b.out)],
        "send_side": [
            lambda: moe.moe_combine_acc_send(sh, y, b.recv_meta, b.counts, b.recv_off, b.expert_off,
                                             b.send_off, b.topk_w, b.cs_buf, b.cr_buf),
            lambda: moe.moe_combine_acc_recv(sh, b.cr_buf, b.topk_idx, b.send_pos, b.out)],
    }
    res = {}
    outs = {}
    for kind, fns in calls.items():
        for _ in range(warmup):
            for f in fns:
                f()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for k in range(steps):
            for i, f in enumerate(fns):
                evs[k][i].record(st)
                f()
            evs[k][2].record(st)
        torch.cuda.synchronize()
        send = sum(evs[k][0].elapsed_time(evs[k][1]) for k in range(steps)) * 1e3 / steps
        recv = sum(evs[k][1].elapsed_time(evs[k][2]) for k in range(steps)) * 1e3 / steps
        res[kind] = {"send_us": round(send, 2), "recv_us": round(recv, 2), "combine_us": round(send + recv, 2)}
        outs[kind] = b.out.clone()
    status = int(b.status.item())
    if status != 0:
        raise RuntimeError(f"device status word {status}")
    # rows back: one per routed slot, or one per (token, owner rank)
    idx = b.topk_idx.cpu().numpy().reshape(c.N * c.T, c.R)
    owners = np.sort(idx // c.L, axis=1)
    G = int(c.N * c.T + (owners[:, 1:] != owners[:, :-1]).sum())
    NT, M, Pc = c.N * c.T, c.N * c.T * c.R, 2 * c.H
    acc_bytes = (M * Pc + M * 12 + G * Pc) + (2 * G * Pc + M * 8) + (G * Pc + NT * Pc + M * 8)
    std_bytes = alg_bytes(c)["combine"]
    res["receive_side"]["alg_bytes"] = std_bytes
    res["send_side"]["alg_bytes"] = acc_bytes
    for kind in res:
        res[kind]["gbs"] = round(res[kind]["alg_bytes"] / (res[kind]["combine_us"] * 1e3), 1)

    def key(t):
        u = t.view(torch.int16).to(torch.int32) & 0xFFFF
        return torch.where(u >= 0x8000, -(u & 0x7FFF), u)
    dist = (key(outs["send_side"]) - key(outs["receive_side"])).abs()
    out = {"workload": name, "rows_sent_back": {"receive_side": M, "send_side": G},
           "us": res, "speedup": round(res["receive_side"]["combine_us"] / res["send_side"]["combine_us"], 3),
           "accuracy_vs_receive_side": {"max_bf16_ulp": int(dist.max().item()),
                                        "frac_equal": round(float((dist == 0).float().mean().item()), 4)},
           "experts": "identity"}
    del b, outs
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--extra", default=",".join(EXTRA),
                    help="comma-separated workloads reported beside the headline ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-copy-calibration", action="store_true")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the send/receive-split overlap leg")
    ap.add_argument("--no-rank-leg", action="store_true",
                    help="skip the one-rank-share timing leg")
    ap.add_argument("--no-microbatch", action="store_true",
                    help="skip the two-micro-batch pipelining leg")
    ap.add_argument("--no-acc-combine", action="store_true",
                    help="skip the leg timing the combine with the sum on the sending side")
    ap.add_argument("--no-flush-mall", action="store_true",
                    help="headline from steps run back to back instead of with the memory-side "
                         "cache flushed between steps (a 1 GiB scratch read, untimed by the per-call "
                         "events, included in ms_per_step); both are measured and reported")
    ap.add_argument("--tokens-sweep", default="",
                    help="comma-separated tokens per rank: also time the headline workload's shape "
                         "at each (cache flushed between steps), reported as tokens_sweep")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the N expert-parallel ranks are simulated inside one "
              "GPU's HBM (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import moe_synth as ms
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if ms.CONFIGS[args.workload].layout != "decode":
        print("the headline workload must use the decode layout (prefill workloads run as extras)",
              file=sys.stderr)
        sys.exit(2)

    flush = not args.no_flush_mall
    calib = None if args.no_copy_calibration else copy_calibration()
    head = run_workload(args.workload, args.steps, args.warmup, check=not args.no_check,
                        flush_mall=flush)
    extras = {}
    for name in [e for e in args.extra.split(",") if e and e != args.workload]:
        if ms.CONFIGS[name].layout == "prefill":
            r = run_prefill_workload(name, args.steps, args.warmup, check=not args.no_check, flush_mall=flush)
            r["frac_of_peak"] = round(r["gbs"] / PEAK_HBM_GBS, 4)
            extras[name] = r
            continue
        r = run_workload(name, args.steps, args.warmup, check=not args.no_check, flush_mall=flush)
        extras[name] = {k: (round(v, 2) if isinstance(v, float) else v) for k, v in r.items()
                        if k in ("layer_us", "layer_mean_us", "dispatch_us", "combine_us", "gbs",
                                 "per_call_us", "per_call_gbs", "check", "dtype", "other_protocol",
                                 "hbm_only", "graph_replay_us_per_step", "N", "T", "H", "E", "R")}
        extras[name]["frac_of_peak"] = round(r["gbs"] / PEAK_HBM_GBS, 4)
        if "hbm_only" in r:
            extras[name]["frac_of_peak_note"] = ("effective: the bytes count the unpack's read of the "
                                                 "exchanged rows, which the memory-side cache serves; "
                                                 "hbm_only.frac_of_peak leaves them out")
    line = {
        "metric": METRIC,
        "value": round(head["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["wall_ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if head["dtype"] == "bf16" else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": args.workload, "N": head["N"], "T": head["T"], "H": head["H"],
                   "E": head["E"], "R": head["R"], "payload": head["dtype"],
                   "ranks_simulated_on_one_gpu": head["N"]},
        "us_per_layer": round(head["layer_us"], 2),
        "timing": "per-call HIP events on the kernels' stream; medians over the steps, summed",
        "dispatch_us": round(head["dispatch_us"], 2),
        "combine_us": round(head["combine_us"], 2),
        "frac_of_peak": round(head["gbs"] / PEAK_HBM_GBS, 4),
        "alg_bytes_per_layer": head["alg_bytes"]["total"],
        "per_call_us": head["per_call_us"],
        "us_per_layer_mean": round(head["layer_mean_us"], 2),
        "per_call_mean_us": head["per_call_mean_us"],
        "mall_flushed_between_steps": flush,
        "other_protocol": head["other_protocol"],
        "per_call_gbs": head["per_call_gbs"],
        "graph_replay_us_per_step": head["graph_replay_us_per_step"],
        "check": head.get("check"),
        "roofline": dominant_kernel(head, calib),
        "other_workloads": extras,
    }
    if not args.no_overlap:
        line["overlap"] = overlap_leg(HEADLINE)
    if not args.no_microbatch:
        line["micro_batches"] = microbatch_leg(HEADLINE)
    if not args.no_rank_leg:
        line["one_rank_share"] = [rank_leg(w) for w in (HEADLINE, "kimi_k2_worst")]
    if not args.no_acc_combine:
        line["acc_combine"] = [acc_combine_leg(w) for w in (HEADLINE, "kimi_k2_worst")]
    if calib is not None:
        line["copy_ceiling"] = calib
        line["frac_of_copy_ceiling"] = round(head["gbs"] / calib["stream_copy"]["gbs"], 4)
    if args.tokens_sweep:
        line["tokens_sweep"] = tokens_sweep(args.workload, [int(t) for t in args.tokens_sweep.split(",")],
                                            args.steps, args.warmup, check=not args.no_check)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    line["children_at_exit"] = end_children()
    print(json.dumps(line), flush=True)


def tokens_sweep(name, ts, steps, warmup, check=True) -> list:
    """The workload's shape at other tokens per rank (decode batch sizes): per-call medians with
    the memory-side cache flushed between steps, as the headline is timed."""
    import dataclasses

    import moe_synth as ms

    base = ms.CONFIGS[name]
    out = []
    for T in ts:
        c = dataclasses.replace(base, name=f"{name}@T{T}", T=T, desc=f"{base.desc} at T = {T}")
        ms.CONFIGS[c.name] = c
        try:
            r = run_workload(c.name, steps, warmup, check=check, flush_mall=True)
        finally:
            del ms.CONFIGS[c.name]
        out.append({"T": T, "us_per_layer": round(r["layer_us"], 2),
                    "frac_of_peak": round(r["gbs"] / PEAK_HBM_GBS, 4),
                    "graph_replay_us_per_step": r["graph_replay_us_per_step"],
                    "per_call_us": r["per_call_us"]})
    return out


def end_children() -> int:
    """Child processes this run left (none are started on purpose): end them so that nothing
    outlives the benchmark, and report how many there were."""
    try:
        import psutil
    except ImportError:
        return -1
    kids = psutil.Process().children(recursive=True)
    for k in kids:
        try:
            k.terminate()
        except psutil.Error:
            pass
    psutil.wait_procs(kids, timeout=5)
    for k in kids:
        try:
            if k.is_running():
                k.kill()
        except psutil.Error:
            pass
    return len(kids)


if __name__ == "__main__":
    main()
