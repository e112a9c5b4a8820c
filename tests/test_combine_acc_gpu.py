"""GPU parity of the combine with the sum taken on the sending side (moe_combine_acc*).

The dispatch runs first and is checked as in test_parity_gpu; the combine then runs on the same
buffers and is compared with the oracle's oracle_combine_acc: the fp32-step mode (mode 1) bit
for bit -- every partial row where it belongs, rows that hold no partial untouched, the output --
and the distance to the fp64-step mode (mode 0) and to the receive-side combine is reported.
"""
import numpy as np
import pytest
import torch

import moe_synth as ms
import oracle
import parity

pytestmark = pytest.mark.gpu

POISON = 0x5A5A


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _first_rows(recv_meta_d, ro_d, T, R):
    """Receive rows of one rank that are their token's first row there (ro_d = recv_off[d])."""
    tok = (recv_meta_d[:, 0] % (T * R)) // R
    n = len(tok)
    first = np.ones(n, bool)
    if n > 1:
        first[1:] = tok[1:] != tok[:-1]
    first[ro_d[:-1][ro_d[:-1] < n]] = True  # every segment starts a token
    return first


def _acc_run(b, N, T, H, E, R, split=False):
    import combine_moe_route_top_amd as moe
    for t in (b.cs_buf, b.cr_buf, b.out):
        t.view(torch.int16).fill_(POISON)
    b.status.zero_()
    if split:
        moe.moe_combine_acc_send(b.shape, b.expert_y, b.recv_meta, b.counts, b.recv_off, b.expert_off,
                                 b.send_off, b.topk_w, b.cs_buf, b.cr_buf)
        ev = torch.cuda.Event()
        ev.record()
        side = torch.cuda.Stream()
        side.wait_event(ev)
        moe.moe_combine_acc_recv(b.shape, b.cr_buf, b.topk_idx, b.send_pos, b.out, side)
        torch.cuda.current_stream().wait_stream(side)
    else:
        moe.run_combine_acc(b)
    torch.cuda.synchronize()
    return parity.fetch(b, N, T, R)


def _check_acc(g, g_std, o, N, T, H, E, R, tokens=None):
    """g: outputs after the accumulating combine; g_std: after the receive-side combine; o: the
    oracle run of the same inputs.  Returns statistics."""
    L = E // N
    TR = T * R
    sh = o["shape"]
    assert g["status"][0] == 0, f"device status word {g['status'][0]}"
    w = o["topk_w"]
    idx = o["topk_idx"].reshape(N, TR)
    acc = {m: oracle.combine_acc(sh, m, o["expert_y"], o["expert_src"], o["expert_rpos"], o["recv_off"],
                                 o["send_off"], idx, o["send_pos"], w) for m in (0, 1)}
    nt = np.full(N, T) if tokens is None else np.asarray(tokens)
    present = (np.arange(T)[None, :] < nt[:, None]).reshape(N * T)
    same_w = np.all(g["topk_w"].reshape(N * T, R) == w, axis=1)
    # expert side: partials at each token's first receive row, other rows untouched
    for d in range(N):
        ro = o["recv_off"][d]
        first = _first_rows(g["recv_meta"][d], ro, T, R)
        want = sh.rank_rows(acc[1]["cs_buf"], d)
        got = g["cs_buf"][d]
        assert np.array_equal(got[first], want[first]), f"cs_buf partials, rank {d}"
        assert np.all(got[~first] == POISON), f"cs_buf rank {d}: a row without a partial was written"
    # network back: partials at the send position of each token's first slot per owner
    sp = o["send_pos"]
    for s in range(N):
        n = o["send_off"][s, N]
        holds = np.zeros(n, bool)
        for t in range(int(nt[s])):
            seen = set()
            for k in range(R):
                p = sp[s, t * R + k]
                if p < 0:
                    continue
                d = int(idx[s, t * R + k]) // L
                if d not in seen:
                    seen.add(d)
                    holds[p] = True
        got = g["cr_buf"][s]
        assert np.array_equal(got[holds], acc[1]["cr_buf"][s, :n][holds]), f"cr_buf partials, rank {s}"
        assert np.all(got[~holds] == POISON), f"cr_buf rank {s}: a row without a partial was written"
    out = g["out"].reshape(N * T, H)
    assert np.all(out[~present] == POISON), "combine wrote absent tokens"
    ok = present & same_w
    o1 = acc[1]["out"].reshape(N * T, H)
    assert np.array_equal(out[ok], o1[ok]), "out vs the oracle's fp32 steps"
    stats = {"tokens_checked": int(ok.sum())}
    d0 = parity._bf16_ulp_diff(out[present], acc[0]["out"].reshape(N * T, H)[present])
    dstd = parity._bf16_ulp_diff(out[present], g_std["out"].reshape(N * T, H)[present])
    stats["max_ulp_vs_fp64_steps"] = int(d0.max(initial=0))
    stats["max_ulp_vs_receive_side_sum"] = int(dstd.max(initial=0))
    stats["frac_equal_to_receive_side_sum"] = float((dstd == 0).mean()) if dstd.size else 1.0
    return stats


SMALL = [  # N, T, H, E, R, fp8, bias
    (2, 16, 256, 8, 2, False, "none"),        # the tiny workload
    (3, 37, 264, 9, 3, False, "none"),        # ragged hidden size; L = 3
    (4, 300, 512, 16, 4, True, "none"),       # fp8; two count chunks
    (8, 129, 1024, 64, 8, False, "zipf"),     # skewed
    (1, 50, 128, 7, 3, False, "none"),        # a single rank: one partial per token
    (5, 7, 8, 5, 1, False, "none"),           # R = 1
    (2, 3, 16, 6, 6, False, "none"),          # R = E: 3 rows per token and owner
    (16, 32, 512, 96, 8, True, "kimi"),       # Kimi-shaped: 6 rows of each token at rank 0
    (65, 3, 8, 130, 3, False, "none"),        # 65 ranks
    (2, 20, 256, 64, 16, False, "none"),      # up to 16 rows of a token at one rank (two groups of 8)
    (2, 5, 64, 128, 64, False, "zipf"),       # R = 64: up to 64 rows of a token at one rank
]


def _case_id(c):
    return "N{}_T{}_H{}_E{}_R{}_{}_{}".format(c[0], c[1], c[2], c[3], c[4], "fp8" if c[5] else "bf16", c[6])


@pytest.mark.parametrize("case", SMALL, ids=[_case_id(c) for c in SMALL])
@pytest.mark.parametrize("expert_mode", [0, 1], ids=["identity", "tagged"])
def test_acc_small_shapes(case, expert_mode):
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase acc {_case_id(case)} expert mode {expert_mode}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, 5)
    b, g_std = parity.gpu_run(N, T, H, E, R, fp8, inp, expert_mode=expert_mode)
    o = parity.oracle_run(N, T, H, E, R, fp8, inp, expert_mode=expert_mode)
    parity.compare(g_std, o, N, T, H, E, R, fp8)
    g = _acc_run(b, N, T, H, E, R)
    st = _check_acc(g, g_std, o, N, T, H, E, R)
    print(st, flush=True)
    if R == 1 or N == 1:  # one row per token and owner: the two combines agree exactly
        assert st["max_ulp_vs_receive_side_sum"] == 0


@pytest.mark.parametrize("case", [SMALL[1], SMALL[3], SMALL[6]], ids=lambda c: _case_id(c))
def test_acc_random_expert_outputs(case):
    # arbitrary mixed-sign expert outputs
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase acc random-y {_case_id(case)}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, 6)
    B = N * T * max(R, E // N)
    y = ms.random_y(N, B, H, seed=8)
    b, g_std = parity.gpu_run(N, T, H, E, R, fp8, inp, y=y)
    o = parity.oracle_run(N, T, H, E, R, fp8, inp, y=y)
    parity.compare(g_std, o, N, T, H, E, R, fp8, check_stub=False, check_ulp=False)
    g = _acc_run(b, N, T, H, E, R, split=True)
    print(_check_acc(g, g_std, o, N, T, H, E, R), flush=True)


@pytest.mark.parametrize("case", [SMALL[2], SMALL[3], SMALL[7]], ids=lambda c: _case_id(c))
def test_acc_token_counts_split(case):
    # per-rank token counts (an empty rank, a one-token rank, a full rank); the two halves on
    # different streams
    N, T, H, E, R, fp8, bias = case
    rng = np.random.default_rng(9)
    tokens = rng.integers(0, T + 1, N).astype(np.int32)
    tokens[0], tokens[-1] = 0, T
    tokens[1] = 1
    print(f"\ncase acc tokens {_case_id(case)} {tokens.tolist()}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, 7)
    b, g_std = parity.gpu_run(N, T, H, E, R, fp8, inp, expert_mode=1, tokens=tokens)
    o = parity.oracle_run(N, T, H, E, R, fp8, inp, expert_mode=1, tokens=tokens)
    parity.compare(g_std, o, N, T, H, E, R, fp8)
    g = _acc_run(b, N, T, H, E, R, split=True)
    print(_check_acc(g, g_std, o, N, T, H, E, R, tokens=tokens), flush=True)


@pytest.mark.parametrize("case", [SMALL[3], SMALL[7]], ids=lambda c: _case_id(c))
def test_acc_rank_subrange_calls_compose(case):
    # each rank's send half, then each rank's receive half, gives the all-ranks result
    import combine_moe_route_top_amd as moe
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase acc rank-subrange {_case_id(case)}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, 3)
    b, _ = parity.gpu_run(N, T, H, E, R, fp8, inp, expert_mode=1)
    full = _acc_run(b, N, T, H, E, R)
    for t in (b.cs_buf, b.cr_buf, b.out):
        t.view(torch.int16).fill_(POISON)
    for r in range(N):
        sh = moe.for_ranks(b.shape, r, 1)
        moe.moe_combine_acc_send(sh, b.expert_y, b.recv_meta, b.counts, b.recv_off, b.expert_off,
                                 b.send_off, b.topk_w, b.cs_buf, b.cr_buf)
    for r in range(N):
        sh = moe.for_ranks(b.shape, r, 1)
        moe.moe_combine_acc_recv(sh, b.cr_buf, b.topk_idx, b.send_pos, b.out)
    torch.cuda.synchronize()
    g = parity.fetch(b, N, T, R)
    assert g["status"][0] == 0
    assert np.array_equal(g["out"], full["out"])
    for d in range(N):
        assert np.array_equal(g["cs_buf"][d], full["cs_buf"][d]), d
        assert np.array_equal(g["cr_buf"][d], full["cr_buf"][d]), d


@pytest.mark.parametrize("name", ["deepseek_v3_decode", "kimi_k2_worst"])
def test_acc_full_workload(name):
    # the full-size workloads, tagged experts (every contribution of a token distinct)
    c = ms.CONFIGS[name]
    print(f"\ncase acc full {name}", flush=True)
    inp = ms.config_inputs(c)
    b, g_std = parity.gpu_run(c.N, c.T, c.H, c.E, c.R, c.fp8, inp, expert_mode=1)
    o = parity.oracle_run(c.N, c.T, c.H, c.E, c.R, c.fp8, inp, expert_mode=1)
    parity.compare(g_std, o, c.N, c.T, c.H, c.E, c.R, c.fp8)
    g = _acc_run(b, c.N, c.T, c.H, c.E, c.R)
    print(_check_acc(g, g_std, o, c.N, c.T, c.H, c.E, c.R), flush=True)


def test_acc_bad_expert_ids():
    # dropped slots (out-of-range, negative and repeated ids) add nothing; a token's output depends
    # only on its own rows, so tokens whose ids are untouched match the clean run bit for bit, and
    # a token left with one valid slot of weight 1/2 gives exactly x / 2 (identity experts)
    import combine_moe_route_top_amd as moe
    N, T, H, E, R = 2, 8, 64, 8, 2
    print("\ncase acc bad ids", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, False, "none", 0)
    clean = ms.random_topk(N, T, E, R, seed=1)
    bad = clean.copy()
    bad[0, 0, 0] = E             # out of range
    bad[1, 2, 1] = bad[1, 2, 0]  # repeated within a token
    bad[1, 3, 0] = -1            # negative
    outs = {}
    for name, idx in (("clean", clean), ("bad", bad)):
        b, g = parity.gpu_run(N, T, H, E, R, False, inp, topk_idx=idx)
        assert g["status"][0] == (moe.MOE_EBADIDX if name == "bad" else 0), name
        outs[name] = _acc_run(b, N, T, H, E, R)  # the combine itself finds nothing wrong
        assert outs[name]["status"][0] == 0, name
    touched = np.any(bad != clean, axis=2)
    go, gc = outs["bad"]["out"], outs["clean"]["out"]
    assert np.array_equal(go[~touched], gc[~touched])
    half = ms.to_bf16_bits(ms.bf16_bits_to_f32(inp["x"]) * np.float32(0.5))
    for s, t in zip(*np.nonzero(touched)):
        assert np.array_equal(go[s, t], half[s, t]), (s, t)


def test_acc_graph_replay_matches_eager():
    # the layer with the send-side-sum combine captured in a HIP graph and replayed for new inputs
    import combine_moe_route_top_amd as moe
    N, T, H, E, R = 8, 64, 512, 64, 8
    print("\ncase acc graph", flush=True)
    g_buf = moe.alloc_buffers(N, T, H, E, R)
    e_buf = moe.alloc_buffers(N, T, H, E, R)
    inputs = [ms.make_inputs(N, T, H, E, R, False, "zipf", seed) for seed in range(3)]

    def layer(b):
        moe.moe_route(b.shape, b.logits, b.bias, b.topk_idx, b.topk_w)
        moe.moe_dispatch_send(b.shape, b.x, None, b.topk_idx, b.counts, b.send_off, b.send_pos, b.send_buf,
                              b.send_meta, b.workspace)
        moe.moe_net_dispatch(b.shape, b.send_off, b.send_buf, b.send_meta, b.recv_buf, b.recv_meta, b.recv_off)
        moe.moe_dispatch_recv(b.shape, b.counts, b.recv_off, b.recv_buf, b.recv_meta, b.expert_x, None,
                              b.expert_cnt, b.expert_off, b.expert_src, b.expert_rpos)
        moe.moe_expert_stub(b.shape, 1, b.expert_x, None, b.expert_off, b.expert_y)
        moe.run_combine_acc(b)

    parity.upload_inputs(g_buf, inputs[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(g_buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(g_buf)
    torch.cuda.synchronize()
    for i, inp in enumerate(inputs * 2):
        parity.upload_inputs(g_buf, inp)
        graph.replay()
        parity.upload_inputs(e_buf, inp)
        layer(e_buf)
        torch.cuda.synchronize()
        assert np.array_equal(g_buf.out.cpu().numpy(), e_buf.out.cpu().numpy()), i
        assert int(g_buf.status.item()) == 0
    # and the last replay against the oracle's fp32 steps
    o = parity.oracle_run(N, T, H, E, R, False, inputs[-1], expert_mode=1)
    g = parity.fetch(g_buf, N, T, R)
    acc = oracle.combine_acc(o["shape"], 1, o["expert_y"], o["expert_src"], o["expert_rpos"], o["recv_off"],
                             o["send_off"], o["topk_idx"].reshape(N, T * R), o["send_pos"], o["topk_w"])
    same_w = np.all(g["topk_w"].reshape(N * T, R) == o["topk_w"], axis=1)
    assert same_w.mean() > 0.99
    assert np.array_equal(g["out"].reshape(N * T, H)[same_w], acc["out"].reshape(N * T, H)[same_w])


@pytest.mark.parametrize("seed", range(24))
def test_acc_random_shape_sweep(seed):
    # seeded random configurations: ranks, experts per rank, slots, tokens, hidden size, payload,
    # bias and per-rank token counts drawn together
    rng = np.random.default_rng(2000 + seed)
    N = int(rng.choice([1, 2, 3, 5, 8, 16, 33]))
    L = int(rng.integers(1, 9))
    E = N * L
    R = int(rng.integers(1, min(E, 12) + 1))
    T = int(rng.integers(1, 130))
    fp8 = bool(rng.random() < 0.3)
    H = int(rng.choice([512, 1024])) if fp8 else 8 * int(rng.integers(1, 97))
    bias = str(rng.choice(["none", "zipf"]))
    tokens = rng.integers(0, T + 1, N).astype(np.int32) if rng.random() < 0.4 else None
    print(f"\ncase acc sweep {seed}: N{N} T{T} H{H} E{E} R{R} fp8 {fp8} {bias} tokens "
          f"{None if tokens is None else tokens.tolist()}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, seed)
    b, g_std = parity.gpu_run(N, T, H, E, R, fp8, inp, expert_mode=1, tokens=tokens)
    o = parity.oracle_run(N, T, H, E, R, fp8, inp, expert_mode=1, tokens=tokens)
    parity.compare(g_std, o, N, T, H, E, R, fp8)
    g = _acc_run(b, N, T, H, E, R, split=bool(seed % 2))
    print(_check_acc(g, g_std, o, N, T, H, E, R, tokens=tokens), flush=True)


def test_acc_no_tokens_anywhere():
    # every rank dispatches zero tokens: nothing is received, no partial formed, no output written
    N, T, H, E, R = 4, 16, 64, 8, 2
    print("\ncase acc no tokens", flush=True)
    tokens = np.zeros(N, np.int32)
    inp = ms.make_inputs(N, T, H, E, R, False, "none", 1)
    b, g_std = parity.gpu_run(N, T, H, E, R, False, inp, tokens=tokens)
    assert g_std["status"][0] == 0 and np.all(g_std["recv_off"] == 0)
    g = _acc_run(b, N, T, H, E, R, split=True)
    assert g["status"][0] == 0
    assert np.all(g["out"] == POISON)
