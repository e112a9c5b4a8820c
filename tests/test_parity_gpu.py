"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, stage by stage.

Small shapes span several chunks, blocks and ragged tails; the full workloads run at their
real sizes with the launch configuration the benchmark times.  Every test prints the case it
runs before touching the GPU.
"""
import os

import numpy as np
import pytest
import torch

import moe_synth as ms
import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    yield
    gc.collect()
    torch.cuda.empty_cache()

# N, T, H, E, R, fp8, bias
SMALL = [
    (2, 16, 256, 8, 2, False, "none"),        # the tiny workload
    (3, 37, 264, 9, 3, False, "none"),        # ragged hidden size (33 chunks of 16 B)
    (4, 300, 512, 16, 4, True, "none"),       # fp8; T*R = 1200 spans two count chunks
    (8, 129, 1024, 64, 8, False, "zipf"),     # skewed, 2 chunks
    (1, 50, 128, 7, 3, False, "none"),        # a single rank: a stable counting sort
    (5, 7, 8, 5, 1, False, "none"),           # L = 1, R = 1: personalised all-to-all
    (2, 3, 16, 6, 6, False, "none"),          # R = E
    (16, 32, 512, 96, 8, True, "kimi"),       # Kimi-shaped skew, fp8
    (2, 700, 64, 32, 8, False, "none"),       # 5600 slots per rank: 6 count chunks
    (4, 64, 136, 256, 1, False, "zipf"),      # R = 1, many experts
    (64, 4, 8, 128, 2, False, "none"),        # 64 ranks: offset tables span a whole wave
    (65, 3, 8, 130, 3, False, "none"),        # 65 ranks: offset tables span two waves
]


def _case_id(c):
    return "N{}_T{}_H{}_E{}_R{}_{}_{}".format(c[0], c[1], c[2], c[3], c[4], "fp8" if c[5] else "bf16", c[6])


@pytest.mark.parametrize("case", SMALL, ids=[_case_id(c) for c in SMALL])
@pytest.mark.parametrize("seed", [0, 1])
def test_small_shapes(case, seed):
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase {_case_id(case)} seed {seed}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, seed)
    _, g = parity.gpu_run(N, T, H, E, R, fp8, inp)
    o = parity.oracle_run(N, T, H, E, R, fp8, inp)
    parity.compare(g, o, N, T, H, E, R, fp8)


@pytest.mark.parametrize("case", [SMALL[1], SMALL[2], SMALL[7]], ids=lambda c: _case_id(c))
def test_tagged_expert(case):
    # tagged experts make every expert's output distinct: pins the slot/weight/row pairing
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase tagged {_case_id(case)}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, 5)
    _, g = parity.gpu_run(N, T, H, E, R, fp8, inp, expert_mode=1)
    o = parity.oracle_run(N, T, H, E, R, fp8, inp, expert_mode=1)
    parity.compare(g, o, N, T, H, E, R, fp8)


@pytest.mark.parametrize("case", [SMALL[0], SMALL[3], SMALL[8]], ids=lambda c: _case_id(c))
def test_random_expert_outputs(case):
    # arbitrary expert outputs (mixed signs): combine is bit-exact against the fp32 fma chain
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase random-y {_case_id(case)}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, 2)
    B = N * T * max(R, E // N)
    y = ms.random_y(N, B, H, seed=4)
    idx = ms.random_topk(N, T, E, R, seed=3)
    _, g = parity.gpu_run(N, T, H, E, R, fp8, inp, y=y, topk_idx=idx)
    o = parity.oracle_run(N, T, H, E, R, fp8, inp, y=y, topk_idx=idx)
    parity.compare(g, o, N, T, H, E, R, fp8, check_stub=False, check_ulp=False)


@pytest.mark.parametrize("case", [SMALL[0], SMALL[2], SMALL[3]], ids=lambda c: _case_id(c))
def test_split_combine(case):
    # moe_combine_send then moe_combine_recv (on another stream) == moe_combine == the oracle
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase split-combine {_case_id(case)}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, 6)
    _, g = parity.gpu_run(N, T, H, E, R, fp8, inp, split_combine=True)
    _, f = parity.gpu_run(N, T, H, E, R, fp8, inp)
    assert np.array_equal(g["out"], f["out"])
    o = parity.oracle_run(N, T, H, E, R, fp8, inp)
    parity.compare(g, o, N, T, H, E, R, fp8)


def test_overlap_with_second_stream():
    # dispatch send on stream 1; GEMMs on stream 2 while the transfer and receive run on
    # stream 1; then combine: every output still matches the oracle
    import combine_moe_route_top_amd as moe
    N, T, H, E, R = 8, 129, 1024, 64, 8
    print("\ncase overlap", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, False, "zipf", 1)
    b = moe.alloc_buffers(N, T, H, E, R)
    parity.upload_inputs(b, inp)
    s1 = torch.cuda.current_stream()
    s2 = torch.cuda.Stream()
    a = torch.randn(2048, 2048, device="cuda", dtype=torch.bfloat16)
    moe.moe_route(b.shape, b.logits, b.bias, b.topk_idx, b.topk_w, s1)
    moe.moe_dispatch_send(b.shape, b.x, None, b.topk_idx, b.counts, b.send_off, b.send_pos,
                          b.send_buf, b.send_meta, b.workspace, s1)
    ev = torch.cuda.Event()
    ev.record(s1)
    s2.wait_event(ev)
    with torch.cuda.stream(s2):
        for _ in range(4):
            a = (a @ a) * 0.01
    moe.moe_net_dispatch(b.shape, b.send_off, b.send_buf, b.send_meta, b.recv_buf, b.recv_meta,
                         b.recv_off, s1)
    moe.moe_dispatch_recv(b.shape, b.counts, b.recv_off, b.recv_buf, b.recv_meta, b.expert_x,
                          None, b.expert_cnt, b.expert_off, b.expert_src, b.expert_rpos, s1)
    moe.moe_expert_stub(b.shape, 0, b.expert_x, None, b.expert_off, b.expert_y, s1)
    moe.moe_combine_send(b.shape, b.expert_y, b.expert_rpos, b.recv_off, b.send_off, b.cs_buf,
                         b.cr_buf, s1)
    s1.wait_stream(s2)
    moe.moe_combine_recv(b.shape, b.cr_buf, b.send_pos, b.topk_w, b.out, s1)
    torch.cuda.synchronize()
    g = parity.fetch(b, N, T, R)
    o = parity.oracle_run(N, T, H, E, R, False, inp)
    parity.compare(g, o, N, T, H, E, R, False)


def test_two_micro_batches_pipelined():
    # two micro-batches on two streams in the pipelined order (dispatch B while A's compute runs
    # on stream 2, combine A while B's compute runs): both match the oracle
    import combine_moe_route_top_amd as moe
    N, T, H, E, R = 8, 64, 1024, 64, 8
    print("\ncase micro-batches", flush=True)
    s1 = torch.cuda.current_stream()
    s2 = torch.cuda.Stream()
    inps, bufs = [], []
    for h in range(2):
        inp = ms.make_inputs(N, T, H, E, R, False, "zipf", 10 + h)
        b = moe.alloc_buffers(N, T, H, E, R)
        for k, t in b.t.items():
            if t is not None and k != "status":
                t.view(torch.uint8).fill_(0xA5)
        b.status.zero_()
        parity.upload_inputs(b, inp)
        inps.append(inp)
        bufs.append(b)
    a = torch.randn(2048, 2048, device="cuda", dtype=torch.bfloat16)

    def dispatch(b, st):
        moe.run_dispatch(b, stream=st)
        moe.moe_expert_stub(b.shape, 1, b.expert_x, None, b.expert_off, b.expert_y, st)

    def compute(st):
        nonlocal a
        with torch.cuda.stream(st):
            for _ in range(3):
                a = (a @ a) * 0.01

    def after(wait, done):
        ev = torch.cuda.Event()
        ev.record(done)
        wait.wait_event(ev)

    A, Bm = bufs
    dispatch(A, s1)
    after(s2, s1)
    compute(s2)
    dispatch(Bm, s1)
    after(s1, s2)
    after(s2, s1)
    moe.run_combine(A, stream=s1)
    compute(s2)
    after(s1, s2)
    moe.run_combine(Bm, stream=s1)
    torch.cuda.synchronize()
    for b, inp in zip(bufs, inps):
        g = parity.fetch(b, N, T, R)
        g["poisoned"] = True
        o = parity.oracle_run(N, T, H, E, R, False, inp, expert_mode=1)
        parity.compare(g, o, N, T, H, E, R, False)


@pytest.mark.parametrize("case", [SMALL[3], SMALL[7], SMALL[8], SMALL[11]], ids=lambda c: _case_id(c))
def test_rank_subrange_calls_compose(case):
    # every step called once per rank (as each GPU of a real deployment would), each step for all
    # ranks before the next, gives exactly the all-ranks result; ranges of 2 ranks as well
    import combine_moe_route_top_amd as moe
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase rank-subrange {_case_id(case)}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, 3)
    _, full = parity.gpu_run(N, T, H, E, R, fp8, inp, expert_mode=1)
    for width in (1, 2):
        b = moe.alloc_buffers(N, T, H, E, R, fp8)
        for t in b.t.values():
            if t is not None:
                t.view(torch.uint8).fill_(0x5A)
        b.status.zero_()
        parity.upload_inputs(b, inp)
        ranges = [(r0, min(width, N - r0)) for r0 in range(0, N, width)]
        sub = [moe.for_ranks(b.shape, r0, n) for r0, n in ranges]
        use_bias = inp["bias"] is not None
        for sh in sub:
            moe.moe_route(sh, b.logits, b.bias if use_bias else None, b.topk_idx, b.topk_w)
        for sh in sub:
            moe.moe_dispatch_send(sh, b.x, b.x_scale, b.topk_idx, b.counts, b.send_off, b.send_pos,
                                  b.send_buf, b.send_meta, b.workspace)
        for sh in sub:
            moe.moe_net_dispatch(sh, b.send_off, b.send_buf, b.send_meta, b.recv_buf, b.recv_meta,
                                 b.recv_off)
        for sh in sub:
            moe.moe_dispatch_recv(sh, b.counts, b.recv_off, b.recv_buf, b.recv_meta, b.expert_x,
                                  b.expert_scale, b.expert_cnt, b.expert_off, b.expert_src,
                                  b.expert_rpos)
        for sh in sub:
            moe.moe_expert_stub(sh, 1, b.expert_x, b.expert_scale, b.expert_off, b.expert_y)
        for sh in sub:
            moe.moe_combine_send(sh, b.expert_y, b.expert_rpos, b.recv_off, b.send_off, b.cs_buf,
                                 b.cr_buf)
        for sh in sub:
            moe.moe_combine_recv(sh, b.cr_buf, b.send_pos, b.topk_w, b.out)
        torch.cuda.synchronize()
        g = parity.fetch(b, N, T, R)
        for k in ("topk_idx", "topk_w", "counts", "send_off", "send_pos", "recv_off", "expert_cnt",
                  "expert_off", "out", "status"):
            assert np.array_equal(g[k], full[k]), (width, k)
        for k in ("send_rows", "send_meta", "recv_rows", "recv_meta", "expert_x", "expert_src",
                  "expert_rpos", "expert_y", "cs_buf", "cr_buf"):
            for d in range(N):
                assert np.array_equal(g[k][d], full[k][d]), (width, k, d)


def _token_counts(N, T, seed):
    """Per-rank token counts with an empty rank, a full rank and (N > 2) a one-token rank."""
    t = np.random.default_rng(seed).integers(0, T + 1, N).astype(np.int32)
    t[0], t[-1] = 0, T
    if N > 2:
        t[1] = 1
    return t


VARTOK = [SMALL[1], SMALL[2], SMALL[3], SMALL[7], SMALL[10]]


@pytest.mark.parametrize("case", VARTOK, ids=lambda c: _case_id(c))
@pytest.mark.parametrize("split", [False, True])
def test_variable_tokens(case, split):
    # rank s dispatches only its first tokens[s] tokens; rows of the others are not written
    N, T, H, E, R, fp8, bias = case
    tokens = _token_counts(N, T, 5)
    print(f"\ncase tokens {_case_id(case)} split {split} tokens {tokens.tolist()}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, 2)
    _, g = parity.gpu_run(N, T, H, E, R, fp8, inp, tokens=tokens, split_combine=split)
    o = parity.oracle_run(N, T, H, E, R, fp8, inp, tokens=tokens)
    parity.compare(g, o, N, T, H, E, R, fp8)
    assert g["counts"].sum() == int(tokens.sum()) * R


def test_bad_token_count_sets_status():
    # a count above T flags MOE_EINVAL and the rank dispatches nothing; every kernel finishes
    import combine_moe_route_top_amd as moe
    N, T, H, E, R = 2, 8, 64, 8, 2
    print("\ncase bad token count", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, False, "none", 0)
    tokens = np.array([T + 1, 5], np.int32)
    _, g = parity.gpu_run(N, T, H, E, R, False, inp, tokens=tokens)
    assert g["status"][0] == moe.MOE_EINVAL
    assert g["counts"][0].sum() == 0 and g["counts"][1].sum() == 5 * R
    assert np.all(g["send_pos"][0] == -1)
    assert np.all(g["out"][0] == 0xA5A5)


def _quant_inputs(N, T, H, E, R, bias, seed):
    """bf16 tokens with magnitudes spread over 2^-30 .. 2^30 per token, an all-zero block, a
    block with one large value among small ones, and values in the e4m3 subnormal range."""
    inp = ms.make_inputs(N, T, H, E, R, False, bias, seed)
    xf = ms.bf16_bits_to_f32(inp["x"]).copy()
    rng = np.random.default_rng(seed + 50)
    xf *= np.exp2(rng.integers(-30, 31, (N, T, 1))).astype(np.float32)
    xf[0, 0, :128] = 0.0
    if T > 1:
        xf[0, 1, 128:256] *= np.float32(1e-3)
        xf[0, 1, 130] = 5.0
    inp["x"] = ms.to_bf16_bits(xf.astype(np.float32))
    return inp


QUANT = [  # N, T, H, E, R, bias
    (4, 300, 512, 16, 4, "none"),      # half a pass per token; two count chunks
    (16, 32, 512, 96, 8, "kimi"),
    (2, 5, 7168, 8, 4, "none"),        # seven passes of 1024 values
    (3, 9, 1536, 12, 3, "zipf"),       # one and a half passes
    (8, 129, 1024, 64, 8, "zipf"),
]


@pytest.mark.parametrize("case", QUANT, ids=lambda c: "N{}_T{}_H{}_E{}_R{}_{}".format(*c))
def test_fused_quant(case):
    # bf16 tokens quantised to e4m3 rows by the send pack: every byte of every stage matches the
    # oracle's quantiser followed by the e4m3 path
    N, T, H, E, R, bias = case
    print(f"\ncase quant {case}", flush=True)
    inp = _quant_inputs(N, T, H, E, R, bias, 6)
    _, g = parity.gpu_run(N, T, H, E, R, True, inp, quant=True)
    o = parity.oracle_run(N, T, H, E, R, False, inp, quant=True)
    parity.compare(g, o, N, T, H, E, R, True)


def test_fused_quant_with_token_counts():
    N, T, H, E, R, bias = 8, 129, 1024, 64, 8, "zipf"
    tokens = _token_counts(N, T, 8)
    print(f"\ncase quant + tokens {tokens.tolist()}", flush=True)
    inp = _quant_inputs(N, T, H, E, R, bias, 7)
    _, g = parity.gpu_run(N, T, H, E, R, True, inp, quant=True, tokens=tokens, split_combine=True)
    o = parity.oracle_run(N, T, H, E, R, False, inp, quant=True, tokens=tokens)
    parity.compare(g, o, N, T, H, E, R, True)


def test_tight_capacity():
    # receive buffers sized to the tight bound N*T*min(R, E/N) instead of N*T*max(R, E/N)
    N, T, H, E, R = 4, 40, 64, 32, 8
    print("\ncase tight capacity", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, False, "zipf", 7)
    _, g = parity.gpu_run(N, T, H, E, R, False, inp, capacity=N * T * min(R, E // N))
    o = parity.oracle_run(N, T, H, E, R, False, inp)
    parity.compare(g, o, N, T, H, E, R, False)


def _sweep_case(seed):
    """A seeded random configuration: ranks, experts per rank, slots, tokens, hidden size, payload
    type, bias, per-rank token counts, receive capacity and combine form all drawn together."""
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 33]))
    L = int(rng.integers(1, 7))
    E = N * L
    R = int(rng.integers(1, min(E, 9) + 1))
    T = int(rng.integers(1, 161))
    kind = rng.choice(["bf16", "bf16", "fp8", "quant"])
    H = int(rng.choice([512, 1024])) if kind != "bf16" else 8 * int(rng.integers(1, 97))
    bias = str(rng.choice(["none", "zipf"]))
    with_tokens = rng.random() < 0.4 or os.environ.get("MOE_SWEEP_TOKENS") == "1"
    tokens = rng.integers(0, T + 1, N).astype(np.int32) if with_tokens else None
    tight = bool(rng.random() < 0.25)
    split = bool(rng.random() < 0.5)
    return N, T, H, E, R, str(kind), bias, tokens, tight, split


# 96 seeds by default; a wider one-off run sets MOE_SWEEP_SEEDS=first:last (and MOE_SWEEP_TOKENS=1
# to give every case per-rank token counts)
_SWEEP = [int(v) for v in os.environ.get("MOE_SWEEP_SEEDS", "0:96").split(":")]


@pytest.mark.parametrize("seed", range(*_SWEEP))
def test_random_shape_sweep(seed):
    # random configurations, each compared with the oracle stage by stage
    N, T, H, E, R, kind, bias, tokens, tight, split = _sweep_case(seed)
    print(f"\ncase sweep {seed}: N{N} T{T} H{H} E{E} R{R} {kind} {bias} tokens "
          f"{None if tokens is None else tokens.tolist()} tight {tight} split {split}", flush=True)
    cap = N * T * min(R, E // N) if tight else 0
    if kind == "quant":
        inp = _quant_inputs(N, T, H, E, R, bias, seed)
        _, g = parity.gpu_run(N, T, H, E, R, True, inp, capacity=cap, quant=True, tokens=tokens,
                              split_combine=split)
        o = parity.oracle_run(N, T, H, E, R, False, inp, quant=True, tokens=tokens)
    else:
        fp8 = kind == "fp8"
        inp = ms.make_inputs(N, T, H, E, R, fp8, bias, seed)
        _, g = parity.gpu_run(N, T, H, E, R, fp8, inp, capacity=cap, tokens=tokens,
                              split_combine=split)
        o = parity.oracle_run(N, T, H, E, R, fp8, inp, tokens=tokens)
    parity.compare(g, o, N, T, H, E, R, kind != "bf16")


# the ABI's largest N, E and R with small T and H: tables over 1024 ranks, 1024 experts,
# 64 slots per token (the router's 64-lane groups with 16 experts per lane)
LIMITS = [
    (1024, 2, 8, 1024, 4, False, "none"),     # N = E = 1024: one expert per rank
    (4, 16, 64, 1024, 64, False, "zipf"),     # R = 64 of E = 1024
    (16, 9, 512, 1024, 64, True, "none"),     # R = 64, e4m3, 64 experts per rank
]


@pytest.mark.parametrize("case", LIMITS, ids=_case_id)
def test_largest_supported_shapes(case):
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase limits {_case_id(case)}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, 0)
    _, g = parity.gpu_run(N, T, H, E, R, fp8, inp, split_combine=True)
    o = parity.oracle_run(N, T, H, E, R, fp8, inp)
    parity.compare(g, o, N, T, H, E, R, fp8)


def test_no_tokens_anywhere():
    # every rank dispatches zero tokens: empty counts, segments and receive sides everywhere; no
    # output row is written and every kernel still finishes
    N, T, H, E, R = 8, 33, 64, 32, 4
    print("\ncase zero tokens", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, False, "none", 1)
    tokens = np.zeros(N, np.int32)
    _, g = parity.gpu_run(N, T, H, E, R, False, inp, tokens=tokens)
    o = parity.oracle_run(N, T, H, E, R, False, inp, tokens=tokens)
    parity.compare(g, o, N, T, H, E, R, False)
    assert g["counts"].sum() == 0 and g["recv_off"].sum() == 0 and g["expert_off"].sum() == 0


def test_everything_to_one_rank():
    # bias +16 on rank 0's experts with R <= L: every slot goes to rank 0, the other ranks
    # receive nothing (empty segments and empty ranks everywhere)
    N, T, H, E, R = 4, 33, 64, 16, 4
    print("\ncase all-to-rank-0", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, False, "none", 3)
    inp["bias"] = np.zeros(E, np.float32)
    inp["bias"][:4] = 16.0
    _, g = parity.gpu_run(N, T, H, E, R, False, inp)
    o = parity.oracle_run(N, T, H, E, R, False, inp)
    assert g["recv_off"][1:, N].sum() == 0
    parity.compare(g, o, N, T, H, E, R, False)


def test_repeat_is_deterministic():
    # the same buffers run twice give identical results (nothing depends on stale contents)
    import combine_moe_route_top_amd as moe
    N, T, H, E, R = 8, 129, 1024, 64, 8
    print("\ncase repeat", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, False, "zipf", 0)
    b, g1 = parity.gpu_run(N, T, H, E, R, False, inp)
    b.expert_x.fill_(0x5A5A)
    b.out.fill_(0)
    moe.run_dispatch(b)
    moe.moe_expert_stub(b.shape, 0, b.expert_x, b.expert_scale, b.expert_off, b.expert_y)
    moe.run_combine(b)
    torch.cuda.synchronize()
    g2 = parity.fetch(b, N, T, R)
    for k in ("out", "send_pos", "recv_off"):
        assert np.array_equal(g1[k], g2[k])
    for d in range(N):
        assert np.array_equal(g1["expert_x"][d], g2["expert_x"][d])


def test_bad_expert_ids_set_status():
    # out-of-range ids and a repeated id are dropped and flagged; every kernel still finishes
    N, T, H, E, R = 2, 8, 64, 8, 2
    print("\ncase bad ids", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, False, "none", 0)
    idx = ms.random_topk(N, T, E, R, seed=1)
    idx[0, 0, 0] = E          # out of range
    idx[1, 2, 1] = idx[1, 2, 0]  # repeated within a token
    idx[1, 3, 0] = -1         # negative
    _, g = parity.gpu_run(N, T, H, E, R, False, inp, topk_idx=idx)
    import combine_moe_route_top_amd as moe
    assert g["status"][0] == moe.MOE_EBADIDX
    sp = g["send_pos"].reshape(N, T, R)
    assert sp[0, 0, 0] == -1 and sp[1, 2, 1] == -1 and sp[1, 3, 0] == -1
    assert g["counts"].sum() == N * T * R - 3
    assert np.all(g["send_off"][:, N] == T * R - np.array([1, 2]))


FULL = ["tiny", "mixtral_8x7b_decode", "deepseek_v3_decode", "deepseek_v3_decode_fp8",
        "qwen3_235b_prefill", "kimi_k2_worst", "deepseek_v3_decode_fp8q",
        "deepseek_v3_decode_ragged"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_full_workload(name):
    c = ms.CONFIGS[name]
    print(f"\ncase full {name}", flush=True)
    inp = ms.config_inputs(c)
    tokens = ms.config_tokens(c)
    # every output pre-filled with 0xA5 bytes, as in the small cases: a row no kernel wrote
    # cannot pass for a result
    _, g = parity.gpu_run(c.N, c.T, c.H, c.E, c.R, c.rows_fp8, inp, poison=True,
                          quant=c.quant, tokens=tokens)
    print("  gpu done", flush=True)
    o = parity.oracle_run(c.N, c.T, c.H, c.E, c.R, c.fp8, inp, quant=c.quant, tokens=tokens)
    print("  oracle done", flush=True)
    st = parity.compare(g, o, c.N, c.T, c.H, c.E, c.R, c.rows_fp8)
    print(" ", st, flush=True)
    if name == "kimi_k2_worst":
        assert g["recv_off"][0, c.N] == 49152


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 16, (1 << 24) + 48])
def test_stream_copy_is_exact(nbytes):
    # the copy-ceiling probe: whole blocks and a ragged last block, byte for byte
    import combine_moe_route_top_amd as moe
    print(f"\ncase stream copy {nbytes} bytes", flush=True)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    moe.moe_stream_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())
