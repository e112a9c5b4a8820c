"""GPU parity of the replicated-token (prefill) path through the C ABI against the CPU oracle.

Every rank holds the same tokens: dispatch selects each rank's slots in expert-major order,
combine accumulates each rank's contributions locally and all-reduces the partials.  Layout and
payload bit-exact; partials and output bit-exact against the oracle's fp32 steps and within
1 bf16 ulp of its fp64 sum.  Every test prints its case before touching the GPU.
"""
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
CASES = [
    (2, 16, 256, 8, 2, False, "none"),
    (4, 300, 512, 16, 4, True, "none"),      # e4m3; T*R = 1200 spans two count chunks
    (4, 1030, 264, 128, 8, False, "zipf"),   # 8240 slots: nine chunks; ragged hidden size
    (1, 50, 128, 7, 3, False, "none"),       # one rank
    (8, 33, 1024, 64, 8, False, "kimi"),     # rank 0's experts take six slots of every token
    (3, 7, 16, 6, 6, False, "none"),         # R = E
    (65, 3, 8, 130, 3, False, "none"),       # 65 ranks
]


def _id(c):
    return "N{}_T{}_H{}_E{}_R{}_{}_{}".format(c[0], c[1], c[2], c[3], c[4], "fp8" if c[5] else "bf16", c[6])


@pytest.mark.parametrize("case", CASES, ids=_id)
@pytest.mark.parametrize("split", [False, True])
def test_prefill_small(case, split):
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase prefill {_id(case)} split {split}", flush=True)
    inp = parity.prefill_inputs(T, H, E, R, fp8, bias, 1)
    _, g = parity.gpu_run_prefill(N, T, H, E, R, fp8, inp, split=split)
    o = parity.oracle_run_prefill(N, T, H, E, R, fp8, inp)
    parity.compare_prefill(g, o, N, T, H, E, R, fp8)


@pytest.mark.parametrize("case", [CASES[1], CASES[2], CASES[4]], ids=_id)
def test_prefill_tagged_expert(case):
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase prefill tagged {_id(case)}", flush=True)
    inp = parity.prefill_inputs(T, H, E, R, fp8, bias, 2)
    _, g = parity.gpu_run_prefill(N, T, H, E, R, fp8, inp, expert_mode=1)
    o = parity.oracle_run_prefill(N, T, H, E, R, fp8, inp, expert_mode=1)
    parity.compare_prefill(g, o, N, T, H, E, R, fp8)


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[4]], ids=_id)
def test_prefill_random_expert_outputs(case):
    # arbitrary mixed-sign expert outputs: partial sums and the rank-order all-reduce round
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase prefill random y {_id(case)}", flush=True)
    inp = parity.prefill_inputs(T, H, E, R, fp8, bias, 3)
    B = T * max(R, E // N)
    y = ms.random_y(N, B, H, seed=4)
    _, g = parity.gpu_run_prefill(N, T, H, E, R, fp8, inp, y=y)
    o = parity.oracle_run_prefill(N, T, H, E, R, fp8, inp, y=y)
    parity.compare_prefill(g, o, N, T, H, E, R, fp8, check_stub=False, check_ulp=False)


@pytest.mark.parametrize("case", [CASES[2], CASES[4], CASES[6]], ids=_id)
@pytest.mark.parametrize("width", [1, 2])
def test_prefill_rank_subrange_calls_compose(case, width):
    # each rank's dispatch, stand-in expert and local combine called separately, then the
    # all-reduce: the same result as the all-rank calls
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase prefill ranks {_id(case)} width {width}", flush=True)
    inp = parity.prefill_inputs(T, H, E, R, fp8, bias, 5)
    _, g = parity.gpu_run_prefill(N, T, H, E, R, fp8, inp, width=width)
    o = parity.oracle_run_prefill(N, T, H, E, R, fp8, inp)
    parity.compare_prefill(g, o, N, T, H, E, R, fp8)


def test_prefill_tight_capacity():
    N, T, H, E, R = 4, 40, 64, 32, 8
    print("\ncase prefill tight capacity", flush=True)
    inp = parity.prefill_inputs(T, H, E, R, False, "zipf", 6)
    _, g = parity.gpu_run_prefill(N, T, H, E, R, False, inp, capacity=T * min(R, E // N))
    o = parity.oracle_run_prefill(N, T, H, E, R, False, inp)
    for d in range(N):
        n = int(o["expert_off"][d, -1])
        assert np.array_equal(g["expert_x"][d], o["expert_x"][d, :n])
    assert np.array_equal(g["slot_pos"], o["slot_pos"]) and np.array_equal(g["out"], o["out1"])


def test_prefill_bad_expert_ids_set_status():
    import combine_moe_route_top_amd as moe
    N, T, H, E, R = 2, 8, 64, 8, 2
    print("\ncase prefill bad ids", flush=True)
    inp = parity.prefill_inputs(T, H, E, R, False, "none", 0)
    b = moe.alloc_prefill_buffers(N, T, H, E, R)
    b.status.zero_()
    parity.upload_inputs(b, inp)
    idx = ms.random_topk(1, T, E, R, seed=1).reshape(T, R)
    idx[0, 0] = E
    idx[2, 1] = idx[2, 0]
    idx[3, 0] = -1
    b.topk_idx.copy_(torch.from_numpy(np.ascontiguousarray(idx, np.int32)))
    b.topk_w.fill_(0.5)
    moe.moe_prefill_dispatch(b.shape, b.x, None, b.topk_idx, b.slot_pos, b.expert_x, None,
                             b.expert_cnt, b.expert_off, b.expert_src, b.workspace)
    moe.moe_expert_stub(b.shape, 0, b.expert_x, None, b.expert_off, b.expert_y)
    moe.moe_prefill_combine(b.shape, b.expert_y, b.topk_idx, b.slot_pos, b.topk_w, b.partial, b.out)
    torch.cuda.synchronize()
    assert int(b.status.item()) == moe.MOE_EBADIDX
    sp = b.slot_pos.cpu().numpy()
    assert sp[0, 0] == -1 and sp[2, 1] == -1 and sp[3, 0] == -1
    assert int(b.expert_cnt.sum().item()) == T * R - 3


@pytest.mark.timeout(600)
def test_prefill_full_workload():
    c = ms.CONFIGS["qwen3_235b_prefill_ep"]
    print(f"\ncase prefill full {c.name}", flush=True)
    inp = parity.prefill_inputs(c.T, c.H, c.E, c.R, c.fp8, c.bias, c.seed)
    _, g = parity.gpu_run_prefill(c.N, c.T, c.H, c.E, c.R, c.fp8, inp)
    print("  gpu done", flush=True)
    o = parity.oracle_run_prefill(c.N, c.T, c.H, c.E, c.R, c.fp8, inp)
    print("  oracle done", flush=True)
    print(" ", parity.compare_prefill(g, o, c.N, c.T, c.H, c.E, c.R, c.fp8), flush=True)


def _sweep_case(seed):
    """A seeded random replicated-token configuration: ranks, experts per rank, slots, tokens,
    hidden size, payload and bias drawn together (ranks up to 33, slot counts up to several
    count chunks, hidden sizes that are not multiples of the 64-lane chunk groups)."""
    rng = np.random.default_rng(3000 + seed)
    N = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 33]))
    L = int(rng.integers(1, 9))
    E = N * L
    R = int(rng.integers(1, min(E, 9) + 1))
    T = int(rng.integers(1, 700))
    fp8 = bool(rng.random() < 0.3)
    H = int(rng.choice([512, 1024])) if fp8 else 8 * int(rng.integers(1, 97))
    bias = str(rng.choice(["none", "zipf"]))
    split = bool(rng.random() < 0.5)
    return N, T, H, E, R, fp8, bias, split


@pytest.mark.parametrize("seed", range(24))
def test_prefill_random_shape_sweep(seed):
    N, T, H, E, R, fp8, bias, split = _sweep_case(seed)
    case = (N, T, H, E, R, fp8, bias)
    print(f"\ncase prefill sweep {seed}: {_id(case)} split {split}", flush=True)
    inp = parity.prefill_inputs(T, H, E, R, fp8, bias, 10 + seed)
    _, g = parity.gpu_run_prefill(N, T, H, E, R, fp8, inp, split=split)
    o = parity.oracle_run_prefill(N, T, H, E, R, fp8, inp)
    parity.compare_prefill(g, o, N, T, H, E, R, fp8)
