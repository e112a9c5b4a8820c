"""The oracle's steps split over rank (token) chunks and run on several threads give exactly the
single-call results: the chunked forms only restrict each step's loops to a range of ranks, and
the ranges of one step write disjoint outputs.  This is what the threaded CPU baseline runs."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import moe_synth as ms
import oracle

# N, T, H, E, R, fp8, bias, tokens
CASES = [
    (2, 16, 256, 8, 2, False, "none", None),          # the tiny workload
    (5, 7, 8, 5, 1, False, "none", None),             # one expert per rank, one slot
    (8, 33, 64, 64, 8, False, "zipf", [0, 1, 33, 5, 17, 33, 2, 9]),   # token counts, an empty rank
    (4, 30, 512, 16, 4, True, "none", None),          # e4m3 rows with scales
    (16, 8, 32, 96, 8, False, "kimi", None),          # skewed onto rank 0
    (1, 20, 16, 7, 3, False, "none", None),           # one rank
]


def _single(c, inp):
    N, T, H, E, R, fp8, _, tok = c
    idx, w = oracle.route(inp["logits"], inp["bias"], R)
    sh = oracle.shape(N, T, H, E, R, fp8, tokens=tok)
    r = oracle.dispatch_send(sh, inp["x"], inp["x_scale"], idx.reshape(N, T * R))
    sh = oracle.packed_shape(N, T, H, E, R, fp8, np.diff(r["send_off"], axis=1).sum(axis=0), tok)
    r.update(oracle.net_dispatch(sh, r["send_off"], r["send_buf"], r["send_meta"]))
    r.update(oracle.dispatch_recv(sh, r["counts"], r["recv_off"], r["recv_buf"], r["recv_meta"]))
    y = oracle.expert(sh, 1, r["expert_x"], r["expert_scale"], r["expert_off"])
    for mode in (0, 1):
        c_ = oracle.combine(sh, mode, y, r["expert_rpos"], r["recv_off"], r["send_off"], r["send_pos"], w)
        r.update({f"{k}{mode}": v for k, v in c_.items()})
    r.update(topk_idx=idx, topk_w=w)
    return r, y


def _chunked(c, inp, y, pool, parts):
    N, T, H, E, R, fp8, _, tok = c
    idx, w = oracle.route_chunked(inp["logits"], inp["bias"], R, pool, parts)
    sh = oracle.shape(N, T, H, E, R, fp8, tokens=tok)
    r = oracle.dispatch_send_chunked(sh, inp["x"], inp["x_scale"], idx.reshape(N, T * R), pool, parts)
    sh = oracle.packed_shape(N, T, H, E, R, fp8, np.diff(r["send_off"], axis=1).sum(axis=0), tok)
    r.update(oracle.net_dispatch_chunked(sh, r["send_off"], r["send_buf"], r["send_meta"], pool, parts))
    r.update(oracle.dispatch_recv_chunked(sh, r["counts"], r["recv_off"], r["recv_buf"], r["recv_meta"],
                                          pool, parts))
    for mode in (0, 1):
        c_ = oracle.combine_chunked(sh, mode, y, r["expert_rpos"], r["recv_off"], r["send_off"],
                                    r["send_pos"], w, pool, parts)
        r.update({f"{k}{mode}": v for k, v in c_.items()})
    r.update(topk_idx=idx, topk_w=w)
    return r


@pytest.mark.parametrize("case", CASES, ids=lambda c: "N{}_T{}_H{}_E{}_R{}".format(*c[:5]))
def test_chunked_steps_equal_single_calls(case):
    N, T, H, E, R, fp8, bias, tok = case
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, seed=N + T)
    want, y = _single(case, inp)
    with ThreadPoolExecutor(max_workers=4) as pool:
        for parts in sorted({1, 2, 3, N, 2 * N}):
            for p in (pool, None):
                got = _chunked(case, inp, y, p, parts)
                for k, v in want.items():
                    if v is None:
                        assert got[k] is None, k
                        continue
                    assert np.array_equal(got[k], v), (k, parts, p is None)


def test_rank_chunks_cover_every_rank_once():
    for n in (1, 2, 7, 32, 64):
        for parts in (1, 3, 8, 16, 100):
            ch = oracle.rank_chunks(n, parts)
            assert ch[0][0] == 0 and ch[-1][1] == n and len(ch) <= parts
            assert all(a < b for a, b in ch) and all(ch[i][1] == ch[i + 1][0] for i in range(len(ch) - 1))
