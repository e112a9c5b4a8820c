"""Pins of the CPU oracle against things other than itself (CPU only).

Pins used: library routines for the number formats (torch's bf16 / e4m3 conversions), exact
rational rounding over a table of every bf16 value, 60-digit decimal softmax, a sort-based
brute-force layout of every (source, token, slot) entry, closed forms of combine for identity
and tagged experts, special cases that reduce to a library sort, and the load arithmetic the
pages print (tests/golden/pages_arithmetic.json).
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import brute
import moe_synth as ms
import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_arithmetic.json")))


def f32_ulp(x: float) -> float:
    x = abs(float(np.float32(x)))
    return float(np.spacing(np.float32(x)))


# ------------------------------------------------------------------ number formats


def test_bf16_from_float_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    # exact ties: low 16 bits 0x8000 with even and odd kept halves
    u = rng.integers(0, 2**31, 4000, dtype=np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).astype(np.uint32).view(np.float32)
    ties = ties[np.isfinite(ties)]
    specials = np.array([0.0, -0.0, 1e-40, -1e-40, 3.3e38, 3.39e38, -3.39e38, 1.0, 65504.0],
                        np.float32)
    allv = np.concatenate([x, ties, specials])
    want = torch.from_numpy(allv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(v)) for v in allv], np.uint16)
    assert np.array_equal(got, want)


def test_bf16_from_double_exact_rounding():
    rnd = random.Random(5)
    vals = []
    for _ in range(3000):
        m = rnd.uniform(-4, 4)
        vals.append(m * 2.0 ** rnd.randint(-140, 127))
    # doubles that sit exactly on a bf16 midpoint, and just off it
    for _ in range(500):
        b = rnd.randint(0x0001, 0x7F7E)
        lo = brute.bf16_bits_to_fraction(b)
        hi = brute.bf16_bits_to_fraction(b + 1)
        mid = (lo + hi) / 2
        vals += [float(mid), float(mid) * (1 + 2**-40), float(mid) * (1 - 2**-40)]
    vals += [3.3961e38, 3.4e38, 1e39, 2.0**-133, 2.0**-134, 1.5 * 2.0**-134, 2.0**-135]
    for v in vals:
        assert oracle.bf16_from_double(v) == brute.bf16_round_exact(Fraction(v)), v
        assert oracle.bf16_from_double(-v) == brute.bf16_round_exact(-Fraction(v)), -v


def test_bf16_to_double_roundtrip():
    for b in list(range(0, 0x7F81, 97)) + [0x8000 | b for b in range(0, 0x7F81, 101)]:
        assert Fraction(oracle.bf16_to_double(b)) == (
            brute.bf16_bits_to_fraction(b) if b & 0x8000 == 0 else -brute.bf16_bits_to_fraction(b & 0x7FFF))


def test_e4m3_decode_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib_vals = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    table = brute.e4m3_table()
    for c in range(256):
        got = oracle.e4m3_to_double(c)
        if table[c] is None:
            assert math.isnan(got) and math.isnan(lib_vals[c])
        else:
            assert Fraction(got) == table[c] == Fraction(float(lib_vals[c])), c
    assert oracle.e4m3_to_double(0x7E) == 448.0


# ------------------------------------------------------------------ routing


@pytest.mark.parametrize("E,R,bias", [(8, 2, "none"), (16, 4, "zipf"), (64, 8, "none"),
                                      (384, 8, "kimi"), (12, 12, "none"), (5, 1, "zipf")])
def test_route_brute(E, R, bias):
    rng = np.random.default_rng(E * 31 + R)
    logits = rng.standard_normal((40, E), dtype=np.float32)
    b = ms.make_bias(bias, E)
    idx, w = oracle.route(logits, b, R)
    bidx, bw = brute.route(logits, b, R)
    assert np.array_equal(idx, bidx)
    for t in range(logits.shape[0]):
        for k in range(R):
            exact = Fraction(str(bw[t][k]))
            err = abs(Fraction(float(w[t, k])) - exact)
            assert err <= Fraction(f32_ulp(w[t, k])) / 2 * Fraction(1000001, 1000000), (t, k)
    # weights are non-increasing along slots and sum to one up to fp32 rounding
    assert np.all(np.diff(w.astype(np.float64), axis=1) <= 0)
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=R * 2**-24)


def test_route_special_cases():
    # R = 1: the weight is exactly one
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((50, 32), dtype=np.float32)
    _, w = oracle.route(lg, None, 1)
    assert np.all(w == 1.0)
    # all-equal scores: ties go to the lower expert id; weights are 1/R
    lg = np.full((3, 10), 0.25, np.float32)
    idx, w = oracle.route(lg, None, 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (3, 1)))
    assert np.all(w == np.float32(0.25))
    # -0 and +0 compare equal: lower id wins
    lg = np.full((1, 4), -1.0, np.float32)
    lg[0, 3] = 0.0
    lg[0, 1] = -0.0
    idx, _ = oracle.route(lg, None, 2)
    assert list(idx[0]) == [1, 3]
    # R = E: a full softmax over all experts, in descending order
    lg = rng.standard_normal((4, 6), dtype=np.float32)
    idx, w = oracle.route(lg, None, 6)
    for t in range(4):
        assert list(idx[t]) == sorted(range(6), key=lambda e: (-lg[t, e], e))
        p = np.exp(lg[t].astype(np.float64) - lg[t].max())
        p /= p.sum()
        assert np.allclose(w[t], p[idx[t]], rtol=2**-22)
    # the bias enters before selection: +16 on experts 0..5 always wins (Kimi-shaped input)
    lg = rng.standard_normal((64, 384), dtype=np.float32)
    idx, _ = oracle.route(lg, ms.make_bias("kimi", 384), 8)
    assert np.all(np.sort(idx[:, :6], axis=1) == np.arange(6))


# ------------------------------------------------------------------ dispatch layout

SMALL = [  # N, T, H, E, R, fp8
    (1, 7, 8, 5, 2, False), (2, 16, 16, 8, 2, False), (3, 5, 8, 9, 3, False),
    (4, 9, 512, 8, 3, True), (4, 6, 8, 4, 1, False), (2, 3, 8, 6, 6, False),
    (8, 4, 16, 16, 4, False), (3, 11, 512, 12, 5, True), (5, 3, 8, 20, 8, False),
]


def run_small(N, T, H, E, R, fp8, seed=0, bias="none", idx=None):
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, seed)
    sh = oracle.shape(N, T, H, E, R, fp8)
    if idx is None:
        idx, w = oracle.route(inp["logits"], inp["bias"], R)
    else:
        w = np.full((N * T, R), 1.0 / R, np.float32)
    idx = idx.reshape(N, T * R)
    res = oracle.dispatch_send(sh, inp["x"], inp["x_scale"], idx)
    res.update(oracle.net_dispatch(sh, res["send_off"], res["send_buf"], res["send_meta"]))
    res.update(oracle.dispatch_recv(sh, res["counts"], res["recv_off"], res["recv_buf"],
                                    res["recv_meta"]))
    res["w"], res["idx"], res["inp"], res["sh"] = w, idx, inp, sh
    return res


def token_row_bytes(inp, s, t, fp8):
    if fp8:
        return inp["x"][s, t].tobytes() + inp["x_scale"][s, t].tobytes()
    return inp["x"][s, t].tobytes()


@pytest.mark.parametrize("case", SMALL)
@pytest.mark.parametrize("seed", [0, 1])
def test_dispatch_matches_brute_force(case, seed):
    N, T, H, E, R, fp8 = case
    res = run_small(*case, seed=seed)
    check_layout_brute(res, case, brute.dispatch(N, T, E, R, res["idx"]))


def check_layout_brute(res, case, bf):
    N, T, H, E, R, fp8 = case
    inp = res["inp"]
    L = E // N
    assert np.array_equal(res["counts"], bf["counts"])
    assert np.array_equal(res["send_off"], bf["send_off"])
    assert np.array_equal(res["send_pos"], bf["send_pos"])
    TR = T * R
    for s in range(N):
        for pos, (t, k, e) in enumerate(bf["send_order"][s]):
            assert res["send_buf"][s, pos].tobytes() == token_row_bytes(inp, s, t, fp8)
            assert res["send_meta"][s, pos, 0] == e * TR + t * R + k
            assert res["send_meta"][s, pos, 1] == bf["rank_e"][(s, t, k)]
    B = res["sh"].B
    for d in range(N):
        order = bf["recv_order"][d]
        assert res["recv_off"][d, N] == len(order)
        for s in range(N):
            assert res["recv_off"][d, s] == sum(1 for z in order if z[0] < s)
        for r, (s, t, k, e) in enumerate(order):
            assert res["recv_buf"][d, r].tobytes() == token_row_bytes(inp, s, t, fp8)
            assert res["recv_meta"][d, r, 0] == e * TR + t * R + k
        eorder = bf["expert_order"][d]
        for j in range(L):
            assert res["expert_cnt"][d, j] == sum(1 for z in eorder if z[3] == d * L + j)
        assert res["expert_off"][d, 0] == 0 and res["expert_off"][d, L] == len(eorder)
        for q, (s, t, k, e) in enumerate(eorder):
            assert res["expert_src"][d, q] == s * TR + t * R + k
            assert order[res["expert_rpos"][d, q]] == (s, t, k, e)
            if fp8:
                assert res["expert_x"][d, q].tobytes() == inp["x"][s, t].tobytes()
                assert res["expert_scale"][d, q].tobytes() == inp["x_scale"][s, t].tobytes()
            else:
                assert res["expert_x"][d, q].tobytes() == inp["x"][s, t].tobytes()
        assert len(eorder) <= N * T * min(R, L) <= B


@pytest.mark.parametrize("case", [SMALL[1], SMALL[3], SMALL[6], SMALL[8]])
def test_variable_tokens_brute(case):
    # rank s dispatches only its first tokens[s] tokens: the layout is the brute-force layout
    # of those tokens alone, absent slots get send_pos -1, and combine leaves absent rows alone
    N, T, H, E, R, fp8 = case
    rng = np.random.default_rng(21)
    tokens = rng.integers(0, T + 1, N)
    tokens[0], tokens[-1] = 0, T
    inp = ms.make_inputs(N, T, H, E, R, fp8, "none", 4)
    sh = oracle.shape(N, T, H, E, R, fp8, tokens=tokens)
    idx, w = oracle.route(inp["logits"], inp["bias"], R)
    idx = idx.reshape(N, T * R)
    res = oracle.dispatch_send(sh, inp["x"], inp["x_scale"], idx)
    res.update(oracle.net_dispatch(sh, res["send_off"], res["send_buf"], res["send_meta"]))
    res.update(oracle.dispatch_recv(sh, res["counts"], res["recv_off"], res["recv_buf"],
                                    res["recv_meta"]))
    res["w"], res["idx"], res["inp"], res["sh"] = w, idx, inp, sh
    bf = brute.dispatch(N, T, E, R, idx, tokens)
    check_layout_brute(res, case, bf)
    assert res["counts"].sum() == int(tokens.sum()) * R
    _, out = _combine(res, 0, 0)
    for s in range(N):
        assert not out["out"][s, tokens[s]:].any(), "rows of absent tokens were written"
        for t in range(tokens[s]):
            y = _dequant_bf16(inp, s, t, fp8)
            sw = sum(Fraction(float(w[s * T + t, k])) for k in range(R))
            want = [brute.bf16_round_exact(brute.bf16_bits_to_fraction(int(v) & 0x7FFF) * sw *
                                           (-1 if int(v) & 0x8000 else 1)) for v in y]
            assert list(out["out"][s, t]) == want


def test_all_tokens_present_equals_fixed_count():
    case = SMALL[6]
    N, T, H, E, R, fp8 = case
    a = run_small(*case, seed=3)
    sh = oracle.shape(N, T, H, E, R, fp8, tokens=np.full(N, T))
    b = oracle.dispatch_send(sh, a["inp"]["x"], a["inp"]["x_scale"], a["idx"])
    for k in ("counts", "send_off", "send_pos", "send_buf", "send_meta"):
        assert np.array_equal(a[k], b[k]), k


# ------------------------------------------------------------------ fp8 block quantisation


def _e4m3_probe_values():
    """fp32 values at every e4m3 value, at the midpoints between neighbours and one fp32 step
    either side of each midpoint, beyond 448, and random over the range; both signs."""
    tab = brute.e4m3_table()
    pos = sorted(float(tab[c]) for c in range(0x7F))
    vals = []
    for a, b in zip(pos, pos[1:] + [480.0]):
        m = np.float32((a + b) / 2)   # exact: neighbours have at most 4 significant bits
        vals += [a, m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    vals += [470.0, 1e6]
    rng = np.random.default_rng(5)
    vals += list(rng.uniform(0, 448, 2000))
    vals += list(np.exp(rng.uniform(np.log(1e-5), np.log(448), 2000)))
    v = np.array(vals, np.float32)
    return np.concatenate([v, -v])


def test_e4m3_encode_matches_torch():
    # torch's float8_e4m3fn conversion is round-to-nearest-even (it has no saturation: clamp first)
    v = _e4m3_probe_values()
    mine = np.array([oracle.e4m3_from_float_sat(x) for x in v], np.uint8)
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(mine[i]), int(ref[i])) for i in bad[:5]]


def test_e4m3_encode_brute_nearest():
    v = _e4m3_probe_values()
    pick = np.concatenate([np.arange(0, 4 * 127 + 2), np.arange(4 * 127 + 2, v.size, 37)])
    for i in pick:
        assert oracle.e4m3_from_float_sat(v[i]) == brute.e4m3_nearest(v[i]), float(v[i])


def _spacing_e4m3(a: Fraction) -> Fraction:
    """Distance between adjacent e4m3 values around the magnitude a (<= 448)."""
    if a < Fraction(1, 64):
        return Fraction(1, 512)
    e = 0
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    while Fraction(2) ** e > a:
        e -= 1
    return Fraction(2) ** (e - 3)


@pytest.mark.parametrize("scale_exp", [0, -24, 30])
def test_quantize_blocks(scale_exp):
    rng = np.random.default_rng(100 + scale_exp)
    xf = (rng.standard_normal((6, 512)) * 2.0 ** scale_exp).astype(np.float32)
    xf[1, 128:256] = 0.0                                   # an all-zero block
    xf[2, 256:384] = -np.abs(xf[2, 256:384])               # largest magnitude negative
    xf[3, 0:128] = xf[3, 0:128] * (2.0 ** -12)             # subnormal-range codes in a block
    xf[3, 5] = 3.0 * 2.0 ** scale_exp
    xb = ms.to_bf16_bits(xf)
    xv = ms.bf16_bits_to_f32(xb)
    q, sc = oracle.quantize_e4m3(xb)
    tab = brute.e4m3_table()
    for n in range(6):
        for b in range(4):
            blk = xv[n, b * 128:(b + 1) * 128]
            qb = q[n, b * 128:(b + 1) * 128]
            amax = float(np.abs(blk).max())
            if amax == 0.0:
                assert sc[n, b] == 1.0 and not qb.any()
                continue
            # the scale is amax / 448 to within one fp32 rounding
            assert abs(Fraction(float(sc[n, b])) * 448 - Fraction(amax)) <= Fraction(amax) / 2 ** 23
            # the largest magnitude lands on +-448
            i = int(np.argmax(np.abs(blk)))
            assert qb[i] & 0x7F == 0x7E and (qb[i] >> 7) == int(blk[i] < 0)
            # every code is within half an e4m3 step of x / scale (plus the quotient's rounding)
            S = Fraction(float(sc[n, b]))
            for h in range(128):
                x = Fraction(float(blk[h]))
                v = x / S
                err = abs(tab[int(qb[h])] - v)
                assert err <= _spacing_e4m3(min(abs(v), Fraction(448))) / 2 + abs(v) / 2 ** 23, (n, b, h)
                assert (int(qb[h]) >> 7) == int(blk[h] < 0) or qb[h] & 0x7F == 0
    # an independent implementation (numpy division and torch's conversion) agrees bit for bit
    q2, sc2 = ms.quantize_e4m3(xv)
    assert np.array_equal(sc, sc2) and np.array_equal(q, q2)


# ------------------------------------------------------------------ prefill (replicated tokens)

PREFILL = [  # N, T, H, E, R, fp8
    (2, 9, 16, 8, 2, False), (4, 13, 8, 16, 4, False), (3, 7, 512, 12, 3, True),
    (1, 10, 8, 6, 3, False), (8, 5, 8, 16, 8, False),
]


def run_prefill(N, T, H, E, R, fp8, seed=0, bias="none"):
    inp = ms.make_inputs(1, T, H, E, R, fp8, bias, seed)      # one replicated token set
    idx, w = oracle.route(inp["logits"], inp["bias"], R)
    B = T * min(R, E // N)
    sh = oracle.shape(N, T, H, E, R, fp8, B=B)
    x = inp["x"].reshape(T, H)
    xs = None if not fp8 else inp["x_scale"].reshape(T, H // 128)
    res = oracle.prefill_dispatch(sh, x, xs, idx)
    res.update(idx=idx, w=w, x=x, xs=xs, sh=sh)
    return res


@pytest.mark.parametrize("case", PREFILL)
def test_prefill_dispatch_brute(case):
    N, T, H, E, R, fp8 = case
    res = run_prefill(*case, seed=3)
    order, pos = brute.prefill_layout(N, T, E, R, res["idx"])
    L = E // N
    for (t, k), q in pos.items():
        assert res["slot_pos"][t, k] == q
    assert sum(len(o) for o in order) == T * R
    for d in range(N):
        assert res["expert_off"][d, 0] == 0 and res["expert_off"][d, L] == len(order[d])
        for j in range(L):
            assert res["expert_cnt"][d, j] == sum(1 for z in order[d] if z[0] == j)
            assert res["expert_off"][d, j + 1] - res["expert_off"][d, j] == res["expert_cnt"][d, j]
        for q, (j, t, k) in enumerate(order[d]):
            assert res["expert_src"][d, q] == t * R + k
            assert res["expert_x"][d, q].tobytes() == res["x"][t].tobytes()
            if fp8:
                assert res["expert_scale"][d, q].tobytes() == res["xs"][t].tobytes()
        assert len(order[d]) <= T * min(R, L)


def test_prefill_single_rank_equals_decode_layout():
    # with one rank, replicated-input dispatch and the decode path's receive side agree
    N, T, H, E, R = 1, 12, 16, 9, 3
    res = run_prefill(N, T, H, E, R, False, seed=5)
    dec = run_small(N, T, H, E, R, False, seed=5)
    n = int(dec["expert_off"][0, -1])
    assert np.array_equal(res["expert_off"], dec["expert_off"])
    assert np.array_equal(res["expert_src"][0, :n], dec["expert_src"][0, :n])
    assert np.array_equal(res["expert_x"][0, :n], dec["expert_x"][0, :n])


@pytest.mark.parametrize("case", PREFILL)
def test_prefill_combine_identity_closed_form(case):
    # identity experts: out = bf16(x * sum_k w_k) whichever rank each slot lives on
    N, T, H, E, R, fp8 = case
    res = run_prefill(*case, seed=4)
    sh = res["sh"]
    y = oracle.expert(sh, 0, res["expert_x"], res["expert_scale"], res["expert_off"])
    c = oracle.prefill_combine(sh, 0, y, res["slot_pos"], res["idx"], res["w"])
    inp = {"x": res["x"][None], "x_scale": None if not fp8 else res["xs"][None]}
    for t in range(T):
        yv = _dequant_bf16(inp, 0, t, fp8)
        sw = sum(Fraction(float(res["w"][t, k])) for k in range(R))
        want = [brute.bf16_round_exact(brute.bf16_bits_to_fraction(int(v) & 0x7FFF) * sw *
                                       (-1 if int(v) & 0x8000 else 1)) for v in yv]
        assert list(c["out"][t]) == want


@pytest.mark.parametrize("case", PREFILL[:2] + PREFILL[4:])
def test_prefill_combine_fp32_steps_brute(case):
    # mode 1 (fp32 partials per rank in slot order, then an fp32 sum over ranks in order) against
    # exact-rational emulation of each fp32 operation, on random mixed-sign expert outputs
    N, T, H, E, R, fp8 = case
    res = run_prefill(*case, seed=6)
    sh = res["sh"]
    L = E // N
    y = ms.random_y(N, sh.B, H, seed=8)
    c = oracle.prefill_combine(sh, 1, y, res["slot_pos"], res["idx"], res["w"])
    for t in range(T):
        for h in range(H):
            parts = []
            for d in range(N):
                acc = np.float32(0.0)
                for k in range(R):
                    e = int(res["idx"][t, k])
                    if e // L != d:
                        continue
                    yv = brute.bf16_bits_to_fraction(int(y[d, res["slot_pos"][t, k], h]))
                    acc = brute.fma_f32_exact(res["w"][t, k], yv, acc)
                assert c["partial"][d, t, h] == acc
                parts.append(acc)
            s_ = np.float32(0.0)
            for p_ in parts:
                s_ = brute.f32_round_exact(Fraction(float(s_)) + Fraction(float(p_)))
            assert c["out"][t, h] == brute.bf16_round_exact(Fraction(float(s_)))


def test_prefill_allreduce_rank_order():
    # partials 2^28, -2^28 and 0.25 on ranks 0, 1, 2: summed in rank order the big ones cancel
    # first and 0.25 survives (the exact result); any other order absorbs 0.25 into 2^28 in fp32
    N, T, H, E, R = 3, 1, 8, 3, 3
    sh = oracle.shape(N, T, H, E, R, False, B=1)
    idx = np.array([[0, 1, 2]], np.int32)
    w = np.full((1, 3), 0.25, np.float32)
    x = np.zeros((T, H), np.uint16)
    res = oracle.prefill_dispatch(sh, x, None, idx)
    assert res["slot_pos"].tolist() == [[0, 0, 0]]
    y = np.zeros((N, 1, H), np.uint16)
    y[0, 0, :] = oracle.bf16_from_double(2.0 ** 30)
    y[1, 0, :] = oracle.bf16_from_double(-2.0 ** 30)
    y[2, 0, :] = oracle.bf16_from_double(1.0)
    quarter = oracle.bf16_from_double(0.25)
    for mode in (0, 1):
        c = oracle.prefill_combine(sh, mode, y, res["slot_pos"], idx, w)
        assert np.all(c["out"] == quarter), mode
    c = oracle.prefill_combine(sh, 1, y, res["slot_pos"], idx, w)
    assert c["partial"][:, 0, 0].tolist() == [2.0 ** 28, -2.0 ** 28, 0.25]


@pytest.mark.parametrize("case", [PREFILL[1], PREFILL[2]])
def test_prefill_combine_tagged_closed_form(case):
    # tagged experts: out = bf16(sum_k w_k * bf16(x * c_{e_k})): each slot's weight meets the row
    # of that slot's expert on that slot's rank
    N, T, H, E, R, fp8 = case
    res = run_prefill(*case, seed=7)
    sh = res["sh"]
    y = oracle.expert(sh, 1, res["expert_x"], res["expert_scale"], res["expert_off"])
    c = oracle.prefill_combine(sh, 0, y, res["slot_pos"], res["idx"], res["w"])
    tab = brute.e4m3_table()
    for t in range(T):
        for h in range(0, H, max(1, H // 16)):
            if fp8:
                xv = tab[int(res["x"][t, h])] * Fraction(float(res["xs"][t, h // 128]))
            else:
                b_ = int(res["x"][t, h])
                xv = brute.bf16_bits_to_fraction(b_ & 0x7FFF) * (-1 if b_ & 0x8000 else 1)
            acc = Fraction(0)
            for k in range(R):
                e = int(res["idx"][t, k])
                yk = brute.bf16_round_exact(xv * Fraction(64 + e % 64, 64))
                acc += Fraction(float(res["w"][t, k])) * brute.bf16_bits_to_fraction(yk & 0x7FFF) * \
                    (-1 if yk & 0x8000 else 1)
            assert c["out"][t, h] == brute.bf16_round_exact(acc), (t, h)


def test_dispatch_invariants_at_scale():
    # DeepSeek-V3-shaped routing with a tiny payload: invariants the method fixes at any size
    N, T, H, E, R = 32, 128, 8, 256, 8
    res = run_small(N, T, H, E, R, False, bias="zipf")
    assert np.all(res["counts"].sum(1) == T * R)                 # counts per source sum to T*R
    assert res["counts"].sum() == N * T * R
    assert np.all(res["send_off"][:, N] == T * R)
    assert np.all(np.diff(res["send_off"], axis=1) >= 0)
    for s in range(N):                                         # send_pos is a permutation
        assert np.array_equal(np.sort(res["send_pos"][s]), np.arange(T * R))
    tot = res["recv_off"][:, N]
    assert tot.sum() == N * T * R
    assert np.all(tot <= N * T * min(R, E // N))
    # every (s, t, k) appears exactly once in the expert-major tensors across ranks
    src = np.concatenate([res["expert_src"][d, :tot[d]] + d * 0 for d in range(N)])
    assert np.array_equal(np.sort(src), np.arange(N * T * R))
    # meta's per-expert rank equals the expert-major offset arithmetic
    L = E // N
    B = res["sh"].B
    for d in range(N):
        for r in range(tot[d]):
            m0, m1 = res["recv_meta"][d, r]
            e = m0 // (T * R)
            s = np.searchsorted(res["recv_off"][d], r, side="right") - 1
            q = res["expert_off"][d, e - d * L] + res["counts"][:s, e].sum() + m1
            assert res["expert_rpos"][d, q] == r


def test_single_rank_is_stable_counting_sort():
    N, T, E, R = 1, 50, 7, 3
    res = run_small(N, T, 8, E, R, False, seed=4)
    e_flat = res["idx"].reshape(-1)
    order = np.argsort(e_flat, kind="stable")  # library stable sort by expert id
    tot = res["recv_off"][0, 1]
    assert np.array_equal(res["expert_src"][0, :tot], order)
    assert np.array_equal(res["expert_cnt"][0], np.bincount(e_flat, minlength=E))


def test_one_expert_per_rank_one_slot_is_all_to_all():
    # L = 1, R = 1: a personalised all-to-all; rank d receives, source by source, the tokens
    # whose expert is d, in token order
    N, T = 4, 9
    rng = np.random.default_rng(2)
    idx = rng.integers(0, N, (N, T, 1)).astype(np.int32)
    res = run_small(N, T, 8, N, 1, False, idx=idx)
    for d in range(N):
        want = [s * T + t for s in range(N) for t in range(T) if idx[s, t, 0] == d]
        tot = res["recv_off"][d, N]
        assert list(res["expert_src"][d, :tot]) == want


def test_duplicate_expert_in_token_is_rejected():
    # The oracle's contract is R distinct experts per token; a duplicate is a contract breach.
    import subprocess
    import sys
    code = ("import numpy as np, oracle, moe_synth as ms\n"
            "inp = ms.make_inputs(1, 2, 8, 4, 2)\n"
            "sh = oracle.shape(1, 2, 8, 4, 2)\n"
            "idx = np.array([[1, 1, 0, 2]], np.int32)\n"
            "oracle.dispatch_send(sh, inp['x'], None, idx)\n")
    p = subprocess.run([sys.executable, "-c", code], cwd=os.path.dirname(os.path.dirname(
        os.path.abspath(__file__))), capture_output=True)
    assert p.returncode != 0


# ------------------------------------------------------------------ combine


def _combine(res, mode_expert, mode_combine, y=None):
    sh = res["sh"]
    if y is None:
        y = oracle.expert(sh, mode_expert, res["expert_x"], res["expert_scale"], res["expert_off"])
    out = oracle.combine(sh, mode_combine, y, res["expert_rpos"], res["recv_off"], res["send_off"],
                         res["send_pos"], res["w"])
    return y, out


def _dispatched_exact(inp, s, t, fp8):
    """The dispatched value of token (s, t) as exact rationals (bf16 value, or e4m3 * scale)."""
    if not fp8:
        return [brute.bf16_bits_to_fraction(int(v) & 0x7FFF) * (-1 if int(v) & 0x8000 else 1)
                for v in inp["x"][s, t]]
    tab = brute.e4m3_table()
    H = inp["x"].shape[-1]
    return [tab[int(inp["x"][s, t, h])] * Fraction(float(inp["x_scale"][s, t, h // 128]))
            for h in range(H)]


def _dequant_bf16(inp, s, t, fp8):
    """The identity expert's output for token (s, t): bf16 bits of the dispatched value."""
    if not fp8:
        return inp["x"][s, t].astype(np.int64)
    tab = brute.e4m3_table()
    H = inp["x"].shape[-1]
    return np.array([brute.bf16_round_exact(tab[int(inp["x"][s, t, h])] *
                                            Fraction(float(inp["x_scale"][s, t, h // 128])))
                     for h in range(H)], np.int64)


@pytest.mark.parametrize("case", [SMALL[1], SMALL[2], SMALL[3], SMALL[6]])
def test_identity_combine_closed_form(case):
    # identity experts: out = bf16(y * sum_k w_k), y the dispatched value of the token
    N, T, H, E, R, fp8 = case
    res = run_small(*case, seed=9)
    _, out = _combine(res, 0, 0)
    for s in range(N):
        for t in range(T):
            y = _dequant_bf16(res["inp"], s, t, fp8)
            sw = sum(Fraction(float(res["w"][s * T + t, k])) for k in range(R))
            want = [brute.bf16_round_exact(brute.bf16_bits_to_fraction(int(v) & 0x7FFF) * sw *
                                           (-1 if int(v) & 0x8000 else 1)) for v in y]
            assert list(out["out"][s, t]) == want


@pytest.mark.parametrize("case", [SMALL[1], SMALL[3], SMALL[7], SMALL[8]])
def test_tagged_combine_closed_form(case):
    # tagged experts scale by c_e = (64 + e % 64) / 64: out = bf16(y * sum_k w_k c_{e_k}),
    # which pins that each slot's weight meets the row of that slot's expert
    N, T, H, E, R, fp8 = case
    res = run_small(*case, seed=11)
    _, out = _combine(res, 1, 0)
    for s in range(N):
        for t in range(T):
            y = _dispatched_exact(res["inp"], s, t, fp8)
            for h in range(H):
                yv = y[h]
                acc = Fraction(0)
                for k in range(R):
                    e = int(res["idx"][s, t * R + k])
                    # the tagged expert rounds its exact product to bf16 once
                    tagged = brute.bf16_round_exact(yv * Fraction(64 + e % 64, 64))
                    acc += Fraction(float(res["w"][s * T + t, k])) * (
                        brute.bf16_bits_to_fraction(tagged & 0x7FFF) * (-1 if tagged & 0x8000 else 1))
                assert out["out"][s, t, h] == brute.bf16_round_exact(acc)


@pytest.mark.parametrize("case", [SMALL[2], SMALL[4], SMALL[6]])
def test_random_expert_outputs_brute(case):
    # arbitrary expert outputs: out[s][t] = bf16(exact sum_k w_k * y[row of (s, t, k)]), the
    # row found by the brute-force expert-major order; mode 1 = exact fp32 fma chain
    N, T, H, E, R, fp8 = case
    res = run_small(*case, seed=13)
    sh = res["sh"]
    y = ms.random_y(N, sh.B, H, seed=3)
    bf = brute.dispatch(N, T, E, R, res["idx"])
    where = {}
    for d in range(N):
        for q, (s, t, k, e) in enumerate(bf["expert_order"][d]):
            where[(s, t, k)] = (d, q)

    def y_of(s, t, k):
        d, q = where[(s, t, k)]
        return [int(v) for v in y[d, q]]

    _, out0 = _combine(res, None, 0, y=y)
    want = brute.combine_exact(N, T, R, E, y_of, res["w"])
    assert np.array_equal(out0["out"], want)
    _, out1 = _combine(res, None, 1, y=y)
    for s in range(N):
        for t in range(T):
            ys = [y_of(s, t, k) for k in range(R)]
            for h in range(H):
                acc = np.float32(0)
                for k in range(R):
                    acc = brute.fma_f32_exact(res["w"][s * T + t, k],
                                              float(brute.bf16_bits_to_fraction(ys[k][h] & 0x7FFF)) *
                                              (-1 if ys[k][h] & 0x8000 else 1), acc)
                assert out1["out"][s, t, h] == brute.bf16_round_exact(Fraction(float(acc)))


# ------------------------------------------------------------------ random small configurations


@pytest.mark.parametrize("seed", range(16))
def test_random_small_configurations_brute(seed):
    # seeded random tiny shapes (ranks, experts per rank, slots, tokens, bias): the whole layout
    # against the brute-force sort, both combines against their exact-rational definitions
    rng = np.random.default_rng(3000 + seed)
    N = int(rng.integers(1, 7))
    L = int(rng.integers(1, 5))
    E = N * L
    R = int(rng.integers(1, min(E, 5) + 1))
    T = int(rng.integers(1, 10))
    H = int(rng.choice([8, 16]))
    bias = str(rng.choice(["none", "zipf"]))
    case = (N, T, H, E, R, False)
    res = run_small(*case, seed=seed, bias=bias)
    bf = brute.dispatch(N, T, E, R, res["idx"])
    check_layout_brute(res, case, bf)
    y = ms.random_y(N, res["sh"].B, H, seed=seed)
    _, y_of = _y_lookup(res, N, T, E, R, y)
    _, out0 = _combine(res, None, 0, y=y)
    assert np.array_equal(out0["out"], brute.combine_exact(N, T, R, E, y_of, res["w"]))
    for mode in (0, 1):
        want, _ = brute.combine_acc_exact(N, T, R, L, res["idx"], y_of, res["w"], mode)
        assert np.array_equal(_combine_acc(res, y, mode)["out"], want), mode


# ------------------------------------------------------------------ combine, sum on the sending side


def _combine_acc(res, y, mode):
    return oracle.combine_acc(res["sh"], mode, y, res["expert_src"], res["expert_rpos"],
                              res["recv_off"], res["send_off"], res["idx"], res["send_pos"], res["w"])


def _y_lookup(res, N, T, E, R, y):
    bf = brute.dispatch(N, T, E, R, res["idx"])
    where = {}
    for d in range(N):
        for q, (s, t, k, e) in enumerate(bf["expert_order"][d]):
            where[(s, t, k)] = (d, q)

    def y_of(s, t, k):
        d, q = where[(s, t, k)]
        return [int(v) for v in y[d, q]]
    return bf, y_of


# shapes where a token's slots share owner ranks (L = 4, 3, 2, 2, 4)
ACC = [SMALL[1], SMALL[2], SMALL[3], SMALL[6], SMALL[8]]


@pytest.mark.parametrize("case", ACC)
def test_combine_acc_brute(case):
    # arbitrary expert outputs: every token's partial per owner rank and the final sum equal the
    # definition worked out with exact rationals; the partial sits at the receive position of the
    # token's first row at that rank and at the send position of its first slot owned there
    N, T, H, E, R, fp8 = case
    L = E // N
    res = run_small(*case, seed=17)
    y = ms.random_y(N, res["sh"].B, H, seed=5)
    bf, y_of = _y_lookup(res, N, T, E, R, y)
    for mode in (0, 1):
        o = _combine_acc(res, y, mode)
        want, parts = brute.combine_acc_exact(N, T, R, L, res["idx"], y_of, res["w"], mode)
        assert np.array_equal(o["out"], want), mode
        for (s, t, d), prow in parts.items():
            k0 = min(k for k in range(R) if int(res["idx"][s, t * R + k]) // L == d)
            assert list(o["cr_buf"][s, res["send_pos"][s, t * R + k0]]) == prow, (mode, s, t, d)
            r0 = bf["recv_order"][d].index((s, t, k0, int(res["idx"][s, t * R + k0])))
            assert list(o["cs_buf"][d, r0]) == prow, (mode, s, t, d)


@pytest.mark.parametrize("case", [SMALL[4], (3, 6, 16, 9, 1, False)])
def test_combine_acc_one_slot_equals_combine(case):
    # R = 1: one row per token, the partial is bf16(w * y) and the final sum adds nothing to it,
    # so both modes equal the receive-side combine bit for bit
    N, T, H, E, R, fp8 = case
    res = run_small(*case, seed=19)
    y = ms.random_y(N, res["sh"].B, H, seed=6)
    for mode in (0, 1):
        _, ref = _combine(res, None, mode, y=y)
        assert np.array_equal(_combine_acc(res, y, mode)["out"], ref["out"]), mode


@pytest.mark.parametrize("case", [SMALL[0], (1, 9, 16, 12, 6, False)])
def test_combine_acc_one_rank_equals_combine(case):
    # N = 1: every slot has the same owner, one partial per token holds the whole weighted sum,
    # rounded once; the final sum of one bf16 value is exact, so the result equals the
    # receive-side combine in both modes
    N, T, H, E, R, fp8 = case
    res = run_small(*case, seed=21)
    y = ms.random_y(N, res["sh"].B, H, seed=7)
    for mode in (0, 1):
        _, ref = _combine(res, None, mode, y=y)
        assert np.array_equal(_combine_acc(res, y, mode)["out"], ref["out"]), mode


@pytest.mark.parametrize("case", [SMALL[1], SMALL[3], SMALL[8]])
def test_combine_acc_identity_error_bound(case):
    # identity experts: every contribution of a token has the sign of its value, so each bf16
    # rounding (one per partial, one at the end) adds at most 2^-8 relative error:
    # |out - y * sum_k w_k| <= (2^-8 + 2^-8 + 2^-16) * |y * sum_k w_k| (plus fp32 terms in mode 1)
    N, T, H, E, R, fp8 = case
    res = run_small(*case, seed=23)
    y = oracle.expert(res["sh"], 0, res["expert_x"], res["expert_scale"], res["expert_off"])
    for mode in (0, 1):
        out = _combine_acc(res, y, mode)["out"]
        for s in range(N):
            for t in range(T):
                yv = _dequant_bf16(res["inp"], s, t, fp8)
                sw = sum(Fraction(float(res["w"][s * T + t, k])) for k in range(R))
                for h in range(H):
                    exact = brute.bf16_bits_to_fraction(int(yv[h])) * sw
                    got = brute.bf16_bits_to_fraction(int(out[s, t, h]))
                    assert abs(got - exact) <= abs(exact) * (Fraction(2, 2**8) + Fraction(1, 2**15)), \
                        (mode, s, t, h)


# ------------------------------------------------------------------ the pages' arithmetic


def test_pages_two_tokens_reach_at_most_16_experts():
    g = GOLDEN["two_tokens_reach_16_experts"]
    rng = np.random.default_rng(0)
    for _ in range(20):
        lg = rng.standard_normal((g["tokens"], g["E"]), dtype=np.float32)
        idx, _ = oracle.route(lg, None, g["R"])
        assert g["R"] <= len(set(idx.reshape(-1).tolist())) <= g["max_distinct_experts"]
    lg = np.zeros((2, g["E"]), np.float32)
    lg[0, :8] = 5.0
    lg[1, 8:16] = 5.0
    idx, _ = oracle.route(lg, None, g["R"])
    assert len(set(idx.reshape(-1).tolist())) == g["max_distinct_experts"]


def test_pages_groupgemm_mean_tokens_per_expert():
    g = GOLDEN["groupgemm_tokens_per_expert_ep128"]
    N, T, E, R = g["N"], g["T"], g["E"], g["R"]
    assert E // N == GOLDEN["experts_per_gpu_ep128"]["experts_per_rank"]
    inp = ms.make_inputs(N, T, 8, E, R, seed=0)
    sh = oracle.shape(N, T, 8, E, R)
    res = oracle.run_all(sh, inp, tight=True)
    assert res["expert_cnt"].shape == (N, 2)
    assert res["expert_cnt"].sum() / E == g["mean_tokens_per_expert"]


def test_pages_qwen_prefill_mean_tokens_per_expert():
    g = GOLDEN["qwen_prefill_tokens_per_expert"]
    N = 4
    T = g["tokens"] // N
    inp = ms.make_inputs(N, T, 8, g["E"], g["R"], seed=0)
    res = oracle.run_all(oracle.shape(N, T, 8, g["E"], g["R"]), inp, tight=True)
    assert res["expert_cnt"].sum() / g["E"] == g["mean_tokens_per_expert"]


@pytest.mark.parametrize("name", ["tiny", "mixtral_8x7b_decode", "deepseek_v3_decode",
                                  "qwen3_235b_prefill", "kimi_k2_worst"])
def test_pages_receive_bound(name):
    c = ms.CONFIGS[name]
    inp = ms.make_inputs(c.N, c.T, 8 if not c.fp8 else 512, c.E, c.R, c.fp8, c.bias, c.seed)
    idx, _ = oracle.route(inp["logits"], inp["bias"], c.R)
    sh = oracle.shape(c.N, c.T, 8 if not c.fp8 else 512, c.E, c.R, c.fp8)
    res = oracle.dispatch_send(sh, inp["x"], inp["x_scale"], idx.reshape(c.N, -1))
    recv = np.diff(res["send_off"], axis=1).sum(axis=0)
    assert recv.max() <= c.N * c.T * min(c.R, c.L) <= c.N * c.T * max(c.R, c.L) == c.B
    if name == "kimi_k2_worst":
        assert recv[0] == c.N * c.T * 6 == 49152


def test_pages_intra_node_share():
    g = GOLDEN["intra_node_share"]
    for N, share in g["cases"]:
        T, E, R = 128, 256, 8
        idx = ms.random_topk(N, T, E, R, seed=N)
        sh = oracle.shape(N, T, 8, E, R)
        inp = ms.make_inputs(N, T, 8, E, R, seed=1)
        res = oracle.dispatch_send(sh, inp["x"], None, idx.reshape(N, -1))
        n = np.diff(res["send_off"], axis=1)
        node = np.arange(N) // g["gpus_per_node"]
        intra = sum(n[s, d] for s in range(N) for d in range(N) if node[s] == node[d])
        assert abs(intra / n.sum() - share) < 0.02
