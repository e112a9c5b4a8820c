"""Brute-force references for pinning the oracle (pure Python, small inputs only).

These are written from the definitions, not from the oracle: orders come from Python's stable
``sorted`` over explicit keys, weights from 60-digit ``decimal`` arithmetic, and rounding to
bf16 / fp32 from exact rationals and a table of every representable value.  None of this code
is shared with the oracle or the HIP path.
"""
from __future__ import annotations

import bisect
import decimal
import math
from fractions import Fraction

import numpy as np

# ------------------------------------------------------------------ exact rounding helpers


def _bf16_table():
    """All finite non-negative bf16 values as (Fraction, bits), sorted by value."""
    vals = []
    for bits in range(0x0000, 0x7F80):  # +0 .. largest finite
        f = np.array([bits << 16], np.uint32).view(np.float32)[0]
        vals.append((Fraction(float(f)), bits))
    return vals


_BF16 = None


def bf16_round_exact(x) -> int:
    """Nearest bf16 bit pattern to the rational x, ties to the even pattern; overflow -> inf."""
    global _BF16
    if _BF16 is None:
        t = _bf16_table()
        _BF16 = ([v for v, _ in t], [b for _, b in t])
    vals, bits = _BF16
    X = Fraction(x)
    sign = 0x8000 if X < 0 else 0
    a = abs(X)
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | bits[i]
    if i == len(vals):
        # beyond the largest finite value: rounds to inf once past max + half an ulp
        top, prev = vals[-1], vals[-2]
        half = (top - prev) / 2
        if a < top + half:
            return sign | bits[-1]
        if a == top + half:  # tie between max (odd pattern 0x7F7F) and inf (even): inf
            return sign | 0x7F80
        return sign | 0x7F80
    lo, hi = vals[i - 1], vals[i]
    if a - lo < hi - a:
        return sign | bits[i - 1]
    if hi - a < a - lo:
        return sign | bits[i]
    return sign | (bits[i - 1] if bits[i - 1] % 2 == 0 else bits[i])


def f32_round_exact(x) -> np.float32:
    """Nearest fp32 to the rational x, ties to even (no overflow handling needed here)."""
    X = Fraction(x)
    f = np.float32(float(X))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - X)
        key = (d, int(np.array([c], np.float32).view(np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def fma_f32_exact(a, b, c) -> np.float32:
    return f32_round_exact(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def bf16_bits_to_fraction(b: int) -> Fraction:
    f = np.array([int(b) << 16], np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def e4m3_table():
    """OCP E4M3 (exponent bias 7, 3 mantissa bits, no inf, S.1111.111 = NaN) -> Fraction."""
    out = {}
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            out[code] = None
            continue
        v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out[code] = -v if s else v
    return out


def e4m3_nearest(v) -> int:
    """The e4m3 code nearest to the rational v by search over every finite code, ties to the
    even code, magnitudes beyond 448 clamped to 448."""
    tab = e4m3_table()
    X = Fraction(float(v))
    sign = 0x80 if (X < 0 or (X == 0 and math.copysign(1.0, float(v)) < 0)) else 0
    a = min(abs(X), Fraction(448))
    best = None
    for code in range(0x7F):          # +0 .. 448
        d = abs(tab[code] - a)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return sign | best[1] if best[1] else sign


# ------------------------------------------------------------------ routing


def route(logits: np.ndarray, bias, R: int):
    """Top-R by (v desc, e asc) with v = fp32(logit + bias); weights = exact softmax (Decimal)."""
    n, E = logits.shape
    idx = np.zeros((n, R), np.int64)
    wx = []
    ctx = decimal.Context(prec=60)
    for t in range(n):
        v = logits[t].astype(np.float32)
        if bias is not None:
            v = (v + bias.astype(np.float32)).astype(np.float32)  # one IEEE fp32 add per element
        order = sorted(range(E), key=lambda e: (-float(v[e]), e))
        sel = order[:R]
        idx[t] = sel
        v0 = decimal.Decimal(float(v[sel[0]]))
        z = [ctx.exp(decimal.Decimal(float(v[e])) - v0) for e in sel]
        tot = sum(z, decimal.Decimal(0))
        wx.append([zz / tot for zz in z])
    return idx, wx


# ------------------------------------------------------------------ dispatch / combine


def dispatch(N, T, E, R, idx, tokens=None):
    """Sort-based layout of every (source, token, slot) entry.  With ``tokens``, source s has
    only its first tokens[s] tokens (the other slots get send_pos -1).

    Returns a dict with counts, send_off, send_pos, the send order per source, the receive
    order per destination, the expert-major order per destination and rank_e per entry."""
    L = E // N
    idx = np.asarray(idx).reshape(N, T, R)
    nt = [T] * N if tokens is None else [int(v) for v in tokens]
    counts = np.zeros((N, E), np.int64)
    send_off = np.zeros((N, N + 1), np.int64)
    send_pos = np.full((N, T * R), -1, np.int64)
    send_order = []
    rank_e = {}
    for s in range(N):
        ent = [(int(idx[s, t, k]) // L, t, k, int(idx[s, t, k])) for t in range(nt[s]) for k in range(R)]
        for (_, t, k, e) in ent:
            counts[s, e] += 1
        # rank among earlier entries of this source with the same expert
        for (_, t, k, e) in ent:
            rank_e[(s, t, k)] = sum(1 for (_, t2, k2, e2) in ent if e2 == e and (t2, k2) < (t, k))
        order = sorted(ent, key=lambda z: (z[0], z[1], z[2]))
        send_order.append([(t, k, e) for (_, t, k, e) in order])
        for pos, (d, t, k, e) in enumerate(order):
            send_pos[s, t * R + k] = pos
        for d in range(N):
            send_off[s, d + 1] = sum(1 for z in order if z[0] <= d)
    recv_order, expert_order = [], []
    for d in range(N):
        ent = [(s, t, k, int(idx[s, t, k])) for s in range(N) for t in range(nt[s]) for k in range(R)
               if int(idx[s, t, k]) // L == d]
        recv_order.append(sorted(ent, key=lambda z: (z[0], z[1], z[2])))
        expert_order.append(sorted(ent, key=lambda z: (z[3] - d * L, z[0], z[1], z[2])))
    return dict(counts=counts, send_off=send_off, send_pos=send_pos, send_order=send_order,
                recv_order=recv_order, expert_order=expert_order, rank_e=rank_e)


def prefill_layout(N, T, E, R, idx):
    """Replicated tokens: rank d's expert-major order is every (t, k) whose expert d owns,
    sorted by (local expert, t, k).  Returns the order per rank and each slot's position."""
    L = E // N
    idx = np.asarray(idx).reshape(T, R)
    order, pos = [], {}
    for d in range(N):
        ent = [(int(idx[t, k]) - d * L, t, k) for t in range(T) for k in range(R)
               if int(idx[t, k]) // L == d]
        ent = sorted(ent)
        order.append(ent)
        for q, (_, t, k) in enumerate(ent):
            pos[(t, k)] = q
    return order, pos


def combine_exact(N, T, R, E, y_of_entry, w):
    """out[s][t] = bf16(sum_k w[s,t,k] * y(s,t,k)) with the sum exact (Fractions).

    y_of_entry(s, t, k) -> list of bf16 bit patterns; w float32[N*T][R]."""
    out = []
    for s in range(N):
        rows = []
        for t in range(T):
            ys = [y_of_entry(s, t, k) for k in range(R)]
            H = len(ys[0])
            row = []
            for h in range(H):
                acc = Fraction(0)
                for k in range(R):
                    acc += Fraction(float(w[s * T + t, k])) * bf16_bits_to_fraction(ys[k][h])
                row.append(bf16_round_exact(acc))
            rows.append(row)
        out.append(rows)
    return np.array(out, np.uint16)


def combine_acc_exact(N, T, R, L, idx, y_of_entry, w, mode):
    """Combine with the sum on the sending side, from its definition: the token's slots grouped by
    owner rank e // L in the order of each owner's first slot; each group's partial is
    bf16(sum of w * y) (mode 0: exact sum; mode 1: fp32 fused multiply-adds in slot order, each
    exactly rounded); out = bf16(sum of the partials) (mode 0: exact; mode 1: fp32 additions in
    group order).  idx int32[N][T*R] (-1 never occurs here); returns (out, partials) with
    partials[(s, t, owner)] = bf16 bits per hidden position."""
    out = []
    partials = {}
    for s in range(N):
        rows = []
        for t in range(T):
            owners = []
            for k in range(R):
                d = int(idx[s, t * R + k]) // L
                if d not in owners:
                    owners.append(d)
            ys = {k: y_of_entry(s, t, k) for k in range(R)}
            H = len(ys[0])
            for d in owners:
                ks = [k for k in range(R) if int(idx[s, t * R + k]) // L == d]
                prow = []
                for h in range(H):
                    if mode == 0:
                        acc = Fraction(0)
                        for k in ks:
                            acc += Fraction(float(w[s * T + t, k])) * bf16_bits_to_fraction(ys[k][h])
                        prow.append(bf16_round_exact(acc))
                    else:
                        acc = np.float32(0)
                        for k in ks:
                            acc = fma_f32_exact(w[s * T + t, k], float(bf16_bits_to_fraction(ys[k][h])), acc)
                        prow.append(bf16_round_exact(Fraction(float(acc))))
                partials[(s, t, d)] = prow
            row = []
            for h in range(H):
                if mode == 0:
                    acc = sum((bf16_bits_to_fraction(partials[(s, t, d)][h]) for d in owners), Fraction(0))
                    row.append(bf16_round_exact(acc))
                else:
                    acc = np.float32(0)
                    for d in owners:
                        acc = f32_round_exact(Fraction(float(acc)) + bf16_bits_to_fraction(partials[(s, t, d)][h]))
                    row.append(bf16_round_exact(Fraction(float(acc))))
            rows.append(row)
        out.append(rows)
    return np.array(out, np.uint16), partials
