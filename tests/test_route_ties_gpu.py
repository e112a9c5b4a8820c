"""Router tie-break on the GPU: scores that tie, through the whole path, against the oracle.

The selection order is descending fp32 (logit + bias), ties to the lower expert id, -0 == +0
(the pages only say the router sorts the scores keeping the indices: [DSK] MoE Router).  Random
N(0,1) scores almost never tie, so these inputs are built to: every score of a row equal, scores
on a few levels, zeros of both signs on top, and scores that only tie once the fp32 bias add
rounds them.  The shapes select every lane-group width of the router kernel (16, 32 and 64 lanes
per token, one to sixteen experts per lane), so equal scores sit in one lane, across lanes of a
16-lane row and across rows.
"""
import numpy as np
import pytest

import moe_synth as ms
import parity

# N, T, H, E, R, the router's lanes per token for this call size
SHAPES = [
    (2, 2048, 64, 8, 2, 16),       # 4096 tokens: 16 lanes, one expert per lane
    (32, 128, 64, 256, 8, 16),     # DeepSeek-V3's router shape: 16 lanes, 16 experts per lane
    (16, 128, 64, 256, 8, 32),     # 2048 tokens: widened to 32 lanes, 8 experts per lane
    (64, 64, 64, 384, 8, 32),      # Kimi-K2's expert count: 32 lanes, 12 experts per lane
    (8, 64, 64, 1024, 8, 64),      # 1024 experts: 64 lanes, 16 experts per lane
    (4, 16, 64, 8, 8, 64),         # R = E: the whole row in order
]


def _ids(c):
    return "N{}_T{}_E{}_R{}_G{}".format(c[0], c[1], c[3], c[4], c[5])


def _boundary_ties(logits, bias, R):
    """Rows whose R-th and (R+1)-th largest fp32 scores are equal, or whose selected scores hold
    a repeated value (a property of the input only)."""
    v = logits if bias is None else (logits + bias[None, :]).astype(np.float32)
    s = -np.sort(-v, axis=1)
    rep = np.any(s[:, 1:R] == s[:, :R - 1], axis=1) if R > 1 else np.zeros(len(v), bool)
    if R < v.shape[1]:
        rep |= s[:, R - 1] == s[:, R]
    return rep


@pytest.mark.parametrize("kind", ms.TIE_KINDS)
def test_tie_inputs_tie(kind):
    # the generated scores do tie at or inside the selection (CPU, input property only)
    for N, T, H, E, R, _ in SHAPES:
        logits, bias = ms.tie_logits(kind, N * T, E, seed=N + E)
        frac = _boundary_ties(logits, bias, R).mean()
        if kind == "signed_zero" and R == E:
            continue  # R = E selects every score; the zeros still tie among themselves
        assert frac > 0.2, (kind, N, E, R, frac)
    if kind == "signed_zero":
        logits, _ = ms.tie_logits(kind, 4096, 64, seed=1)
        z = logits == 0
        assert np.signbit(logits[z]).any() and (~np.signbit(logits[z])).any()


@pytest.mark.gpu
@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
@pytest.mark.parametrize("kind", ms.TIE_KINDS)
def test_route_ties_full_path(kind, shape):
    N, T, H, E, R, G = shape
    print(f"\ncase ties {kind} {_ids(shape)}", flush=True)
    inp = ms.make_inputs(N, T, H, E, R, False, "none", 0)
    inp["logits"], inp["bias"] = ms.tie_logits(kind, N * T, E, seed=N + E)
    _, g = parity.gpu_run(N, T, H, E, R, False, inp, expert_mode=1)
    o = parity.oracle_run(N, T, H, E, R, False, inp, expert_mode=1)
    parity.compare(g, o, N, T, H, E, R, False)
    if kind == "equal":
        # every row ties everywhere: experts 0..R-1 in order, equal weights
        assert np.array_equal(g["topk_idx"].reshape(N * T, R),
                              np.broadcast_to(np.arange(R, dtype=np.int32), (N * T, R)))
