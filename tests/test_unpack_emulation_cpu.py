"""CPU model of the unpack kernel's indexing (tests/unpack_emul.py) against the oracle, and the
two mistakes a several-rows-per-wave unpack can make, planted in the model.

A prototype in which each unpack wave resolved rows w, w + 4, ... (to reach 8 rows per block for
e4m3 rows) raised an illegal memory access on its first GPU test, the tiny workload, whose rows
take the 4-row block shape.  Its source was not kept, so the model reconstructs the design: with
the descriptor slot bounded by the block's row count, it stays in bounds and reproduces the
oracle's expert-major layout on every shape, 8 rows per block with 2 per wave included.  Without
that bound, two rows per wave on the 4-row shape write a descriptor past rows[4]; in LDS the rank
bases follow rows[], so the write overwrites them and the next wave's rank index runs past the
table, sending its reads and writes outside the buffers -- an illegal access on exactly that test.
The other candidate (descriptors left stale for rows past the call's total) cannot fire on the
tiny workload, whose grid holds no such row.
"""
import numpy as np
import pytest

import moe_synth as ms
import oracle
import unpack_emul as ue


def _setup(N, T, H, E, R, fp8, bias, seed=0):
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, seed)
    idx, _ = oracle.route(inp["logits"], inp["bias"], R)
    sh = oracle.shape(N, T, H, E, R, fp8)
    r = oracle.dispatch_send(sh, inp["x"], inp["x_scale"], idx.reshape(N, T * R))
    r.update(oracle.net_dispatch(sh, r["send_off"], r["send_buf"], r["send_meta"]))
    ref = oracle.dispatch_recv(sh, r["counts"], r["recv_off"], r["recv_buf"], r["recv_meta"])
    return sh, r, ref


def _model(case, rpb, u, rows_per_wave=1, check_slot=True, rb=0, rc=None, stride=None, stale=None,
           write_unresolved=True):
    N, T, H, E, R, fp8, bias = case
    sh, r, ref = _setup(*case)
    B = sh.B
    rc = rc or N
    D = dict(N=N, T=T, H=H, E=E, R=R, B=B, fp8=fp8, rb=rb, rc=rc)
    ex = np.zeros_like(ref["expert_x"])
    es = np.zeros_like(ref["expert_scale"]) if fp8 else None
    esrc = np.full((N, B), -1, np.int32)
    erp = np.full((N, B), -1, np.int32)
    st = ue.emulate_unpack(D, r["counts"], r["recv_off"], r["recv_buf"], r["recv_meta"], ex, es, esrc, erp,
                           rpb, u, rows_per_wave, check_slot, stride, stale, write_unresolved)
    for d in range(rb, rb + rc):
        n = r["recv_off"][d, N]
        assert np.array_equal(ex[d, :n], ref["expert_x"][d, :n]), d
        assert np.array_equal(esrc[d, :n], ref["expert_src"][d, :n]), d
        assert np.array_equal(erp[d, :n], ref["expert_rpos"][d, :n]), d
        if fp8:
            assert np.array_equal(es[d, :n], ref["expert_scale"][d, :n]), d
    return st


TINY = (2, 16, 256, 8, 2, False, "none")
FP8 = (4, 30, 512, 16, 4, True, "none")
RAGGED = (3, 37, 264, 9, 3, False, "none")     # 333 rows: the last 4-row block has 3 past the total
SKEW = (8, 20, 512, 64, 8, True, "zipf")


# (case, rows per block, chunks per thread): the launcher's shapes for these rows, and the 8-row
# several-rows-per-wave target for e4m3 rows
@pytest.mark.parametrize("case,rpb,u,rpw", [
    (TINY, 4, 1, 1), (FP8, 4, 8, 1), (RAGGED, 4, 1, 1), (SKEW, 4, 8, 1),
    (FP8, 8, 8, 2), (SKEW, 8, 8, 2), (RAGGED, 8, 1, 2)])
def test_model_matches_oracle(case, rpb, u, rpw):
    st = _model(case, rpb, u, rpw)
    assert st["overruns"] == 0


def test_model_matches_oracle_for_rank_ranges():
    # a call for one rank with a capped grid whose blocks stride over the rows
    for rb in range(3):
        _model(RAGGED, 4, 1, rb=rb, rc=1, stride=4)
    _model(SKEW, 8, 8, rows_per_wave=2, rb=5, rc=2, stride=3)


def test_planted_descriptor_overrun_breaks_the_tiny_workload():
    # two rows per wave on the 4-row shape, no bound on the descriptor slot
    with pytest.raises(ue.Violation, match="rank index .* past the"):
        _model(TINY, 4, 1, rows_per_wave=2, check_slot=False)
    # with the bound the same configuration is exact
    _model(TINY, 4, 1, rows_per_wave=2, check_slot=True)


def test_planted_stale_descriptors_need_rows_past_the_total():
    garbage = np.random.default_rng(0).integers(0, 2 ** 31, 4096)
    # the tiny workload's grid has no row past its total: stale descriptors are never read
    _model(TINY, 4, 1, stale=garbage, write_unresolved=False)
    # a grid with rows past the total reads them as addresses
    with pytest.raises(ue.Violation):
        _model(RAGGED, 4, 1, stale=garbage, write_unresolved=False)
