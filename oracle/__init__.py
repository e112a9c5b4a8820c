"""CPU oracle for MoE dispatch/combine -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The product path (``combine_moe_route_top_amd``) never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only builds it with gcc and
marshals numpy arrays through ctypes.  Each wrapper allocates its outputs and returns them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: every fp32 operation in oracle.c is one IEEE operation (no implicit FMA).
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (always when ``force``)."""
    stale = (not os.path.exists(_LIB)) or any(
        os.path.getmtime(p) > os.path.getmtime(_LIB) for p in (_SRC, _HDR))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """Load liboracle.so (building it if stale).  MOE_ORACLE_LIB names another build of
    oracle.c to load instead; the mutation tests use it to run the pins on planted mistakes."""
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_ORACLE_LIB")
        if not path:
            path = build()
        _lib = ctypes.CDLL(path)
        _lib.oracle_bf16_from_double.restype = ctypes.c_uint16
        _lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        _lib.oracle_bf16_to_double.restype = ctypes.c_double
        _lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        _lib.oracle_e4m3_to_double.restype = ctypes.c_double
        _lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        _lib.oracle_e4m3_from_float_sat.restype = ctypes.c_uint8
        _lib.oracle_e4m3_from_float_sat.argtypes = [ctypes.c_float]
        _lib.oracle_row_bytes.restype = ctypes.c_long
    return _lib


class Shape(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("E", ctypes.c_int), ("R", ctypes.c_int), ("fp8", ctypes.c_int),
                ("B", ctypes.c_long), ("rbase", ctypes.c_void_p), ("tokens", ctypes.c_void_p)]

    # With rbase set (an int64 array of N+1 row bases kept alive here), receive-side arrays are
    # packed: rank d owns rows rbase[d] .. rbase[d+1]-1 of one [rows][...] array.
    _rbase_arr = None
    # With tokens set (an int32 array of N token counts kept alive here), rank s dispatches only
    # its first tokens[s] tokens.
    _tokens_arr = None

    def set_tokens(self, tokens):
        if tokens is None:
            self.tokens, self._tokens_arr = None, None
        else:
            t = np.ascontiguousarray(tokens, np.int32)
            assert t.shape == (self.N,) and t.min() >= 0 and t.max() <= self.T
            self._tokens_arr = t
            self.tokens = t.ctypes.data
        return self

    def ntok(self, s) -> int:
        return self.T if self._tokens_arr is None else int(self._tokens_arr[s])

    def rows(self) -> int:
        return int(self._rbase_arr[-1]) if self._rbase_arr is not None else self.N * self.B

    def lead(self):
        """Leading dimensions of a receive-side array."""
        return (self.rows(),) if self._rbase_arr is not None else (self.N, self.B)

    def rank_rows(self, arr, d, n=None):
        """The first n receive-side rows of rank d (all of its rows if n is None)."""
        if self._rbase_arr is None:
            return arr[d] if n is None else arr[d, :n]
        b0, b1 = int(self._rbase_arr[d]), int(self._rbase_arr[d + 1])
        return arr[b0:b1] if n is None else arr[b0:b0 + n]


def packed_shape(N, T, H, E, R, fp8, rows_per_rank, tokens=None) -> Shape:
    """A shape whose receive-side arrays hold exactly rows_per_rank[d] rows for rank d."""
    rb = np.zeros(N + 1, np.int64)
    rb[1:] = np.cumsum(np.asarray(rows_per_rank, np.int64))
    sh = Shape(N, T, H, E, R, int(bool(fp8)), int(max(1, np.max(rows_per_rank))), rb.ctypes.data,
               None)
    sh._rbase_arr = rb
    return sh.set_tokens(tokens)


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def shape(N, T, H, E, R, fp8=False, B=None, tokens=None) -> Shape:
    if B is None:
        B = N * T * max(R, E // N)
    return Shape(N, T, H, E, R, int(bool(fp8)), B, None, None).set_tokens(tokens)


def row_bytes(sh: Shape) -> int:
    return int(lib().oracle_row_bytes(ctypes.byref(sh)))


def bf16_from_double(x: float) -> int:
    return int(lib().oracle_bf16_from_double(float(x)))


def bf16_to_double(b: int) -> float:
    return float(lib().oracle_bf16_to_double(int(b)))


def e4m3_to_double(b: int) -> float:
    return float(lib().oracle_e4m3_to_double(int(b)))


def e4m3_from_float_sat(v: float) -> int:
    return int(lib().oracle_e4m3_from_float_sat(float(v)))


def quantize_e4m3(x_bf16: np.ndarray):
    """bf16 bits uint16[..., H] -> (e4m3 codes uint8[..., H], scales f32[..., H/128])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    H = x.shape[-1]
    n = x.size // H
    q = np.empty(x.shape, np.uint8)
    sc = np.empty(x.shape[:-1] + (H // 128,), np.float32)
    lib().oracle_quantize_e4m3(ctypes.c_long(n), ctypes.c_int(H), _p(x), _p(q), _p(sc))
    return q, sc


def route(logits: np.ndarray, bias, R: int):
    """logits f32[n][E], bias f32[E] or None -> (idx i32[n][R], w f32[n][R])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    n, E = logits.shape
    idx = np.empty((n, R), np.int32)
    w = np.empty((n, R), np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib().oracle_route(ctypes.c_int(n), ctypes.c_int(E), ctypes.c_int(R), _p(logits), _p(b),
                       _p(idx), _p(w))
    return idx, w


def dispatch_send(sh: Shape, x: np.ndarray, x_scale, topk_idx: np.ndarray):
    """x: uint16[N][T][H] (bf16 bits) or uint8[N][T][H] (e4m3 codes); x_scale f32[N][T][H/128]."""
    N, T, E, R = sh.N, sh.T, sh.E, sh.R
    P = row_bytes(sh)
    x = np.ascontiguousarray(x)
    xs = None if not sh.fp8 else np.ascontiguousarray(x_scale, dtype=np.float32)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    counts = np.empty((N, E), np.int32)
    send_off = np.empty((N, N + 1), np.int32)
    send_pos = np.full((N, T * R), -1, np.int32)
    send_buf = np.zeros((N, T * R, P), np.uint8)
    send_meta = np.zeros((N, T * R, 2), np.int32)
    lib().oracle_dispatch_send(ctypes.byref(sh), _p(x), _p(xs), _p(idx), _p(counts), _p(send_off),
                               _p(send_pos), _p(send_buf), _p(send_meta))
    return dict(counts=counts, send_off=send_off, send_pos=send_pos, send_buf=send_buf,
                send_meta=send_meta)


def net_dispatch(sh: Shape, send_off, send_buf, send_meta):
    N = sh.N
    P = row_bytes(sh)
    recv_buf = np.zeros(sh.lead() + (P,), np.uint8)
    recv_meta = np.zeros(sh.lead() + (2,), np.int32)
    recv_off = np.empty((N, N + 1), np.int32)
    lib().oracle_net_dispatch(ctypes.byref(sh), _p(send_off), _p(send_buf), _p(send_meta),
                              _p(recv_buf), _p(recv_meta), _p(recv_off))
    return dict(recv_buf=recv_buf, recv_meta=recv_meta, recv_off=recv_off)


def dispatch_recv(sh: Shape, counts, recv_off, recv_buf, recv_meta):
    N, H = sh.N, sh.H
    L = sh.E // N
    lead = sh.lead()
    if sh.fp8:
        expert_x = np.zeros(lead + (H,), np.uint8)
        expert_scale = np.zeros(lead + (H // 128,), np.float32)
    else:
        expert_x = np.zeros(lead + (H,), np.uint16)
        expert_scale = None
    expert_cnt = np.empty((N, L), np.int32)
    expert_off = np.empty((N, L + 1), np.int32)
    expert_src = np.full(lead, -1, np.int32)
    expert_rpos = np.full(lead, -1, np.int32)
    lib().oracle_dispatch_recv(ctypes.byref(sh), _p(counts), _p(recv_off), _p(recv_buf),
                               _p(recv_meta), _p(expert_x), _p(expert_scale), _p(expert_cnt),
                               _p(expert_off), _p(expert_src), _p(expert_rpos))
    return dict(expert_x=expert_x, expert_scale=expert_scale, expert_cnt=expert_cnt,
                expert_off=expert_off, expert_src=expert_src, expert_rpos=expert_rpos)


def expert(sh: Shape, mode: int, expert_x, expert_scale, expert_off):
    y = np.zeros(sh.lead() + (sh.H,), np.uint16)
    lib().oracle_expert(ctypes.byref(sh), ctypes.c_int(mode), _p(np.ascontiguousarray(expert_x)),
                        _p(expert_scale), _p(expert_off), _p(y))
    return y


def combine(sh: Shape, mode: int, expert_y, expert_rpos, recv_off, send_off, send_pos, topk_w):
    N, H, T, R = sh.N, sh.H, sh.T, sh.R
    cs = np.zeros(sh.lead() + (H,), np.uint16)
    cr = np.zeros((N, T * R, H), np.uint16)
    out = np.zeros((N, T, H), np.uint16)   # rows of absent tokens stay zero (not written)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    lib().oracle_combine(ctypes.byref(sh), ctypes.c_int(mode), _p(expert_y), _p(expert_rpos),
                         _p(recv_off), _p(send_off), _p(send_pos), _p(w), _p(cs), _p(cr),
                         _p(out))
    return dict(cs_buf=cs, cr_buf=cr, out=out)


def combine_acc(sh: Shape, mode: int, expert_y, expert_src, expert_rpos, recv_off, send_off,
                topk_idx, send_pos, topk_w):
    """Combine with the sum taken on the sending side (one bf16 partial row per token and owner
    rank).  cs_buf/cr_buf start filled with bf16 3.0 (0x4040), which rows that hold no partial
    keep: a sum that reads such a row shows."""
    N, H, T, R = sh.N, sh.H, sh.T, sh.R
    cs = np.full(sh.lead() + (H,), 0x4040, np.uint16)
    cr = np.full((N, T * R, H), 0x4040, np.uint16)
    out = np.zeros((N, T, H), np.uint16)
    lib().oracle_combine_acc(ctypes.byref(sh), ctypes.c_int(mode),
                             _p(np.ascontiguousarray(expert_y, np.uint16)),
                             _p(np.ascontiguousarray(expert_src, np.int32)),
                             _p(np.ascontiguousarray(expert_rpos, np.int32)),
                             _p(np.ascontiguousarray(recv_off, np.int32)),
                             _p(np.ascontiguousarray(send_off, np.int32)),
                             _p(np.ascontiguousarray(topk_idx, np.int32)),
                             _p(np.ascontiguousarray(send_pos, np.int32)),
                             _p(np.ascontiguousarray(topk_w, np.float32)), _p(cs), _p(cr), _p(out))
    return dict(cs_buf=cs, cr_buf=cr, out=out)


def prefill_dispatch(sh: Shape, x: np.ndarray, x_scale, topk_idx: np.ndarray):
    """Replicated tokens: x uint16[T][H] (bf16 bits) or uint8[T][H] (e4m3), x_scale f32[T][H/128];
    topk_idx i32[T][R].  sh.B is the per-rank row stride of the receive-side arrays."""
    N, T, H, E, R = sh.N, sh.T, sh.H, sh.E, sh.R
    L = E // N
    x = np.ascontiguousarray(x)
    xs = None if not sh.fp8 else np.ascontiguousarray(x_scale, dtype=np.float32)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    slot_pos = np.full((T, R), -1, np.int32)
    expert_x = np.zeros((N, sh.B, H), np.uint8 if sh.fp8 else np.uint16)
    expert_scale = np.zeros((N, sh.B, H // 128), np.float32) if sh.fp8 else None
    expert_cnt = np.empty((N, L), np.int32)
    expert_off = np.empty((N, L + 1), np.int32)
    expert_src = np.full((N, sh.B), -1, np.int32)
    lib().oracle_prefill_dispatch(ctypes.byref(sh), _p(x), _p(xs), _p(idx), _p(slot_pos),
                                  _p(expert_x), _p(expert_scale), _p(expert_cnt), _p(expert_off),
                                  _p(expert_src))
    return dict(slot_pos=slot_pos, expert_x=expert_x, expert_scale=expert_scale,
                expert_cnt=expert_cnt, expert_off=expert_off, expert_src=expert_src)


def prefill_combine(sh: Shape, mode: int, expert_y, slot_pos, topk_idx, topk_w):
    N, T, H = sh.N, sh.T, sh.H
    partial = np.zeros((N, T, H), np.float32)
    out = np.zeros((T, H), np.uint16)
    lib().oracle_prefill_combine(ctypes.byref(sh), ctypes.c_int(mode),
                                 _p(np.ascontiguousarray(expert_y, np.uint16)),
                                 _p(np.ascontiguousarray(slot_pos, np.int32)),
                                 _p(np.ascontiguousarray(topk_idx, np.int32)),
                                 _p(np.ascontiguousarray(topk_w, np.float32)), _p(partial), _p(out))
    return dict(partial=partial, out=out)


def run_all(sh: Shape, inp: dict, expert_mode: int = 0, combine_mode: int = 0,
            tight: bool = False) -> dict:
    """The whole path on one input set (see moe_synth.make_inputs).

    With ``tight`` the receive-side arrays are packed: rank d gets exactly the rows it receives
    (keeps host memory small for the large, skewed workloads); ``res["shape"]`` is the shape
    actually used (see Shape.rank_rows)."""
    res = {}
    idx, w = route(inp["logits"], inp["bias"], sh.R)
    res["topk_idx"], res["topk_w"] = idx, w
    res.update(dispatch_send(sh, inp["x"], inp.get("x_scale"), idx.reshape(sh.N, sh.T * sh.R)))
    if tight:
        n = np.diff(res["send_off"], axis=1)          # n[s][d]
        sh = packed_shape(sh.N, sh.T, sh.H, sh.E, sh.R, sh.fp8, n.sum(axis=0), sh._tokens_arr)
    res["shape"] = sh
    res.update(net_dispatch(sh, res["send_off"], res["send_buf"], res["send_meta"]))
    res.update(dispatch_recv(sh, res["counts"], res["recv_off"], res["recv_buf"],
                             res["recv_meta"]))
    res["expert_y"] = expert(sh, expert_mode, res["expert_x"], res["expert_scale"],
                             res["expert_off"])
    res.update(combine(sh, combine_mode, res["expert_y"], res["expert_rpos"], res["recv_off"],
                       res["send_off"], res["send_pos"], w))
    return res


# ------------------------------------------------------------------ the steps over rank chunks

def rank_chunks(n: int, parts: int):
    """[r0, r1) ranges splitting 0..n into at most `parts` contiguous, non-empty chunks."""
    parts = max(1, min(int(parts), n))
    b = [n * i // parts for i in range(parts + 1)]
    return [(b[i], b[i + 1]) for i in range(parts) if b[i] < b[i + 1]]


def _over_chunks(pool, fn, n, parts):
    """fn(r0, r1) for every chunk, on the pool's threads (each call is one C call, during which
    ctypes releases the interpreter lock), all finished before returning."""
    chunks = rank_chunks(n, parts)
    if pool is None or len(chunks) == 1:
        for r0, r1 in chunks:
            fn(r0, r1)
        return
    for f in [pool.submit(fn, r0, r1) for r0, r1 in chunks]:
        f.result()


def route_chunked(logits, bias, R, pool, parts):
    """route() with the tokens split into chunks; the same outputs."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    n, E = logits.shape
    idx = np.empty((n, R), np.int32)
    w = np.empty((n, R), np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    _over_chunks(pool, lambda t0, t1: lib().oracle_route_tokens(
        ctypes.c_int(t0), ctypes.c_int(t1), ctypes.c_int(E), ctypes.c_int(R), _p(logits), _p(b),
        _p(idx), _p(w)), n, parts)
    return idx, w


def dispatch_send_chunked(sh: Shape, x, x_scale, topk_idx, pool, parts):
    N, T, E, R = sh.N, sh.T, sh.E, sh.R
    P = row_bytes(sh)
    x = np.ascontiguousarray(x)
    xs = None if not sh.fp8 else np.ascontiguousarray(x_scale, dtype=np.float32)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    counts = np.empty((N, E), np.int32)
    send_off = np.empty((N, N + 1), np.int32)
    send_pos = np.full((N, T * R), -1, np.int32)
    send_buf = np.zeros((N, T * R, P), np.uint8)
    send_meta = np.zeros((N, T * R, 2), np.int32)
    _over_chunks(pool, lambda r0, r1: lib().oracle_dispatch_send_ranks(
        ctypes.byref(sh), ctypes.c_int(r0), ctypes.c_int(r1), _p(x), _p(xs), _p(idx), _p(counts),
        _p(send_off), _p(send_pos), _p(send_buf), _p(send_meta)), N, parts)
    return dict(counts=counts, send_off=send_off, send_pos=send_pos, send_buf=send_buf,
                send_meta=send_meta)


def net_dispatch_chunked(sh: Shape, send_off, send_buf, send_meta, pool, parts):
    N = sh.N
    P = row_bytes(sh)
    recv_buf = np.zeros(sh.lead() + (P,), np.uint8)
    recv_meta = np.zeros(sh.lead() + (2,), np.int32)
    recv_off = np.empty((N, N + 1), np.int32)
    _over_chunks(pool, lambda r0, r1: lib().oracle_net_dispatch_ranks(
        ctypes.byref(sh), ctypes.c_int(r0), ctypes.c_int(r1), _p(send_off), _p(send_buf),
        _p(send_meta), _p(recv_buf), _p(recv_meta), _p(recv_off)), N, parts)
    return dict(recv_buf=recv_buf, recv_meta=recv_meta, recv_off=recv_off)


def dispatch_recv_chunked(sh: Shape, counts, recv_off, recv_buf, recv_meta, pool, parts):
    N, H = sh.N, sh.H
    L = sh.E // N
    lead = sh.lead()
    if sh.fp8:
        expert_x = np.zeros(lead + (H,), np.uint8)
        expert_scale = np.zeros(lead + (H // 128,), np.float32)
    else:
        expert_x = np.zeros(lead + (H,), np.uint16)
        expert_scale = None
    expert_cnt = np.empty((N, L), np.int32)
    expert_off = np.empty((N, L + 1), np.int32)
    expert_src = np.full(lead, -1, np.int32)
    expert_rpos = np.full(lead, -1, np.int32)
    _over_chunks(pool, lambda r0, r1: lib().oracle_dispatch_recv_ranks(
        ctypes.byref(sh), ctypes.c_int(r0), ctypes.c_int(r1), _p(counts), _p(recv_off),
        _p(recv_buf), _p(recv_meta), _p(expert_x), _p(expert_scale), _p(expert_cnt),
        _p(expert_off), _p(expert_src), _p(expert_rpos)), N, parts)
    return dict(expert_x=expert_x, expert_scale=expert_scale, expert_cnt=expert_cnt,
                expert_off=expert_off, expert_src=expert_src, expert_rpos=expert_rpos)


def combine_chunked(sh: Shape, mode: int, expert_y, expert_rpos, recv_off, send_off, send_pos,
                    topk_w, pool, parts):
    """combine() as its three steps, each over rank chunks: the shuffle (by destination), the
    network back (by source), the weighted sum (by source)."""
    N, H, T, R = sh.N, sh.H, sh.T, sh.R
    cs = np.zeros(sh.lead() + (H,), np.uint16)
    cr = np.zeros((N, T * R, H), np.uint16)
    out = np.zeros((N, T, H), np.uint16)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    y = np.ascontiguousarray(expert_y, np.uint16)
    _over_chunks(pool, lambda r0, r1: lib().oracle_combine_pack_ranks(
        ctypes.byref(sh), ctypes.c_int(r0), ctypes.c_int(r1), _p(y), _p(expert_rpos),
        _p(recv_off), _p(cs)), N, parts)
    _over_chunks(pool, lambda r0, r1: lib().oracle_combine_net_ranks(
        ctypes.byref(sh), ctypes.c_int(r0), ctypes.c_int(r1), _p(recv_off), _p(send_off), _p(cs),
        _p(cr)), N, parts)
    _over_chunks(pool, lambda r0, r1: lib().oracle_combine_sum_ranks(
        ctypes.byref(sh), ctypes.c_int(r0), ctypes.c_int(r1), ctypes.c_int(mode), _p(send_pos),
        _p(w), _p(cr), _p(out)), N, parts)
    return dict(cs_buf=cs, cr_buf=cr, out=out)
