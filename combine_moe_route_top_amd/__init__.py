"""Python binding of libmoe (MoE expert-parallel dispatch and combine on MI355X).

Argument marshalling only: every function passes tensor data pointers and the current HIP
stream to the C ABI declared in include/moe.h, whose names it keeps.  Every step of the path
runs in the HIP kernels of libmoe.so; there is no fallback.  Importing this package fails
loudly if libmoe.so has not been built (python -m combine_moe_route_top_amd.build).

PyTorch provides device memory and streams.  torch is imported before libmoe.so is loaded so
that the library binds to the HIP runtime torch already loaded (same SONAME).
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch  # noqa: F401  (must precede the CDLL load: shared HIP runtime)

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB names another build of the same sources (e.g. one compiled with different launch-shape
# constants); default: the in-tree libmoe.so.
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m combine_moe_route_top_amd.build` "
        "(there is no fallback implementation)")

_lib = ctypes.CDLL(LIB_PATH)

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP, MOE_EBADIDX, MOE_ENOSCRATCH = 0, -1, -2, -3, -5, -6
MOE_STATIC_SCRATCH_BYTES = 4 << 20
MOE_BF16, MOE_FP8_E4M3, MOE_BF16_TO_FP8 = 0, 1, 2
MOE_LAYOUT_DECODE, MOE_LAYOUT_PREFILL = 0, 1


class moe_shape(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("E", ctypes.c_int32), ("R", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rank_begin", ctypes.c_int32), ("rank_count", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("status", ctypes.c_void_p),
                ("tokens", ctypes.c_void_p), ("layout", ctypes.c_int32)]


_SIZE_FIELDS = ["capacity", "row_bytes", "logits", "bias", "topk_idx", "topk_w", "x", "x_scale",
                "counts", "send_off", "send_pos", "send_buf", "send_meta", "recv_buf",
                "recv_meta", "recv_off", "expert_x", "expert_scale", "expert_cnt", "expert_off",
                "expert_src", "expert_rpos", "expert_y", "cs_buf", "cr_buf", "out", "workspace",
                "slot_pos", "partial"]


class moe_sizes_t(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in _SIZE_FIELDS]


_vp = ctypes.c_void_p
_SIGS = {
    "moe_sizes": [ctypes.POINTER(moe_shape), ctypes.POINTER(moe_sizes_t)],
    "moe_route": [ctypes.POINTER(moe_shape), _vp, _vp, _vp, _vp, _vp],
    "moe_dispatch_send": [ctypes.POINTER(moe_shape)] + [_vp] * 10,
    "moe_dispatch_send_noalloc": [ctypes.POINTER(moe_shape)] + [_vp] * 9,
    "moe_net_dispatch": [ctypes.POINTER(moe_shape)] + [_vp] * 7,
    "moe_dispatch_recv": [ctypes.POINTER(moe_shape)] + [_vp] * 11,
    "moe_combine": [ctypes.POINTER(moe_shape)] + [_vp] * 10,
    "moe_combine_send": [ctypes.POINTER(moe_shape)] + [_vp] * 7,
    "moe_combine_recv": [ctypes.POINTER(moe_shape)] + [_vp] * 5,
    "moe_combine_acc": [ctypes.POINTER(moe_shape)] + [_vp] * 13,
    "moe_combine_acc_send": [ctypes.POINTER(moe_shape)] + [_vp] * 10,
    "moe_combine_acc_recv": [ctypes.POINTER(moe_shape)] + [_vp] * 5,
    "moe_expert_stub": [ctypes.POINTER(moe_shape), ctypes.c_int32] + [_vp] * 5,
    "moe_prefill_dispatch": [ctypes.POINTER(moe_shape)] + [_vp] * 11,
    "moe_prefill_combine_local": [ctypes.POINTER(moe_shape)] + [_vp] * 6,
    "moe_prefill_allreduce": [ctypes.POINTER(moe_shape)] + [_vp] * 3,
    "moe_prefill_combine": [ctypes.POINTER(moe_shape)] + [_vp] * 7,
    "moe_stream_copy": [_vp, _vp, ctypes.c_int64, _vp],
    "moe_strerror": [ctypes.c_int],
    "moe_abi_version": [],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_char_p if _name == "moe_strerror" else ctypes.c_int


def header_functions() -> list:
    """Names of the functions include/moe.h declares."""
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(moe_\w+)\s*\(", src, re.M)))


class MoeError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {code} ({moe_strerror(code)})")
        self.code = code


def moe_strerror(code: int) -> str:
    return _lib.moe_strerror(int(code)).decode()


def moe_abi_version() -> int:
    return int(_lib.moe_abi_version())


def moe_stream_copy(src, dst, nbytes, stream=None):
    _check("moe_stream_copy", _lib.moe_stream_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)))


def _ptr(t):
    """A device address: None, an int (a raw device pointer), or a contiguous GPU tensor.  Host
    tensors and strided views are refused here: the kernels would read host addresses or assume
    the wrong layout."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libmoe takes device memory: got a tensor on " + str(t.device))
    if not t.is_contiguous():
        raise ValueError("libmoe takes dense row-major buffers: got a strided view")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(name, rc):
    if rc != MOE_OK:
        raise MoeError(name, rc)


def make_shape(N, T, H, E, R, fp8=False, capacity=0, status=None, rank_begin=0,
               rank_count=0, quant=False, tokens=None, prefill=False) -> moe_shape:
    """quant: bf16 tokens quantised to e4m3 rows by the send pack (MOE_BF16_TO_FP8);
    tokens: a device int32[N] tensor of per-rank token counts, or None;
    prefill: the replicated-token layout (MOE_LAYOUT_PREFILL)."""
    dtype = MOE_BF16_TO_FP8 if quant else (MOE_FP8_E4M3 if fp8 else MOE_BF16)
    return moe_shape(N, T, H, E, R, dtype, rank_begin, rank_count, capacity, _ptr(status),
                     _ptr(tokens), MOE_LAYOUT_PREFILL if prefill else MOE_LAYOUT_DECODE)


def for_ranks(shape: moe_shape, rank_begin: int, rank_count: int) -> moe_shape:
    """The same shape restricted to ranks [rank_begin, rank_begin + rank_count)."""
    return moe_shape(shape.N, shape.T, shape.H, shape.E, shape.R, shape.dtype, rank_begin,
                     rank_count, shape.capacity, shape.status, shape.tokens, shape.layout)


def moe_sizes(shape: moe_shape) -> dict:
    out = moe_sizes_t()
    _check("moe_sizes", _lib.moe_sizes(ctypes.byref(shape), ctypes.byref(out)))
    return {f: int(getattr(out, f)) for f in _SIZE_FIELDS}


def moe_route(shape, logits, bias, topk_idx, topk_w, stream=None):
    _check("moe_route", _lib.moe_route(ctypes.byref(shape), _ptr(logits), _ptr(bias),
                                       _ptr(topk_idx), _ptr(topk_w), _stream(stream)))


def moe_dispatch_send(shape, x, x_scale, topk_idx, counts, send_off, send_pos, send_buf,
                      send_meta, workspace, stream=None):
    _check("moe_dispatch_send", _lib.moe_dispatch_send(
        ctypes.byref(shape), _ptr(x), _ptr(x_scale), _ptr(topk_idx), _ptr(counts),
        _ptr(send_off), _ptr(send_pos), _ptr(send_buf), _ptr(send_meta), _ptr(workspace),
        _stream(stream)))


def moe_dispatch_send_noalloc(shape, x, x_scale, topk_idx, counts, send_off, send_pos, send_buf,
                              send_meta, stream=None):
    _check("moe_dispatch_send_noalloc", _lib.moe_dispatch_send_noalloc(
        ctypes.byref(shape), _ptr(x), _ptr(x_scale), _ptr(topk_idx), _ptr(counts), _ptr(send_off),
        _ptr(send_pos), _ptr(send_buf), _ptr(send_meta), _stream(stream)))


def moe_net_dispatch(shape, send_off, send_buf, send_meta, recv_buf, recv_meta, recv_off,
                     stream=None):
    _check("moe_net_dispatch", _lib.moe_net_dispatch(
        ctypes.byref(shape), _ptr(send_off), _ptr(send_buf), _ptr(send_meta), _ptr(recv_buf),
        _ptr(recv_meta), _ptr(recv_off), _stream(stream)))


def moe_dispatch_recv(shape, counts, recv_off, recv_buf, recv_meta, expert_x, expert_scale,
                      expert_cnt, expert_off, expert_src, expert_rpos, stream=None):
    _check("moe_dispatch_recv", _lib.moe_dispatch_recv(
        ctypes.byref(shape), _ptr(counts), _ptr(recv_off), _ptr(recv_buf), _ptr(recv_meta),
        _ptr(expert_x), _ptr(expert_scale), _ptr(expert_cnt), _ptr(expert_off),
        _ptr(expert_src), _ptr(expert_rpos), _stream(stream)))


def moe_combine(shape, expert_y, expert_rpos, recv_off, send_off, send_pos, topk_w, cs_buf,
                cr_buf, out, stream=None):
    _check("moe_combine", _lib.moe_combine(
        ctypes.byref(shape), _ptr(expert_y), _ptr(expert_rpos), _ptr(recv_off), _ptr(send_off),
        _ptr(send_pos), _ptr(topk_w), _ptr(cs_buf), _ptr(cr_buf), _ptr(out), _stream(stream)))


def moe_combine_send(shape, expert_y, expert_rpos, recv_off, send_off, cs_buf, cr_buf,
                     stream=None):
    _check("moe_combine_send", _lib.moe_combine_send(
        ctypes.byref(shape), _ptr(expert_y), _ptr(expert_rpos), _ptr(recv_off), _ptr(send_off),
        _ptr(cs_buf), _ptr(cr_buf), _stream(stream)))


def moe_combine_recv(shape, cr_buf, send_pos, topk_w, out, stream=None):
    _check("moe_combine_recv", _lib.moe_combine_recv(
        ctypes.byref(shape), _ptr(cr_buf), _ptr(send_pos), _ptr(topk_w), _ptr(out),
        _stream(stream)))


def moe_combine_acc(shape, expert_y, recv_meta, counts, recv_off, expert_off, send_off, topk_w,
                    topk_idx, send_pos, cs_buf, cr_buf, out, stream=None):
    _check("moe_combine_acc", _lib.moe_combine_acc(
        ctypes.byref(shape), _ptr(expert_y), _ptr(recv_meta), _ptr(counts), _ptr(recv_off),
        _ptr(expert_off), _ptr(send_off), _ptr(topk_w), _ptr(topk_idx), _ptr(send_pos),
        _ptr(cs_buf), _ptr(cr_buf), _ptr(out), _stream(stream)))


def moe_combine_acc_send(shape, expert_y, recv_meta, counts, recv_off, expert_off, send_off, topk_w,
                         cs_buf, cr_buf, stream=None):
    _check("moe_combine_acc_send", _lib.moe_combine_acc_send(
        ctypes.byref(shape), _ptr(expert_y), _ptr(recv_meta), _ptr(counts), _ptr(recv_off),
        _ptr(expert_off), _ptr(send_off), _ptr(topk_w), _ptr(cs_buf), _ptr(cr_buf),
        _stream(stream)))


def moe_combine_acc_recv(shape, cr_buf, topk_idx, send_pos, out, stream=None):
    _check("moe_combine_acc_recv", _lib.moe_combine_acc_recv(
        ctypes.byref(shape), _ptr(cr_buf), _ptr(topk_idx), _ptr(send_pos), _ptr(out),
        _stream(stream)))


def moe_expert_stub(shape, mode, expert_x, expert_scale, expert_off, expert_y, stream=None):
    _check("moe_expert_stub", _lib.moe_expert_stub(
        ctypes.byref(shape), int(mode), _ptr(expert_x), _ptr(expert_scale), _ptr(expert_off),
        _ptr(expert_y), _stream(stream)))


def moe_prefill_dispatch(shape, x, x_scale, topk_idx, slot_pos, expert_x, expert_scale,
                         expert_cnt, expert_off, expert_src, workspace, stream=None):
    _check("moe_prefill_dispatch", _lib.moe_prefill_dispatch(
        ctypes.byref(shape), _ptr(x), _ptr(x_scale), _ptr(topk_idx), _ptr(slot_pos),
        _ptr(expert_x), _ptr(expert_scale), _ptr(expert_cnt), _ptr(expert_off), _ptr(expert_src),
        _ptr(workspace), _stream(stream)))


def moe_prefill_combine_local(shape, expert_y, topk_idx, slot_pos, topk_w, partial, stream=None):
    _check("moe_prefill_combine_local", _lib.moe_prefill_combine_local(
        ctypes.byref(shape), _ptr(expert_y), _ptr(topk_idx), _ptr(slot_pos), _ptr(topk_w),
        _ptr(partial), _stream(stream)))


def moe_prefill_allreduce(shape, partial, out, stream=None):
    _check("moe_prefill_allreduce", _lib.moe_prefill_allreduce(
        ctypes.byref(shape), _ptr(partial), _ptr(out), _stream(stream)))


def moe_prefill_combine(shape, expert_y, topk_idx, slot_pos, topk_w, partial, out, stream=None):
    _check("moe_prefill_combine", _lib.moe_prefill_combine(
        ctypes.byref(shape), _ptr(expert_y), _ptr(topk_idx), _ptr(slot_pos), _ptr(topk_w),
        _ptr(partial), _ptr(out), _stream(stream)))


# ------------------------------------------------------------------ buffers (plumbing)


@dataclass
class Buffers:
    """Every device buffer of one dispatch/combine layer, allocated once with torch and reused.

    Shapes follow include/moe.h; byte-typed buffers are uint8 views of the right size."""
    shape: moe_shape
    sizes: dict
    t: dict

    def __getattr__(self, k):
        try:
            return self.__dict__["t"][k]
        except KeyError as ex:
            raise AttributeError(k) from ex


def alloc_buffers(N, T, H, E, R, fp8=False, capacity=0, device="cuda", with_status=True,
                  quant=False, tokens=False) -> Buffers:
    """Allocate every buffer of the path for one shape (torch.empty; contents undefined).
    quant: bf16 tokens, e4m3 rows made by the send pack.  tokens: also allocate the per-rank
    token counts (int32[N], filled with T) and point the shape at them."""
    fp8 = fp8 or quant
    shape = make_shape(N, T, H, E, R, fp8, capacity, quant=quant)
    sz = moe_sizes(shape)
    B, P = sz["capacity"], sz["row_bytes"]
    L = E // N
    dev = torch.device(device)
    i32, f32, u8, i16 = torch.int32, torch.float32, torch.uint8, torch.int16
    xdt = u8 if fp8 else i16
    t = dict(
        logits=torch.empty((N * T, E), dtype=f32, device=dev),
        bias=torch.zeros((E,), dtype=f32, device=dev),
        topk_idx=torch.empty((N, T * R), dtype=i32, device=dev),
        topk_w=torch.empty((N * T, R), dtype=f32, device=dev),
        x=torch.empty((N, T, H), dtype=i16 if quant else xdt, device=dev),
        x_scale=torch.empty((N, T, H // 128), dtype=f32, device=dev) if fp8 and not quant else None,
        counts=torch.empty((N, E), dtype=i32, device=dev),
        send_off=torch.empty((N, N + 1), dtype=i32, device=dev),
        send_pos=torch.empty((N, T * R), dtype=i32, device=dev),
        send_buf=torch.empty((N, T * R, P), dtype=u8, device=dev),
        send_meta=torch.empty((N, T * R, 2), dtype=i32, device=dev),
        recv_buf=torch.empty((N, B, P), dtype=u8, device=dev),
        recv_meta=torch.empty((N, B, 2), dtype=i32, device=dev),
        recv_off=torch.empty((N, N + 1), dtype=i32, device=dev),
        expert_x=torch.empty((N, B, H), dtype=xdt, device=dev),
        expert_scale=torch.empty((N, B, H // 128), dtype=f32, device=dev) if fp8 else None,
        expert_cnt=torch.empty((N, L), dtype=i32, device=dev),
        expert_off=torch.empty((N, L + 1), dtype=i32, device=dev),
        expert_src=torch.empty((N, B), dtype=i32, device=dev),
        expert_rpos=torch.empty((N, B), dtype=i32, device=dev),
        expert_y=torch.empty((N, B, H), dtype=i16, device=dev),
        cs_buf=torch.empty((N, B, H), dtype=i16, device=dev),
        cr_buf=torch.empty((N, T * R, H), dtype=i16, device=dev),
        out=torch.empty((N, T, H), dtype=i16, device=dev),
        workspace=torch.empty((max(sz["workspace"], 16),), dtype=u8, device=dev),
        status=torch.zeros((1,), dtype=i32, device=dev) if with_status else None,
        tokens=torch.full((N,), T, dtype=i32, device=dev) if tokens else None,
    )
    if with_status:
        shape.status = t["status"].data_ptr()
    if tokens:
        shape.tokens = t["tokens"].data_ptr()
    return Buffers(shape, sz, t)


def alloc_prefill_buffers(N, T, H, E, R, fp8=False, capacity=0, device="cuda",
                          with_status=True) -> Buffers:
    """Every buffer of the replicated-token (prefill) path for one shape (contents undefined)."""
    shape = make_shape(N, T, H, E, R, fp8, capacity, prefill=True)
    sz = moe_sizes(shape)
    B = sz["capacity"]
    L = E // N
    dev = torch.device(device)
    i32, f32, u8, i16 = torch.int32, torch.float32, torch.uint8, torch.int16
    xdt = u8 if fp8 else i16
    t = dict(
        logits=torch.empty((T, E), dtype=f32, device=dev),
        bias=torch.zeros((E,), dtype=f32, device=dev),
        topk_idx=torch.empty((T, R), dtype=i32, device=dev),
        topk_w=torch.empty((T, R), dtype=f32, device=dev),
        x=torch.empty((T, H), dtype=xdt, device=dev),
        x_scale=torch.empty((T, H // 128), dtype=f32, device=dev) if fp8 else None,
        slot_pos=torch.empty((T, R), dtype=i32, device=dev),
        expert_x=torch.empty((N, B, H), dtype=xdt, device=dev),
        expert_scale=torch.empty((N, B, H // 128), dtype=f32, device=dev) if fp8 else None,
        expert_cnt=torch.empty((N, L), dtype=i32, device=dev),
        expert_off=torch.empty((N, L + 1), dtype=i32, device=dev),
        expert_src=torch.empty((N, B), dtype=i32, device=dev),
        expert_y=torch.empty((N, B, H), dtype=i16, device=dev),
        partial=torch.empty((N, T, H), dtype=f32, device=dev),
        out=torch.empty((T, H), dtype=i16, device=dev),
        workspace=torch.empty((max(sz["workspace"], 16),), dtype=u8, device=dev),
        status=torch.zeros((1,), dtype=i32, device=dev) if with_status else None,
    )
    if with_status:
        shape.status = t["status"].data_ptr()
    return Buffers(shape, sz, t)


def run_prefill_dispatch(b: Buffers, bias=True, stream=None):
    """route -> prefill dispatch on the buffers' replicated inputs."""
    moe_route(b.shape, b.logits, b.bias if bias else None, b.topk_idx, b.topk_w, stream)
    moe_prefill_dispatch(b.shape, b.x, b.x_scale, b.topk_idx, b.slot_pos, b.expert_x,
                         b.expert_scale, b.expert_cnt, b.expert_off, b.expert_src, b.workspace,
                         stream)


def run_dispatch(b: Buffers, bias=True, stream=None):
    """route -> dispatch_send -> network -> dispatch_recv on the buffers' inputs."""
    moe_route(b.shape, b.logits, b.bias if bias else None, b.topk_idx, b.topk_w, stream)
    moe_dispatch_send(b.shape, b.x, b.x_scale, b.topk_idx, b.counts, b.send_off, b.send_pos,
                      b.send_buf, b.send_meta, b.workspace, stream)
    moe_net_dispatch(b.shape, b.send_off, b.send_buf, b.send_meta, b.recv_buf, b.recv_meta,
                     b.recv_off, stream)
    moe_dispatch_recv(b.shape, b.counts, b.recv_off, b.recv_buf, b.recv_meta, b.expert_x,
                      b.expert_scale, b.expert_cnt, b.expert_off, b.expert_src, b.expert_rpos,
                      stream)


def run_combine(b: Buffers, expert_y=None, stream=None):
    y = b.expert_y if expert_y is None else expert_y
    moe_combine(b.shape, y, b.expert_rpos, b.recv_off, b.send_off, b.send_pos, b.topk_w,
                b.cs_buf, b.cr_buf, b.out, stream)


def run_combine_acc(b: Buffers, expert_y=None, stream=None):
    """The combine with the sum taken on the sending side, on the same buffers."""
    y = b.expert_y if expert_y is None else expert_y
    moe_combine_acc(b.shape, y, b.recv_meta, b.counts, b.recv_off, b.expert_off, b.send_off,
                    b.topk_w, b.topk_idx, b.send_pos, b.cs_buf, b.cr_buf, b.out, stream)
