"""moe_dispatch_send_noalloc: the dispatch send without a workspace argument (its histograms in
the library's static device array), against moe_dispatch_send with a caller workspace.

Two calls in a row on one GPU, the second on a smaller problem, so the second runs over the
array the first left behind; every output must equal the workspace call's bit for bit.
"""
import numpy as np
import pytest
import torch

import combine_moe_route_top_amd as moe
import moe_synth as ms


def _dispatch_send_pair(N, T, H, E, R, fp8, bias, seed):
    """Route once, then run both send calls on the same inputs into separate output buffers;
    returns the host copies of both calls' outputs."""
    inp = ms.make_inputs(N, T, H, E, R, fp8, bias, seed)
    a = moe.alloc_buffers(N, T, H, E, R, fp8)
    b = moe.alloc_buffers(N, T, H, E, R, fp8)
    assert a.workspace is not None and a.workspace.numel() > 0  # several count chunks per rank
    for buf in (a, b):
        for k in ("counts", "send_off", "send_pos", "send_buf", "send_meta"):
            getattr(buf, k).view(torch.uint8).fill_(0xA5)
        buf.status.zero_()
    a.logits.copy_(torch.from_numpy(inp["logits"]))
    use_bias = inp["bias"] is not None
    if use_bias:
        a.bias.copy_(torch.from_numpy(inp["bias"]))
    x = inp["x"]
    a.x.copy_(torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x))
    if fp8:
        a.x_scale.copy_(torch.from_numpy(inp["x_scale"]))
    moe.moe_route(a.shape, a.logits, a.bias if use_bias else None, a.topk_idx, a.topk_w)
    moe.moe_dispatch_send(a.shape, a.x, a.x_scale, a.topk_idx, a.counts, a.send_off, a.send_pos,
                          a.send_buf, a.send_meta, a.workspace)
    moe.moe_dispatch_send_noalloc(b.shape, a.x, a.x_scale, a.topk_idx, b.counts, b.send_off,
                                  b.send_pos, b.send_buf, b.send_meta)
    torch.cuda.synchronize()
    out = []
    for buf in (a, b):
        g = {k: getattr(buf, k).cpu().numpy() for k in ("counts", "send_off", "send_pos", "status")}
        so = g["send_off"]
        g["send_buf"] = [buf.send_buf[s, :so[s, N]].cpu().numpy() for s in range(N)]
        g["send_meta"] = [buf.send_meta[s, :so[s, N]].cpu().numpy() for s in range(N)]
        out.append(g)
    return out


@pytest.mark.gpu
def test_noalloc_send_equals_workspace_send():
    # the first call: 4 ranks of 4096 tokens, 32 count chunks per rank; the second, smaller:
    # 2 ranks of 700 tokens, e4m3 rows, 6 chunks per rank
    cases = [(4, 4096, 256, 128, 8, False, "zipf", 0), (2, 700, 512, 32, 8, True, "none", 1)]
    for N, T, H, E, R, fp8, bias, seed in cases:
        print(f"\ncase noalloc N{N} T{T} H{H} E{E} R{R} fp8 {fp8}", flush=True)
        ref, got = _dispatch_send_pair(N, T, H, E, R, fp8, bias, seed)
        assert ref["status"][0] == 0 and got["status"][0] == 0
        assert ref["counts"].sum() == N * T * R
        for k in ("counts", "send_off", "send_pos"):
            assert np.array_equal(ref[k], got[k]), k
        for s in range(N):
            assert np.array_equal(ref["send_buf"][s], got["send_buf"][s]), ("send_buf", s)
            assert np.array_equal(ref["send_meta"][s], got["send_meta"][s]), ("send_meta", s)


def test_noalloc_send_refuses_calls_beyond_its_scratch():
    # 1024 ranks and experts with 1600 slots per rank need 1024 * 7 * 1024 int32 histograms,
    # more than the static array holds: refused on the host, before any device work
    good = 1 << 20
    sh = moe.make_shape(1024, 200, 64, 1024, 8)
    assert moe.moe_sizes(sh)["workspace"] > moe.MOE_STATIC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError) as ex:
        moe.moe_dispatch_send_noalloc(sh, good, None, good, good, good, good, good, good, stream=0)
    assert ex.value.code == moe.MOE_ENOSCRATCH
    # the same on a range of ranks small enough to fit is accepted by validation (not run here)
    small = moe.moe_sizes(moe.make_shape(4, 200, 64, 1024, 8))["workspace"]
    assert 0 < small <= moe.MOE_STATIC_SCRATCH_BYTES
