"""The whole layer captured in a HIP graph (torch.cuda.graph) and replayed: the calls enqueue
kernels only (no host synchronisation, no allocation, counts stay on the device), so a captured
layer replays correctly for new inputs written into the same buffers.  Every replay is checked
against an eager run of the same inputs, with eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

import moe_synth as ms
import parity

pytestmark = pytest.mark.gpu


def _layer(moe, b, use_bias, fp8):
    moe.moe_route(b.shape, b.logits, b.bias if use_bias else None, b.topk_idx, b.topk_w)
    moe.moe_dispatch_send(b.shape, b.x, b.x_scale, b.topk_idx, b.counts, b.send_off, b.send_pos,
                          b.send_buf, b.send_meta, b.workspace)
    moe.moe_net_dispatch(b.shape, b.send_off, b.send_buf, b.send_meta, b.recv_buf, b.recv_meta,
                         b.recv_off)
    moe.moe_dispatch_recv(b.shape, b.counts, b.recv_off, b.recv_buf, b.recv_meta, b.expert_x,
                          b.expert_scale, b.expert_cnt, b.expert_off, b.expert_src, b.expert_rpos)
    moe.moe_expert_stub(b.shape, 1, b.expert_x, b.expert_scale, b.expert_off, b.expert_y)
    moe.moe_combine(b.shape, b.expert_y, b.expert_rpos, b.recv_off, b.send_off, b.send_pos,
                    b.topk_w, b.cs_buf, b.cr_buf, b.out)


@pytest.mark.parametrize("case", [(8, 64, 512, 64, 8, False, "zipf"),
                                  (4, 300, 512, 16, 4, True, "none")],
                         ids=["bf16", "fp8-2chunks"])
def test_graph_replay_matches_eager(case):
    import combine_moe_route_top_amd as moe
    N, T, H, E, R, fp8, bias = case
    print(f"\ncase graph {case}", flush=True)
    g_buf = moe.alloc_buffers(N, T, H, E, R, fp8)
    e_buf = moe.alloc_buffers(N, T, H, E, R, fp8)
    inputs = [ms.make_inputs(N, T, H, E, R, fp8, bias, seed) for seed in range(4)]
    parity.upload_inputs(g_buf, inputs[0])
    use_bias = inputs[0]["bias"] is not None
    # warm up on a side stream (as torch's graph capture expects), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _layer(moe, g_buf, use_bias, fp8)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _layer(moe, g_buf, use_bias, fp8)
    torch.cuda.synchronize()
    for i, inp in enumerate(inputs * 2):
        parity.upload_inputs(g_buf, inp)          # eager writes into the captured buffers
        graph.replay()
        parity.upload_inputs(e_buf, inp)
        _layer(moe, e_buf, use_bias, fp8)          # eager reference on separate buffers
        torch.cuda.synchronize()
        gg = parity.fetch(g_buf, N, T, R)
        ee = parity.fetch(e_buf, N, T, R)
        for k in ("topk_idx", "topk_w", "counts", "send_off", "send_pos", "recv_off",
                  "expert_cnt", "expert_off", "out", "status"):
            assert np.array_equal(gg[k], ee[k]), (i, k)
        for k in ("recv_rows", "expert_x", "expert_src", "expert_rpos", "cs_buf", "cr_buf"):
            for d in range(N):
                assert np.array_equal(gg[k][d], ee[k][d]), (i, k, d)
    # and the last replay against the oracle
    o = parity.oracle_run(N, T, H, E, R, fp8, inputs[-1], expert_mode=1)
    parity.compare(gg, o, N, T, H, E, R, fp8)


def test_graph_replay_with_changing_token_counts():
    # one captured layer serves every batch mix: the per-rank token counts live on the device and
    # are rewritten between replays; every replay matches the oracle for that mix, and rows of
    # absent tokens keep what was there before
    import combine_moe_route_top_amd as moe
    N, T, H, E, R = 8, 64, 512, 64, 8
    print("\ncase graph with token counts", flush=True)
    b = moe.alloc_buffers(N, T, H, E, R, tokens=True)
    inp = ms.make_inputs(N, T, H, E, R, False, "zipf", 3)
    parity.upload_inputs(b, inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _layer(moe, b, True, False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _layer(moe, b, True, False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    mixes = [np.full(N, T, np.int32), rng.integers(0, T + 1, N).astype(np.int32),
             np.zeros(N, np.int32), rng.integers(1, T + 1, N).astype(np.int32)]
    for i, tokens in enumerate(mixes):
        print(f"  replay {i} tokens {tokens.tolist()}", flush=True)
        b.out.fill_(0x5A5A)
        b.topk_idx.fill_(-5)
        b.tokens.copy_(torch.from_numpy(tokens))
        graph.replay()
        torch.cuda.synchronize()
        g = parity.fetch(b, N, T, R)
        present = (np.arange(T)[None, :] < tokens[:, None])
        assert np.all(g["out"][~present] == 0x5A5A), i
        assert np.all(g["topk_idx"].reshape(N, T, R)[~present] == -5), i
        o = parity.oracle_run(N, T, H, E, R, False, inp, expert_mode=1, tokens=tokens)
        parity.compare(g, o, N, T, H, E, R, False)
