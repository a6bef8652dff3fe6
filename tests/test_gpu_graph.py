"""The per-rank step captured into a HIP graph gives the eager result on every replay.

The step (pack -> simulated exchange -> unpack -> attention -> reverse merge) is
launched through the C ABI on the capturing stream.  The graph is replayed
several times with unrelated eager work and synchronisations in between, and
every replay is compared bit for bit with the eager run on the same inputs.
"""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("W,B,Sl,H,D", [(2, 1, 64, 4, 64), (4, 2, 72, 8, 128)])
def test_graph_replay_matches_eager(W, B, Sl, H, D):
    import context_attention_diffusion_amd as cp

    dev = "cuda:0"
    g = torch.Generator(device="cpu").manual_seed(W * 100 + Sl)
    Hl = H // W
    shards = [[torch.randn((B, Sl, H, D), generator=g).to(torch.bfloat16).to(dev) for _ in range(3)]
              for _ in range(W)]
    staging = [torch.empty((W, B * Sl, Hl, 3 * D), dtype=torch.bfloat16, device=dev) for _ in range(W)]
    for r in range(1, W):
        cp.cp_pack_qkv_dst_major(*shards[r], W, staging=staging[r])
    recv = torch.empty_like(staging[0])
    q_hs, k_hs, v_hs = (torch.empty((B, W * Sl, Hl, D), dtype=torch.bfloat16, device=dev) for _ in range(3))
    o_hs = torch.empty_like(q_hs)
    snd = torch.empty((W, B, Sl, Hl, D), dtype=torch.bfloat16, device=dev)
    peers = [None] + [torch.randn((W, B, Sl, Hl, D), generator=g).to(torch.bfloat16).to(dev)
                      for _ in range(1, W)]
    rcv = torch.empty_like(snd)
    out = torch.empty((B, Sl, H, D), dtype=torch.bfloat16, device=dev)

    def step():
        cp.cp_pack_qkv_dst_major(*shards[0], W, staging=staging[0])
        cp.cp_sim_exchange(staging, 0, recv=recv)
        cp.cp_unpack_head_sharded(recv, B, W, out=(q_hs, k_hs, v_hs))
        cp.cp_attn_localq_globalkv(q_hs, k_hs, v_hs, out=o_hs)
        s = o_hs.view(snd.shape) if B == 1 else cp.cp_output_reverse(0, o_hs, W, B, out=snd)
        cp.cp_sim_exchange([s] + peers[1:], 0, recv=rcv)
        cp.cp_output_reverse(1, rcv, W, B, out=out)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (staging[0], recv, q_hs, k_hs, v_hs, o_hs, rcv, out)]

    step()
    ref = snapshot()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        # clobber every output, do unrelated eager work, then replay
        for t in (staging[0], recv, q_hs, k_hs, v_hs, o_hs, rcv, out):
            t.fill_(float(rep + 1))
        junk = torch.randn(1 << 16, device=dev).sum()
        torch.cuda.synchronize()
        del junk
        graph.replay()
        got = snapshot()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
    print(f"graph replays match eager: W={W} B={B} S_l={Sl} H={H} D={D}", flush=True)
