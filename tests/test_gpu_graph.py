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


def _replays_match(step, outs, what):
    """Eager run, then four graph replays with the outputs clobbered and unrelated
    eager work in between; every replay must equal the eager outputs bit for bit."""
    dev = torch.device("cuda:0")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.fill_(float(rep + 1))
        junk = torch.randn(1 << 16, device=dev).sum()
        torch.cuda.synchronize()
        del junk
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"{what}: replay {rep} differs from the eager run"
    print(f"graph replays match eager: {what}", flush=True)


def _randn(shape, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16).to("cuda:0")


def test_graph_replay_fused_split_and_packed_paths():
    """The other calls the bench times under graph replay: split-KV attention (its
    workspace and merge kernel), the fused receive -> send call, its 2D form, and the
    packed-document remap + attention."""
    import context_attention_diffusion_amd as cp
    # split-KV: 4 query blocks against 4096 keys split over several workgroups
    q, k, v = _randn((1, 130, 2, 128), 1), _randn((1, 4096, 2, 128), 2), _randn((1, 4096, 2, 128), 3)
    o = torch.empty_like(q)
    ws = torch.zeros(cp.cp_attn_workspace_bytes(1, 130, 4096, 2, 128), dtype=torch.uint8, device="cuda:0")
    _replays_match(lambda: cp.cp_attn_localq_globalkv(q, k, v, None, out=o, workspace=ws), [o], "split-KV")
    # the same split through the library's own scratch array (nothing allocated per call)
    o2 = torch.empty_like(q)
    _replays_match(lambda: cp.cp_attn_localq_globalkv_noalloc(q, k, v, out=o2), [o2], "split-KV, no allocation")
    assert torch.equal(o2, o)
    # fused receive -> send, Ulysses W = 2, B = 2 (chunked rows)
    W, B, Sl, Hl, D = 2, 2, 70, 3, 128
    recv = _randn((W, B * Sl, Hl, 3 * D), 4)
    snd = torch.empty((W, B, Sl, Hl, D), dtype=torch.bfloat16, device="cuda:0")
    _replays_match(lambda: cp.cp_attn_recv_to_send(recv, B, W, None, out=snd, split=False), [snd], "recv_to_send")
    # 2D form: the other AllGather rank's K/V first
    recv1 = _randn((W, Sl, Hl, 3 * D), 5)
    ko, vo = _randn((1, 2 * Sl, Hl, D), 6), _randn((1, 2 * Sl, Hl, D), 7)
    snd1 = torch.empty((W, 1, Sl, Hl, D), dtype=torch.bfloat16, device="cuda:0")
    _replays_match(lambda: cp.cp_attn_recv_to_send_2d(recv1, ko, vo, 1, W, True, out=snd1, split=False), [snd1],
                   "recv_to_send_2d")
    # packed documents: remap on the device, then the packed attention of rank 1 of 2
    S, H = 600, 2
    qs, ks, vs = _randn((S // 2, H, D), 8), _randn((S, H, D), 9), _randn((S, H, D), 10)
    cu = torch.tensor([0, 170, 171, 420, 600], dtype=torch.int32, device="cuda:0")
    loc = torch.empty_like(cu)
    ov = torch.zeros((S // 2, H, D), dtype=torch.bfloat16, device="cuda:0")

    def packed():
        cp.cp_varlen_remap_cu_seqlens_q(cu, 1, S // 2, out=loc)
        cp.cp_attn_varlen(qs, ks, vs, loc, cu, out=ov)
    _replays_match(packed, [loc, ov], "packed documents")
