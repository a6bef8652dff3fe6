"""GPU parity of the Ulysses layout kernels against the oracle: bit-exact.

Every case runs all W ranks of one Ulysses group through the C ABI (pack ->
simulated exchange -> unpack, then the output reverse) and compares every
intermediate buffer with the oracle element by element, plus the closed form of
the pages' unit test (rank j ends with head slice j of the sequence-concatenated
tensor).
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import layout as L

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    import gpu_util
    return gpu_util


def _check_group(gu, full, W, dtype=torch.bfloat16):
    """full: 3 global uint16 arrays [B, W*S_l, H, D] covering one Ulysses group."""
    B, S, H, D = full[0].shape
    Sl, Hl = S // W, H // W
    shards = [tuple(np.ascontiguousarray(t[:, r * Sl:(r + 1) * Sl]) for t in full) for r in range(W)]
    staging, recv, outs = gu.forward_all_ranks(shards, W, dtype)
    o_staging = [L.pack_qkv_dst_major(*shards[r], W) for r in range(W)]
    o_recv = L.exchange(o_staging)
    for r in range(W):
        np.testing.assert_array_equal(gu.to_bits(staging[r]), o_staging[r], err_msg=f"pack rank {r}")
        np.testing.assert_array_equal(gu.to_bits(recv[r]), o_recv[r], err_msg=f"exchange rank {r}")
        o_out = L.unpack_head_sharded(o_recv[r], B, W)
        for c in range(3):
            got = gu.to_bits(outs[r][c])
            np.testing.assert_array_equal(got, o_out[c], err_msg=f"unpack rank {r} c {c}")
            np.testing.assert_array_equal(got, full[c][:, :, r * Hl:(r + 1) * Hl],
                                          err_msg=f"spec rank {r} c {c}")
            assert outs[r][c].is_contiguous()
    # Output reverse on each head-sharded tensor: oracle parity and round trip (the
    # oracle reverses its own unpacked tensors).
    o_outs = [L.unpack_head_sharded(o_recv[r], B, W) for r in range(W)]
    for c in range(3):
        o_hs = [outs[r][c] for r in range(W)]
        snd, rcv, merged = gu.reverse_all_ranks(o_hs, W, B)
        o_snd = [L.output_reverse_send(o_outs[r][c], W) for r in range(W)]
        o_rcv = L.exchange(o_snd)
        for r in range(W):
            np.testing.assert_array_equal(gu.to_bits(snd[r]), o_snd[r], err_msg=f"send r{r} c{c}")
            np.testing.assert_array_equal(gu.to_bits(rcv[r]), o_rcv[r], err_msg=f"rcv r{r} c{c}")
            m = gu.to_bits(merged[r])
            np.testing.assert_array_equal(m, L.output_reverse_merge(o_rcv[r]), err_msg=f"merge r{r}")
            np.testing.assert_array_equal(m, shards[r][c], err_msg=f"round trip r{r} c{c}")


@pytest.mark.parametrize("W,B,S,H,D", workloads.PAGE_TEST_SHAPES)
def test_page_test_shapes(gu, W, B, S, H, D):
    print(f"[layout] page shape W={W} B={B} S={S} H={H} D={D}", flush=True)
    _check_group(gu, workloads.page_test_tensors(B, S, H, D), W)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_shapes(gu, name):
    wl = workloads.WORKLOADS[name]
    print(f"[layout] workload {name}", flush=True)
    span = wl.W * wl.S_local
    full = [np.ascontiguousarray(t[:, :span]) for t in workloads.global_qkv(wl)]
    _check_group(gu, full, wl.W)


@pytest.mark.parametrize("W,B,S,H,D", [
    (1, 1, 5, 3, 8),       # W = 1: every map is a copy
    (3, 3, 3, 3, 8),       # S_l = 1, H_l = 1, odd B
    (2, 2, 6, 4, 24),      # D = 24: head rows of 3 vectors (generic vector count)
    (4, 1, 36, 8, 64),
    (8, 2, 40, 16, 128),   # H_l = 2, ragged relative to a 1024-vector block
    (5, 1, 25, 10, 16),
])
def test_edge_shapes(gu, W, B, S, H, D):
    print(f"[layout] edge W={W} B={B} S={S} H={H} D={D}", flush=True)
    rng = np.random.default_rng(W * 1000 + S)
    full = [rng.integers(0, 65536, size=(B, S, H, D), dtype=np.uint16) for _ in range(3)]
    _check_group(gu, full, W)


def test_fp16_payload_is_moved_bit_exactly(gu):
    rng = np.random.default_rng(2)
    full = [rng.integers(0, 65536, size=(2, 16, 4, 64), dtype=np.uint16) for _ in range(3)]
    _check_group(gu, full, 2, dtype=torch.float16)


def test_staging_reuse_across_iterations(gu):
    # The same cached staging buffer serves back-to-back calls in stream order.
    import context_attention_diffusion_amd as cp
    W, B, Sl, H, D = 4, 2, 24, 8, 128
    cp.clear_staging()
    ptr = None
    for it in range(3):
        rng = np.random.default_rng(100 + it)
        x = [rng.integers(0, 65536, size=(B, Sl, H, D), dtype=np.uint16) for _ in range(3)]
        st = cp.cp_pack_qkv_dst_major(*(gu.to_dev(t) for t in x), W)
        if ptr is None:
            ptr = st.data_ptr()
        assert st.data_ptr() == ptr
        np.testing.assert_array_equal(gu.to_bits(st), L.pack_qkv_dst_major(*x, W))


def test_unpack_into_gathered_kv_slice(gu):
    # For B == 1 the unpacked K/V of Ulysses group a can be written straight into
    # rows [a*S/A, (a+1)*S/A) of the gathered global K/V buffer.
    import context_attention_diffusion_amd as cp
    W, Sl, H, D, A = 2, 16, 4, 128, 2
    rng = np.random.default_rng(8)
    full = [rng.integers(0, 65536, size=(1, W * Sl, H, D), dtype=np.uint16) for _ in range(3)]
    shards = [tuple(t[:, r * Sl:(r + 1) * Sl] for t in full) for r in range(W)]
    staging, recv, _ = gu.forward_all_ranks(shards, W)
    kg = torch.zeros((1, A * W * Sl, H // W, D), dtype=torch.bfloat16, device=gu.DEV)
    q = torch.empty((1, W * Sl, H // W, D), dtype=torch.bfloat16, device=gu.DEV)
    v = torch.empty_like(q)
    region = kg[:, W * Sl:]            # region a = 1
    cp.cp_unpack_head_sharded(recv[0], 1, W, out=(q, region, v))
    got = gu.to_bits(kg)
    np.testing.assert_array_equal(got[:, W * Sl:], full[1][:, :, :H // W])
    assert (got[:, :W * Sl] == 0).all()


@pytest.mark.parametrize("W,B,S,H,D", [(4, 1, 64, 14, 128), (4, 2, 24, 6, 64), (3, 1, 30, 4, 8), (8, 1, 64, 12, 128)])
def test_padded_pack_and_cropped_merge(gu, W, B, S, H, D):
    """Head padding (H % W != 0): padded pack -> exchange -> unpack, then the reverse
    with the cropped merge, every buffer bit-exact against the oracle."""
    import context_attention_diffusion_amd as cp
    rng = np.random.default_rng(W * 1000 + H * 10 + D)
    full = [rng.integers(1, 65535, size=(B, S, H, D)).astype(np.uint16) for _ in range(3)]
    H_pad = -(-H // W) * W
    Hl, Sl = H_pad // W, S // W
    shards = [tuple(np.ascontiguousarray(t[:, r * Sl:(r + 1) * Sl]) for t in full) for r in range(W)]
    print(f"[layout] padded W={W} B={B} S={S} H={H} H_pad={H_pad} D={D}", flush=True)
    staging = [cp.cp_pack_qkv_dst_major_padded(*(gu.to_dev(x) for x in shards[r]), W, H_pad,
                                               staging=torch.empty((W, B * Sl, Hl, 3 * D), dtype=torch.bfloat16,
                                                                   device=gu.DEV)) for r in range(W)]
    o_staging = [L.pack_qkv_dst_major_padded(*shards[r], W, H_pad) for r in range(W)]
    recv = [cp.cp_sim_exchange(staging, j) for j in range(W)]
    outs = [cp.cp_unpack_head_sharded(recv[j], B, W) for j in range(W)]
    for r in range(W):
        np.testing.assert_array_equal(gu.to_bits(staging[r]), o_staging[r], err_msg=f"padded pack rank {r}")
    # reverse of the unpacked tensors, cropped merge: every rank's original shard;
    # the oracle runs the same chain on its own buffers
    o_recv = L.exchange(o_staging)
    o_outs = [L.unpack_head_sharded(o_recv[j], B, W) for j in range(W)]
    for c in range(3):
        snd = [cp.cp_output_reverse(0, outs[j][c], W, B) for j in range(W)]
        rcv = [cp.cp_sim_exchange(snd, r) for r in range(W)]
        o_rcv = L.exchange([L.output_reverse_send(o_outs[j][c], W) for j in range(W)])
        for r in range(W):
            got = cp.cp_output_merge_cropped(rcv[r], H)
            o_got = L.output_merge_cropped(o_rcv[r], H)
            np.testing.assert_array_equal(gu.to_bits(got), o_got, err_msg=f"cropped merge rank {r} c {c}")
            np.testing.assert_array_equal(gu.to_bits(got), shards[r][c], err_msg=f"round trip rank {r} c {c}")
