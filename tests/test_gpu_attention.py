"""GPU parity of cp_attn_localq_globalkv against the fp64 oracle.

Bar: max|err| <= 2e-2 and mean|err| <= 2e-3 against the fp64 oracle on the same
bf16 inputs.  Every test compares the whole output element by element: small and ragged
shapes, and the full-size workloads (whose oracle results are computed once per
process, tests/oracle_ref.py), plus properties that hold at any size.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as OA
from oracle import bf16

pytestmark = pytest.mark.gpu

MAX_ERR = 2e-2
MEAN_ERR = 2e-3


@pytest.fixture(scope="module")
def gu():
    import gpu_util
    return gpu_util


def _run(gu, q, k, v, mask=None, scale=None):
    import context_attention_diffusion_amd as cp
    qd, kd, vd = gu.to_dev(q), gu.to_dev(k), gu.to_dev(v)
    md = None if mask is None else torch.from_numpy(mask).to(gu.DEV)
    o = cp.cp_attn_localq_globalkv(qd, kd, vd, md, scale=scale)
    torch.cuda.synchronize()
    return gu.to_f64(o)


def _assert_close(got, ref, what):
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    print(f"  {what}: max|err| {mx:.3e} mean|err| {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR, f"{what}: max {mx} mean {mean}"


def _rand_bits(shape, seed, mult=1.0):
    x = np.random.default_rng(seed).standard_normal(shape) * mult
    return bf16.f64_to_bits_rne(x)


def test_tiny_workload_full_compare(gu):
    wl = workloads.WORKLOADS["tiny_w2"]
    q, k, v = workloads.global_qkv(wl)
    q = np.ascontiguousarray(q[:, :wl.attn_rows])
    got = _run(gu, q, k, v, scale=1.0 / math.sqrt(wl.D))
    ref = OA.attention(bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v),
                       scale=1.0 / math.sqrt(wl.D))
    _assert_close(got, ref, "tiny_w2")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sq,Skv", [(1, 1), (7, 5), (127, 63), (129, 65), (300, 200), (33, 513)])
@pytest.mark.parametrize("masked", [False, True])
def test_ragged_shapes(gu, D, Sq, Skv, masked):
    B, H = 2, 3
    seed = Sq * 7919 + Skv * 31 + D + int(masked)
    q = _rand_bits((B, Sq, H, D), seed)
    k = _rand_bits((B, Skv, H, D), seed + 1)
    v = _rand_bits((B, Skv, H, D), seed + 2)
    mask = None
    if masked:
        mask = (np.random.default_rng(seed + 3).random((B, Skv)) > 0.35).astype(np.uint8)
        mask[:, 0] = 1
    print(f"[attn] ragged D={D} Sq={Sq} Skv={Skv} masked={masked}", flush=True)
    got = _run(gu, q, k, v, mask)
    ref = OA.attention(bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v), mask)
    _assert_close(got, ref, f"D{D} Sq{Sq} Skv{Skv} m{int(masked)}")


def test_scale_and_large_logits(gu):
    B, Sq, Skv, H, D = 1, 130, 300, 2, 128
    q = _rand_bits((B, Sq, H, D), 41, mult=4.0)
    k = _rand_bits((B, Skv, H, D), 42, mult=4.0)
    v = _rand_bits((B, Skv, H, D), 43)
    for scale in (0.3, 1.0 / math.sqrt(D), 0.01):
        got = _run(gu, q, k, v, scale=scale)
        ref = OA.attention(bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v), scale=scale)
        _assert_close(got, ref, f"scale {scale}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("big_half", [0, 1])
@pytest.mark.parametrize("mask_first", [False, True])
def test_scores_rising_past_the_running_max(gu, D, big_half, mask_first):
    """Keys whose scores jump well past every earlier key's in the middle of the
    sequence (softmax taken against an older running max until the probabilities
    grow too large): tiles 0-1 at 0, tiles 2-3 with one 32-key half at +30 and
    the other at +27, later tiles at +29, in log2 units of the softmax.  Both
    halves of tiles 2-3 and the later tiles carry weight in the result."""
    B, Sq, Skv, H = 1, 130, 613, 2
    rng = np.random.default_rng(90 + D + 2 * big_half + 4 * int(mask_first))
    j = np.arange(Skv)
    tile, half = j // 64, (j % 64) // 32
    level = np.where(tile < 2, 0.0, np.where(tile < 4, np.where(half == big_half, 30.0, 27.0), 29.0))
    q = rng.standard_normal((B, Sq, H, D)) * 0.1
    q[..., 0] = (1.0 + 0.1 * np.arange(Sq) / Sq)[None, :, None]
    k = rng.standard_normal((B, Skv, H, D)) * 0.1
    k[..., 0] = (level / math.log2(math.e))[None, :, None]
    v = rng.standard_normal((B, Skv, H, D))
    qb, kb, vb = bf16.f64_to_bits_rne(q), bf16.f64_to_bits_rne(k), bf16.f64_to_bits_rne(v)
    mask = None
    if mask_first:
        mask = np.ones((B, Skv), np.uint8)
        mask[:, :128] = 0
    print(f"[attn] rising scores D={D} big_half={big_half} mask_first={mask_first}", flush=True)
    got = _run(gu, qb, kb, vb, mask, scale=1.0)
    ref = OA.attention(bf16.bits_to_f64(qb), bf16.bits_to_f64(kb), bf16.bits_to_f64(vb), mask, 1.0)
    _assert_close(got, ref, f"rising D{D} h{big_half} m{int(mask_first)}")


@pytest.mark.parametrize("B,H,Sq,Skv,masked", [
    (1, 64, 1024, 333, False),   # every head in 256-row blocks, ragged key tail
    (2, 32, 1000, 65, True),     # last block 232 rows (group 1 partly empty), two key tiles, masked
    (1, 64, 900, 1, False),      # last block 132 rows, one key
    (1, 64, 1152, 64, True),     # last block 128 rows (group 1 empty), exactly one key tile
    (1, 64, 800, 333, True),     # last block 32 rows: waves 1-3 of group 0 and all of group 1 idle, six tiles
    (1, 6, 16380, 300, False),   # heads 0-3 in 256-row blocks, heads 4-5 in 128-row blocks
    (2, 6, 8192, 100, True),     # the same split with two batches
])
def test_wide_blocks_match_oracle(gu, B, H, Sq, Skv, masked):
    """Shapes with enough query blocks that a 256-CU part runs some or all heads in
    256-row blocks (two key groups on different rows sharing every K/V tile)."""
    D = 128
    seed = 7000 + Sq + Skv + H
    q = _rand_bits((B, Sq, H, D), seed)
    k = _rand_bits((B, Skv, H, D), seed + 1)
    v = _rand_bits((B, Skv, H, D), seed + 2)
    mask = None
    if masked:
        mask = (np.random.default_rng(seed + 3).random((B, Skv)) > 0.3).astype(np.uint8)
        mask[:, -1] = 1
    print(f"[attn] wide B={B} H={H} Sq={Sq} Skv={Skv} masked={masked}", flush=True)
    got = _run(gu, q, k, v, mask)
    ref = OA.attention(bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v), mask)
    _assert_close(got, ref, f"wide B{B} H{H} Sq{Sq} Skv{Skv} m{int(masked)}")


@pytest.mark.parametrize("B,H,Sq,Skv,split", [
    (2, 3, 200, 1000, False),    # 128-row blocks, both key groups
    (2, 3, 200, 1000, True),     # the same through split-KV
    (1, 64, 1024, 700, False),   # 256-row blocks (group 1 keeps its own mask bits)
    (1, 6, 16380, 300, False),   # heads split between 256- and 128-row blocks
])
def test_sparse_mask_tiles(gu, B, H, Sq, Skv, split):
    """Single invalid keys in a few tiles (adjacent ones, the last one, both key
    groups), every other tile fully valid, and huge values on the invalid keys: a
    tile that skipped its bias would let one of them into the output."""
    import context_attention_diffusion_amd as cp
    D = 128
    seed = 9100 + Sq + Skv + H
    q = _rand_bits((B, Sq, H, D), seed)
    k = _rand_bits((B, Skv, H, D), seed + 1)
    v = _rand_bits((B, Skv, H, D), seed + 2)
    mask = np.ones((B, Skv), np.uint8)
    for b in range(B):
        for key in (7 + 3 * b, 97 + 3 * b, 188 + b, Skv - 2 - b):
            mask[b, key] = 0
            v[b, key] = bf16.f64_to_bits_rne(np.full((H, D), 1000.0))
    print(f"[attn] sparse mask B={B} H={H} Sq={Sq} Skv={Skv} split={split}", flush=True)
    qd, kd, vd = gu.to_dev(q), gu.to_dev(k), gu.to_dev(v)
    md = torch.from_numpy(mask).to(gu.DEV)
    o = cp.cp_attn_localq_globalkv(qd, kd, vd, md, split=split)
    torch.cuda.synchronize()
    ref = OA.attention(bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v), mask)
    _assert_close(gu.to_f64(o), ref, f"sparse mask B{B} H{H} Sq{Sq} Skv{Skv} split{int(split)}")


def test_mask_closed_forms(gu):
    B, Sq, Skv, H, D = 3, 70, 150, 2, 128
    q = _rand_bits((B, Sq, H, D), 51)
    k = _rand_bits((B, Skv, H, D), 52)
    v = _rand_bits((B, Skv, H, D), 53)
    mask = np.zeros((B, Skv), np.uint8)
    mask[0, 77] = 1            # one valid key: every output row is that value row
    mask[2, :] = 1
    mask[2, 100:] = 0          # batch 1 stays fully masked: zeros
    got = _run(gu, q, k, v, mask)
    vf = bf16.bits_to_f64(v)
    for i in range(Sq):
        np.testing.assert_array_equal(got[0, i], vf[0, 77])
    assert (got[1] == 0).all()
    ref = OA.attention(bf16.bits_to_f64(q), bf16.bits_to_f64(k), vf, mask)
    _assert_close(got[2], ref[2], "partial mask")


def test_zero_query_gives_mean_of_valid_values(gu):
    B, Sq, Skv, H, D = 2, 40, 333, 2, 64
    q = np.zeros((B, Sq, H, D), np.uint16)
    k = _rand_bits((B, Skv, H, D), 61)
    v = _rand_bits((B, Skv, H, D), 62)
    mask = (np.random.default_rng(63).random((B, Skv)) > 0.5).astype(np.uint8)
    got = _run(gu, q, k, v, mask)
    vf = bf16.bits_to_f64(v)
    for b in range(B):
        mean = vf[b][mask[b] != 0].mean(axis=0)
        _assert_close(got[b], np.broadcast_to(mean, got[b].shape), f"Q=0 batch {b}")


def test_key_permutation_invariance(gu):
    B, Sq, Skv, H, D = 1, 128, 256, 2, 128
    q = _rand_bits((B, Sq, H, D), 71)
    k = _rand_bits((B, Skv, H, D), 72)
    v = _rand_bits((B, Skv, H, D), 73)
    perm = np.random.default_rng(74).permutation(Skv)
    a = _run(gu, q, k, v)
    b = _run(gu, q, np.ascontiguousarray(k[:, perm]), np.ascontiguousarray(v[:, perm]))
    _assert_close(a, b, "permuted keys")


def test_deterministic(gu):
    B, Sq, Skv, H, D = 1, 256, 700, 4, 128
    q, k, v = (_rand_bits((B, s, H, D), 80 + i) for i, s in enumerate((Sq, Skv, Skv)))
    a = _run(gu, q, k, v)
    b = _run(gu, q, k, v)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("name", ["image_cp4", "image_cp8", "video_u2a2", "joint_cfg_cp4"])
def test_full_size_workloads_whole(gu, name):
    """Rank 0's attention at the workload's full size, every output element against
    the fp64 oracle."""
    from oracle_ref import workload_attention
    wl = workloads.WORKLOADS[name]
    print(f"[attn] full-size {name}", flush=True)
    qg, kg, vg = workloads.global_qkv(wl, heads=wl.attn_heads)
    q = np.ascontiguousarray(qg[:, :wl.attn_rows])
    mask = workloads.key_mask(wl)
    got = _run(gu, q, kg, vg, mask, scale=1.0 / math.sqrt(wl.D))
    ref = workload_attention(name, 0, wl.attn_rows, wl.attn_heads)
    _assert_close(got, ref, f"{name} whole output")
    # Any-size property: every output lies within [min, max] of the valid value rows.
    vf = torch.from_numpy(vg).view(torch.int16).view(torch.bfloat16).float()
    for b in range(wl.B):
        valid = torch.ones(wl.S, dtype=torch.bool) if mask is None else torch.from_numpy(mask[b] != 0)
        vv = vf[b][valid]
        lo, hi = vv.min(dim=0).values.numpy(), vv.max(dim=0).values.numpy()
        assert (got[b] >= lo - 1e-2).all() and (got[b] <= hi + 1e-2).all()


@pytest.mark.parametrize("B,H,Sq,Skv,D,masked", [
    (1, 2, 130, 4096, 128, False),   # 4 query blocks x 32 iterations: every block split over 32 workgroups
    (2, 3, 70, 700, 64, True),       # masked, ragged keys, D 64
    (1, 1, 5, 3000, 128, True),      # one query block split many ways, most rows invalid
    (1, 24, 1088, 4352, 128, False),  # image CP4 share: 216 blocks, split over the compute units
    (1, 24, 512, 2600, 128, False),  # image CP8 rows, ragged keys: 96 blocks, each split over 2 workgroups
    (2, 12, 512, 2600, 128, True),   # the same with two batches and a key mask
])
def test_split_kv_matches_oracle_and_unsplit(gu, B, H, Sq, Skv, D, masked):
    import context_attention_diffusion_amd as cp
    seed = 9000 + Sq + Skv + D
    q = _rand_bits((B, Sq, H, D), seed)
    k = _rand_bits((B, Skv, H, D), seed + 1)
    v = _rand_bits((B, Skv, H, D), seed + 2)
    mask = None
    if masked:
        mask = (np.random.default_rng(seed + 3).random((B, Skv)) > 0.4).astype(np.uint8)
        mask[:, 0] = 1
    qd, kd, vd = gu.to_dev(q), gu.to_dev(k), gu.to_dev(v)
    md = None if mask is None else torch.from_numpy(mask).to(gu.DEV)
    print(f"[attn] split B={B} H={H} Sq={Sq} Skv={Skv} D={D} masked={masked}", flush=True)
    o_split = cp.cp_attn_localq_globalkv(qd, kd, vd, md, split=True)
    o_split2 = cp.cp_attn_localq_globalkv(qd, kd, vd, md, split=True)
    o_whole = cp.cp_attn_localq_globalkv(qd, kd, vd, md, split=False)
    torch.cuda.synchronize()
    assert torch.equal(o_split, o_split2), "split results differ between runs"
    got, whole = gu.to_f64(o_split), gu.to_f64(o_whole)
    ref = OA.attention(bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v), mask)
    _assert_close(got, ref, f"split B{B} H{H} Sq{Sq} Skv{Skv} D{D} m{int(masked)}")
    # the two schedules sum the same terms in a different order
    assert np.abs(got - whole).max() <= 2e-2


# ------------------------------------------- attention fused with unpack and send

def _fused_ref_chain(cp, recv_d, B, W, md):
    """The unfused GPU chain the fused entry point replaces."""
    q, k, v = cp.cp_unpack_head_sharded(recv_d, B, W)
    o = cp.cp_attn_localq_globalkv(q, k, v, md)
    return cp.cp_output_reverse(0, o, W, B)


@pytest.mark.parametrize("B,W,Sl,Hl,D,masked", [
    (1, 2, 128, 2, 64, False),    # tiny-workload shape
    (1, 3, 70, 2, 64, True),      # ragged: 210 rows, tiles and query blocks with tails
    (1, 2, 33, 1, 128, False),    # fewer rows than one tile
    (2, 2, 64, 3, 128, True),     # several batches: rows arrive in chunks of S_l
    (2, 4, 128, 2, 128, False),
    (3, 2, 192, 1, 64, True),
    (1, 4, 1024, 1, 128, False),  # 32 query blocks: split-KV, strided views
    (2, 2, 2048, 1, 128, True),   # 64 query blocks: split-KV, chunked rows
    (2, 2, 70, 2, 128, True),     # S_l % 64 != 0: key tiles span two source ranks' chunks
    (3, 3, 100, 1, 64, False),
    (2, 4, 40, 2, 128, True),     # chunks shorter than a tile: a tile spans up to three chunks
    (2, 3, 8, 1, 64, True),       # eight-row chunks
    (2, 2, 1000, 1, 128, False),  # 32 query blocks with spanning tiles: split-KV
    (2, 2, 1000, 16, 128, True),  # 256 blocks of 256 rows: wide blocks over chunks that tiles span
])
def test_recv_to_send_matches_oracle_and_unfused(gu, B, W, Sl, Hl, D, masked):
    import context_attention_diffusion_amd as cp
    from oracle import cp_share
    seed = 7000 + B * 100 + W * 10 + Sl + D
    recv = _rand_bits((W, B * Sl, Hl, 3 * D), seed)
    S = W * Sl
    mask = None
    if masked:
        mask = (np.random.default_rng(seed + 1).random((B, S)) > 0.3).astype(np.uint8)
        mask[:, S - 1] = 1
    rd = gu.to_dev(recv)
    md = None if mask is None else torch.from_numpy(mask).to(gu.DEV)
    print(f"[attn] recv_to_send B={B} W={W} Sl={Sl} Hl={Hl} D={D} masked={masked}", flush=True)
    got = cp.cp_attn_recv_to_send(rd, B, W, md)
    ref_gpu = _fused_ref_chain(cp, rd, B, W, md)
    torch.cuda.synchronize()
    assert torch.equal(got, ref_gpu), "fused result differs from unpack -> attention -> send"
    ref = cp_share.ulysses_attention_send(bf16.bits_to_f64(recv), B, W, mask)
    _assert_close(gu.to_f64(got), ref, f"recv_to_send B{B} W{W} Sl{Sl} Hl{Hl} D{D}")


@pytest.mark.parametrize("B,W,Sl,Hl,D,So,other_first,masked", [
    (1, 2, 128, 2, 64, 256, False, False),   # region 0 of a U=2 x A=2 layout
    (1, 2, 128, 2, 64, 256, True, False),    # region 1: the other rank's keys first
    (1, 2, 70, 2, 128, 140, True, True),     # ragged: segments end mid-tile, row strides 3D*H vs D*H
    (2, 2, 64, 3, 128, 128, False, True),    # several batches: chunked received rows
    (2, 3, 70, 1, 64, 210, True, True),      # chunked rows whose tiles span chunks, two segments
    (1, 4, 512, 1, 128, 2048, False, False), # split-KV
    (2, 2, 1000, 16, 128, 500, True, True),  # wide blocks: chunked rows, spanning tiles, two segments
])
def test_recv_to_send_2d_matches_oracle_and_unfused(gu, B, W, Sl, Hl, D, So, other_first, masked):
    import context_attention_diffusion_amd as cp
    from oracle import cp_share
    seed = 7500 + B * 100 + W * 10 + Sl + D + So + int(other_first)
    recv = _rand_bits((W, B * Sl, Hl, 3 * D), seed)
    ko, vo = _rand_bits((B, So, Hl, D), seed + 1), _rand_bits((B, So, Hl, D), seed + 2)
    S = W * Sl
    om = xm = None
    if masked:
        rng = np.random.default_rng(seed + 3)
        om = (rng.random((B, S)) > 0.3).astype(np.uint8)
        xm = (rng.random((B, So)) > 0.3).astype(np.uint8)
        om[:, -1] = 1
    rd, kd, vd = gu.to_dev(recv), gu.to_dev(ko), gu.to_dev(vo)
    omd = None if om is None else torch.from_numpy(om).to(gu.DEV)
    xmd = None if xm is None else torch.from_numpy(xm).to(gu.DEV)
    print(f"[attn] recv_to_send_2d B={B} W={W} Sl={Sl} Hl={Hl} D={D} So={So} other_first={other_first} "
          f"masked={masked}", flush=True)
    got = cp.cp_attn_recv_to_send_2d(rd, kd, vd, B, W, other_first, omd, xmd)
    q, k, v = cp.cp_unpack_head_sharded(rd, B, W)
    o = cp.cp_attn_joint(q, k, v, kd, vd, omd, xmd, joint_front=other_first)
    ref_gpu = cp.cp_output_reverse(0, o, W, B)
    torch.cuda.synchronize()
    assert torch.equal(got, ref_gpu), "fused result differs from unpack -> joint attention -> send"
    ref = cp_share.ulysses_2d_attention_send(bf16.bits_to_f64(recv), bf16.bits_to_f64(ko), bf16.bits_to_f64(vo),
                                             B, W, other_first, om, xm)
    _assert_close(gu.to_f64(got), ref, f"recv_to_send_2d B{B} W{W} Sl{Sl} Hl{Hl} D{D} So{So}")


@pytest.mark.parametrize("name", ["image_cp4", "joint_cfg_cp4"])
def test_recv_to_send_full_size_whole(gu, name):
    """Rank 0 of the workload's Ulysses group at full size: the whole send buffer
    against the unfused chain (bit for bit) and against the oracle (every element)."""
    import context_attention_diffusion_amd as cp
    from oracle import layout as OL
    from oracle_ref import workload_attention
    wl = workloads.WORKLOADS[name]
    W, B, Sl, D = wl.W, wl.B, wl.S_local, wl.D
    Hl = wl.H // W
    full = workloads.global_qkv(wl)
    shards = [tuple(np.ascontiguousarray(t[:, r * Sl:(r + 1) * Sl]) for t in full) for r in range(W)]
    recv0 = OL.exchange([OL.pack_qkv_dst_major(*shards[r], W) for r in range(W)])[0]
    mask = workloads.key_mask(wl)
    rd = gu.to_dev(recv0)
    md = None if mask is None else torch.from_numpy(mask).to(gu.DEV)
    print(f"[attn] recv_to_send full {name}", flush=True)
    got = cp.cp_attn_recv_to_send(rd, B, W, md)
    ref_gpu = _fused_ref_chain(cp, rd, B, W, md)
    torch.cuda.synchronize()
    assert torch.equal(got, ref_gpu)
    # rank 0 holds heads [0, Hl) of the sequence-concatenated global tensors; the send
    # layout [W][B][S_l][Hl][D] puts global row r*S_l + s of batch b at [r, b, s]
    ref = workload_attention(name, 0, W * Sl, Hl)
    g = gu.to_f64(got).transpose(1, 0, 2, 3, 4).reshape(B, W * Sl, Hl, D)
    _assert_close(g, ref, f"recv_to_send {name} whole output")


@pytest.mark.parametrize("a", [0, 1])
def test_recv_to_send_2d_full_size_whole(gu, a):
    """The video 2D layout (U 2 x A 2) at full size, Ulysses rank u = 0 of AllGather
    index a: the received buffer of its Ulysses group and the other AllGather rank's
    resident K/V of the same heads; the whole send buffer against the unfused chain
    (bit for bit) and against the oracle (every element)."""
    import context_attention_diffusion_amd as cp
    from oracle import layout as OL
    from oracle_ref import workload_attention
    wl = workloads.WORKLOADS["video_u2a2"]
    U, A, Sl, D = wl.W, wl.A, wl.S_local, wl.D
    Hl = wl.H // U
    full = workloads.global_qkv(wl)
    reg = U * Sl   # rows of one AllGather region
    shards = [tuple(np.ascontiguousarray(t[:, (a * U + r) * Sl:(a * U + r + 1) * Sl]) for t in full)
              for r in range(U)]
    recv0 = OL.exchange([OL.pack_qkv_dst_major(*shards[r], U) for r in range(U)])[0]
    o_reg = slice((1 - a) * reg, (2 - a) * reg)
    ko, vo = (np.ascontiguousarray(t[:, o_reg, :Hl]) for t in full[1:])
    del full, shards
    rd, kd, vd = gu.to_dev(recv0), gu.to_dev(ko), gu.to_dev(vo)
    print(f"[attn] recv_to_send_2d full video_u2a2 a={a}", flush=True)
    got = cp.cp_attn_recv_to_send_2d(rd, kd, vd, 1, U, other_first=(a == 1))
    q, k, v = cp.cp_unpack_head_sharded(rd, 1, U)
    o = cp.cp_attn_joint(q, k, v, kd, vd, None, None, joint_front=(a == 1))
    ref_gpu = cp.cp_output_reverse(0, o, U, 1)
    torch.cuda.synchronize()
    assert torch.equal(got, ref_gpu)
    # rank (a, 0): query rows of region a, heads [0, Hl), against every key row of those heads
    ref = workload_attention("video_u2a2", a * reg, (a + 1) * reg, Hl)
    g = gu.to_f64(got).reshape(1, reg, Hl, D)      # B == 1: the send layout is the row order
    _assert_close(g, ref, f"recv_to_send_2d video a={a} whole output")


# ------------------------------------------ attention over K/V chunks, then merge

# The row sum adds bf16-rounded probabilities (each within 2^-9 relative of the
# exact value), so ln(sum) is within about 2^-9 of the exact log-sum-exp; the
# bound below allows twice that plus fp32 rounding.
LSE_ERR = 5e-3


def _partials(cp, qd, k, v, mask, edges):
    outs, lses = [], []
    for a, b in zip(edges[:-1], edges[1:]):
        kd = torch.from_numpy(np.ascontiguousarray(k[:, a:b]).view(np.int16)).view(torch.bfloat16).to(qd.device)
        vd = torch.from_numpy(np.ascontiguousarray(v[:, a:b]).view(np.int16)).view(torch.bfloat16).to(qd.device)
        md = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask[:, a:b])).to(qd.device)
        o, l = cp.cp_attn_partial(qd, kd, vd, md)
        outs.append(o)
        lses.append(l)
    return torch.stack(outs), torch.stack(lses)


@pytest.mark.parametrize("B,H,Sq,Skv,D,cuts,masked", [
    (1, 2, 130, 1133, 128, (100, 433), False),
    (2, 3, 70, 300, 64, (64,), True),
    (1, 1, 5, 200, 128, (1, 2, 150), True),
    (2, 2, 257, 700, 128, (350,), False),
    (1, 64, 1000, 700, 128, (333,), True),     # every head in 256-row blocks, ragged last block
    (2, 6, 8192, 260, 128, (100,), False),     # heads 0-3 in 256-row blocks, heads 4-5 in 128-row blocks
])
def test_partial_and_merge_match_oracle(gu, B, H, Sq, Skv, D, cuts, masked):
    import context_attention_diffusion_amd as cp
    seed = 8000 + Sq + Skv + D
    q = _rand_bits((B, Sq, H, D), seed)
    k = _rand_bits((B, Skv, H, D), seed + 1)
    v = _rand_bits((B, Skv, H, D), seed + 2)
    mask = None
    if masked:
        mask = (np.random.default_rng(seed + 3).random((B, Skv)) > 0.4).astype(np.uint8)
        mask[:, -1] = 1
    edges = [0, *cuts, Skv]
    print(f"[attn] partial+merge B={B} H={H} Sq={Sq} Skv={Skv} D={D} cuts={cuts} masked={masked}", flush=True)
    qd = gu.to_dev(q)
    o_parts, lses = _partials(cp, qd, k, v, mask, edges)
    merged = cp.cp_attn_merge(o_parts, lses)
    torch.cuda.synchronize()
    qf, kf, vf = bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v)
    got_p = o_parts.double().cpu().numpy()
    got_l = lses.double().cpu().numpy()
    for n, (a, b) in enumerate(zip(edges[:-1], edges[1:])):
        mk = None if mask is None else mask[:, a:b]
        ref_o, ref_l = OA.attention_partial(qf, kf[:, a:b], vf[:, a:b], mk)
        _assert_close(got_p[n], ref_o, f"partial {n}")
        fin = np.isfinite(ref_l)
        assert np.array_equal(np.isfinite(got_l[n]), fin), "lse -inf pattern differs"
        assert np.all(got_p[n][~np.repeat(fin.transpose(0, 2, 1)[..., None], D, axis=3)] == 0)
        lerr = np.abs(got_l[n][fin] - ref_l[fin]).max() if fin.any() else 0.0
        print(f"  lse {n}: max|err| {lerr:.3e}", flush=True)
        assert lerr <= LSE_ERR
    _assert_close(gu.to_f64(merged), OA.attention(qf, kf, vf, mask), "merged")


def test_chunked_kv_arrival_full_size_whole(gu):
    """Image CP4 share with the gathered K/V arriving in four chunks of one rank's rows:
    every element of the merged output against the oracle."""
    import context_attention_diffusion_amd as cp
    from oracle_ref import workload_attention
    wl = workloads.WORKLOADS["image_cp4"]
    q, k, v = workloads.global_qkv(wl)
    q = np.ascontiguousarray(q[:, :wl.attn_rows])
    Sl = wl.S_local
    edges = [r * Sl for r in range(wl.W + 1)]
    print("[attn] chunked K/V image_cp4", flush=True)
    qd = gu.to_dev(q)
    o_parts, lses = _partials(cp, qd, k, v, None, edges)
    merged = cp.cp_attn_merge(o_parts, lses)
    dense = cp.cp_attn_localq_globalkv(qd, gu.to_dev(k), gu.to_dev(v))
    torch.cuda.synchronize()
    got, whole = gu.to_f64(merged), gu.to_f64(dense)
    assert np.abs(got - whole).max() <= 2e-2
    _assert_close(got, workload_attention("image_cp4", 0, wl.attn_rows, wl.attn_heads), "chunked image_cp4 whole")


# ------------------------------------------------- joint text/image key segments

@pytest.mark.parametrize("B,H,Sq,S_img,T,D,front,im_on,jm_on", [
    (1, 2, 130, 256, 77, 128, True, False, True),     # ragged joint segment first
    (2, 3, 70, 130, 64, 64, False, True, True),       # ragged image segment first
    (1, 1, 33, 64, 1, 128, True, True, False),        # one joint key
    (2, 2, 129, 500, 200, 128, False, False, False),  # no masks
    (1, 2, 64, 300, 0, 64, False, True, False),       # no joint tokens
    (1, 1, 256, 4096, 77, 128, True, False, True),    # 2 query blocks: split-KV over two segments
    (1, 64, 1024, 300, 1, 128, True, False, True),    # 256-row blocks: one joint key, then the image keys
    (1, 64, 1000, 64, 333, 128, False, True, True),   # 256-row blocks: a one-tile image segment, then the joint
])
def test_joint_segments_match_oracle(gu, B, H, Sq, S_img, T, D, front, im_on, jm_on):
    import context_attention_diffusion_amd as cp
    seed = 6000 + Sq + S_img + T + D
    q = _rand_bits((B, Sq, H, D), seed)
    ki, vi = _rand_bits((B, S_img, H, D), seed + 1), _rand_bits((B, S_img, H, D), seed + 2)
    kj = _rand_bits((B, T, H, D), seed + 3) if T else None
    vj = _rand_bits((B, T, H, D), seed + 4) if T else None
    rng = np.random.default_rng(seed + 5)
    im = (rng.random((B, S_img)) > 0.3).astype(np.uint8) if im_on else None
    jm = None
    if jm_on and T:
        jm = np.ones((B, T), dtype=np.uint8)
        for b in range(B):
            jm[b, int(rng.integers(1, T + 1)):] = 0     # text padding after L_b tokens
    if im is not None:
        im[:, 0] = 1
    dev = lambda x: None if x is None else (torch.from_numpy(x).to(gu.DEV) if x.dtype == np.uint8 else gu.to_dev(x))
    print(f"[attn] joint B={B} H={H} Sq={Sq} S_img={S_img} T={T} D={D} front={front} masks={im_on},{jm_on}",
          flush=True)
    got = cp.cp_attn_joint(dev(q), dev(ki), dev(vi), dev(kj), dev(vj), dev(im), dev(jm), joint_front=front)
    torch.cuda.synchronize()
    f = bf16.bits_to_f64
    ref = OA.joint_attention(f(q), f(ki), f(vi), None if kj is None else f(kj), None if vj is None else f(vj),
                             im, jm, joint_front=front)
    _assert_close(gu.to_f64(got), ref, f"joint S_img{S_img} T{T} front{int(front)}")


def test_joint_cfg_workload_segments(gu):
    """The joint CFG workload as two segments (4096 image keys, 512 text keys with the
    per-batch text padding mask): rear layout equals the concatenated masked call bit
    for bit (same tiles); the front layout, every element, against the oracle."""
    import context_attention_diffusion_amd as cp
    wl = workloads.WORKLOADS["joint_cfg_cp4"]
    q, k, v = workloads.global_qkv(wl)
    q = np.ascontiguousarray(q[:, :wl.attn_rows])
    S_img = wl.S - wl.text_tokens
    mask = workloads.key_mask(wl)
    ki, vi = np.ascontiguousarray(k[:, :S_img]), np.ascontiguousarray(v[:, :S_img])
    kj, vj = np.ascontiguousarray(k[:, S_img:]), np.ascontiguousarray(v[:, S_img:])
    jm = np.ascontiguousarray(mask[:, S_img:])
    assert mask[:, :S_img].all()
    print("[attn] joint workload segments", flush=True)
    qd = gu.to_dev(q)
    rear = cp.cp_attn_joint(qd, gu.to_dev(ki), gu.to_dev(vi), gu.to_dev(kj), gu.to_dev(vj), None,
                            torch.from_numpy(jm).to(gu.DEV))
    front = cp.cp_attn_joint(qd, gu.to_dev(ki), gu.to_dev(vi), gu.to_dev(kj), gu.to_dev(vj), None,
                             torch.from_numpy(jm).to(gu.DEV), joint_front=True)
    dense = cp.cp_attn_localq_globalkv(qd, gu.to_dev(k), gu.to_dev(v), torch.from_numpy(mask).to(gu.DEV))
    torch.cuda.synchronize()
    assert torch.equal(rear, dense), "rear joint layout differs from the concatenated call"
    assert np.abs(gu.to_f64(front) - gu.to_f64(dense)).max() <= 2e-2
    from oracle_ref import workload_attention
    # the front layout attends the same valid keys in another order: same oracle result
    _assert_close(gu.to_f64(front), workload_attention(wl.name, 0, wl.attn_rows, wl.attn_heads),
                  "joint front whole output")


@pytest.mark.parametrize("B,H,Sq,Skv,D,cuts,masked", [
    (1, 2, 130, 1133, 128, (100, 433), False),
    (2, 3, 70, 300, 64, (64, 65), True),
    (2, 2, 257, 700, 128, (350,), True),
    (1, 64, 1000, 500, 128, (100, 300), True),  # every head in 256-row blocks
    (1, 6, 16380, 300, 128, (64, 200), False),  # heads split between 256- and 128-row blocks
])
def test_partial_accumulate_matches_oracle(gu, B, H, Sq, Skv, D, cuts, masked):
    """partial(chunk 0) -> accumulate in place (middle chunks) -> accumulate with final
    bf16 output; the first chunk of a masked case has no valid key at all."""
    import context_attention_diffusion_amd as cp
    seed = 5000 + Sq + Skv + D
    q = _rand_bits((B, Sq, H, D), seed)
    k = _rand_bits((B, Skv, H, D), seed + 1)
    v = _rand_bits((B, Skv, H, D), seed + 2)
    mask = None
    edges = [0, *cuts, Skv]
    if masked:
        mask = (np.random.default_rng(seed + 3).random((B, Skv)) > 0.4).astype(np.uint8)
        mask[:, :edges[1]] = 0
        mask[:, -1] = 1
    print(f"[attn] accumulate B={B} H={H} Sq={Sq} Skv={Skv} D={D} cuts={cuts} masked={masked}", flush=True)
    qd = gu.to_dev(q)
    f = bf16.bits_to_f64
    qf, kf, vf = f(q), f(k), f(v)

    def chunk(a, b):
        kd = gu.to_dev(np.ascontiguousarray(k[:, a:b]))
        vd = gu.to_dev(np.ascontiguousarray(v[:, a:b]))
        md = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask[:, a:b])).to(gu.DEV)
        mk = None if mask is None else mask[:, a:b]
        return kd, vd, md, mk

    kd, vd, md, mk = chunk(edges[0], edges[1])
    st_o, st_l = cp.cp_attn_partial(qd, kd, vd, md)
    ref_o, ref_l = OA.attention_partial(qf, kf[:, :edges[1]], vf[:, :edges[1]], mk)
    for a, b in zip(edges[1:-2], edges[2:-1]):
        kd, vd, md, mk = chunk(a, b)
        cp.cp_attn_partial_accum(qd, kd, vd, st_o, st_l, md)
        ref_o, ref_l = OA.accumulate_partial(ref_o, ref_l, *OA.attention_partial(qf, kf[:, a:b], vf[:, a:b], mk))
    torch.cuda.synchronize()
    got_l = st_l.double().cpu().numpy()
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(got_l), fin)
    if fin.any():
        assert np.abs(got_l[fin] - ref_l[fin]).max() <= LSE_ERR
        rows = np.repeat(fin.transpose(0, 2, 1)[..., None], D, axis=3)
        _assert_close(st_o.double().cpu().numpy()[rows], ref_o[rows], "accumulated state")
    kd, vd, md, _ = chunk(edges[-2], edges[-1])
    before = st_o.clone()
    out = cp.cp_attn_partial_accum(qd, kd, vd, st_o, st_l, md, final=True)
    torch.cuda.synchronize()
    assert torch.equal(before, st_o), "the final call must leave the state unchanged"
    _assert_close(gu.to_f64(out), OA.attention(qf, kf, vf, mask), "accumulated final")
