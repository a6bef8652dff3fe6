"""Pins for the oracle's attention and the context-parallel rank layouts (CPU only).

The oracle is checked against things it does not contain: a pure-Python triple
loop, torch's scaled_dot_product_attention in float64, closed forms (Q = 0, one
valid key, constant V, a worked two-key example, the hard-max limit) and
invariants (key permutation, convex hull, the AllGather-KV and 2D rank layouts
reassembling single-rank attention).
"""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as A
from oracle import bf16
from oracle import cp_share


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _mask(B, S, seed, p=0.3):
    m = (np.random.default_rng(seed).random((B, S)) > p).astype(np.uint8)
    m[:, 0] = 1
    return m


# ----------------------------------------------------------------- brute force

@pytest.mark.parametrize("Sq,Skv", [(1, 1), (7, 65), (65, 7), (1, 130)])
@pytest.mark.parametrize("masked", [False, True])
def test_matches_triple_loop(Sq, Skv, masked):
    B, H, D = 2, 2, 4
    q, k, v = _rand((B, Sq, H, D), 1), _rand((B, Skv, H, D), 2), _rand((B, Skv, H, D), 3)
    m = _mask(B, Skv, 4) if masked else None
    got = A.attention(q, k, v, m, scale=0.7, chunk=3)
    ref = A.attention_loops(q, k, v, m, scale=0.7)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_config1_shape_matches_triple_loop_sampled_heads():
    wl = workloads.WORKLOADS["tiny_w2"]
    qf, kf, vf = (bf16.bits_to_f64(t) for t in workloads.global_qkv(wl))
    q = qf[:, :wl.attn_rows, :1]
    k, v = kf[:, :, :1], vf[:, :, :1]
    q = q[:, :6]
    got = A.attention(q, k, v)
    ref = A.attention_loops(q, k, v)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- library routine

@pytest.mark.parametrize("masked", [False, True])
def test_matches_torch_sdpa_float64(masked):
    B, Sq, Skv, H, D = 2, 33, 70, 3, 16
    q, k, v = _rand((B, Sq, H, D), 5), _rand((B, Skv, H, D), 6), _rand((B, Skv, H, D), 7)
    m = _mask(B, Skv, 8) if masked else None
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    am = None if m is None else torch.from_numpy(m != 0)[:, None, None, :]
    # scale=None on both sides: torch's default is 1/sqrt(D), which pins the oracle's default.
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am)
    got = A.attention(q, k, v, m)
    np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------- closed forms

def test_worked_two_key_example():
    # q = 1, keys 0 and ln 3, scale 1: weights 1/4 and 3/4; values 0 and 4 -> 3.
    q = np.ones((1, 1, 1, 1))
    k = np.array([0.0, math.log(3.0)]).reshape(1, 2, 1, 1)
    v = np.array([0.0, 4.0]).reshape(1, 2, 1, 1)
    assert A.attention(q, k, v, scale=1.0)[0, 0, 0, 0] == pytest.approx(3.0, abs=1e-14)
    # Masking the second key leaves only the first.
    m = np.array([[1, 0]], dtype=np.uint8)
    assert A.attention(q, k, v, m, scale=1.0)[0, 0, 0, 0] == 0.0
    m = np.array([[0, 1]], dtype=np.uint8)
    assert A.attention(q, k, v, m, scale=1.0)[0, 0, 0, 0] == pytest.approx(4.0, abs=1e-14)


@pytest.mark.parametrize("masked", [False, True])
def test_zero_query_gives_mean_of_valid_values(masked):
    B, Sq, Skv, H, D = 2, 5, 40, 3, 8
    q = np.zeros((B, Sq, H, D))
    k, v = _rand((B, Skv, H, D), 9), _rand((B, Skv, H, D), 10)
    m = _mask(B, Skv, 11) if masked else None
    got = A.attention(q, k, v, m)
    for b in range(B):
        valid = np.ones(Skv, bool) if m is None else m[b] != 0
        mean = v[b][valid].mean(axis=0)             # [H, D]
        for i in range(Sq):
            np.testing.assert_allclose(got[b, i], mean, rtol=1e-12, atol=1e-13)


def test_single_valid_key_returns_its_value():
    B, Sq, Skv, H, D = 2, 4, 9, 2, 8
    q, k, v = _rand((B, Sq, H, D), 12), _rand((B, Skv, H, D), 13), _rand((B, Skv, H, D), 14)
    m = np.zeros((B, Skv), np.uint8)
    m[0, 3] = 1
    m[1, 8] = 1
    got = A.attention(q, k, v, m)
    for i in range(Sq):
        np.testing.assert_allclose(got[0, i], v[0, 3], rtol=0, atol=1e-15)
        np.testing.assert_allclose(got[1, i], v[1, 8], rtol=0, atol=1e-15)


def test_constant_values_return_the_constant():
    B, Sq, Skv, H, D = 1, 6, 50, 2, 4
    q, k = _rand((B, Sq, H, D), 15), _rand((B, Skv, H, D), 16)
    c = np.array([0.5, -2.0, 3.25, 7.0])
    v = np.broadcast_to(c, (B, Skv, H, D)).copy()
    np.testing.assert_allclose(A.attention(q, k, v), np.broadcast_to(c, (B, Sq, H, D)),
                               rtol=1e-13, atol=1e-13)


def test_hard_max_limit_selects_the_best_key():
    # With a very large scale the softmax becomes a hard argmax; an oracle that did
    # not subtract the row maximum would overflow to inf/nan here.
    B, Sq, Skv, H, D = 1, 8, 30, 2, 16
    q, k, v = _rand((B, Sq, H, D), 17), _rand((B, Skv, H, D), 18), _rand((B, Skv, H, D), 19)
    got = A.attention(q, k, v, scale=1e4)
    assert np.isfinite(got).all()
    for i in range(Sq):
        for h in range(H):
            j = int(np.argmax(k[0, :, h] @ q[0, i, h]))
            np.testing.assert_allclose(got[0, i, h], v[0, j, h], rtol=0, atol=1e-9)


def test_fully_masked_batch_gives_zero_rows():
    q, k, v = _rand((2, 3, 1, 4), 20), _rand((2, 5, 1, 4), 21), _rand((2, 5, 1, 4), 22)
    m = np.ones((2, 5), np.uint8)
    m[1] = 0
    got = A.attention(q, k, v, m)
    assert (got[1] == 0).all() and np.isfinite(got).all()
    np.testing.assert_allclose(got[0], A.attention(q[:1], k[:1], v[:1])[0], rtol=1e-13)


# ----------------------------------------------------------------- invariants

def test_key_permutation_invariance():
    B, Sq, Skv, H, D = 2, 9, 77, 2, 8
    q, k, v = _rand((B, Sq, H, D), 23), _rand((B, Skv, H, D), 24), _rand((B, Skv, H, D), 25)
    m = _mask(B, Skv, 26)
    perm = np.random.default_rng(27).permutation(Skv)
    a = A.attention(q, k, v, m)
    b = A.attention(q, k[:, perm], v[:, perm], m[:, perm])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_output_in_convex_hull_of_valid_values():
    B, Sq, Skv, H, D = 2, 11, 64, 2, 8
    q, k, v = 3 * _rand((B, Sq, H, D), 28), _rand((B, Skv, H, D), 29), _rand((B, Skv, H, D), 30)
    m = _mask(B, Skv, 31)
    o = A.attention(q, k, v, m)
    for b in range(B):
        vv = v[b][m[b] != 0]
        lo, hi = vv.min(axis=0), vv.max(axis=0)
        assert (o[b] >= lo - 1e-12).all() and (o[b] <= hi + 1e-12).all()


def test_attention_rows_matches_full():
    B, Sq, Skv, H, D = 2, 10, 40, 3, 8
    q, k, v = _rand((B, Sq, H, D), 32), _rand((B, Skv, H, D), 33), _rand((B, Skv, H, D), 34)
    m = _mask(B, Skv, 35)
    full = A.attention(q, k, v, m)
    rows = [(0, 0, 0), (1, 9, 2), (1, 4, 1), (0, 7, 2)]
    got = A.attention_rows(q, k, v, rows, m)
    for n, (b, i, h) in enumerate(rows):
        np.testing.assert_allclose(got[n], full[b, i, h], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- rank layouts

@pytest.mark.parametrize("Ag", [2, 4])
def test_agkv_ranks_reassemble_full_attention(Ag):
    B, S, H, D = 2, 24, 3, 8
    q, k, v = _rand((B, S, H, D), 36), _rand((B, S, H, D), 37), _rand((B, S, H, D), 38)
    m = _mask(B, S, 39)
    outs = cp_share.agkv_outputs(q, k, v, Ag, m)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), A.attention(q, k, v, m),
                               rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("U,Ag", [(2, 2), (2, 3), (3, 2)])
@pytest.mark.parametrize("masked", [False, True])
def test_2d_ranks_reassemble_full_attention(U, Ag, masked):
    B, S, H, D = 2, 36, 6, 4
    q, k, v = _rand((B, S, H, D), 40), _rand((B, S, H, D), 41), _rand((B, S, H, D), 42)
    m = _mask(B, S, 43) if masked else None
    attn_in, outs = cp_share.composed_2d(q, k, v, U, Ag, m)
    full = A.attention(q, k, v, m)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), full, rtol=1e-12, atol=1e-13)
    # Rank (a, u): region a of heads u for Q; every key row of heads u for K and V.
    Hu, Sa = H // U, S // Ag
    for a in range(Ag):
        for u in range(U):
            g = a * U + u
            qa, ka, va = attn_in[g]
            np.testing.assert_array_equal(qa, q[:, a * Sa:(a + 1) * Sa, u * Hu:(u + 1) * Hu])
            np.testing.assert_array_equal(ka, k[:, :, u * Hu:(u + 1) * Hu])
            np.testing.assert_array_equal(va, v[:, :, u * Hu:(u + 1) * Hu])


@pytest.mark.parametrize("W", [2, 3])
@pytest.mark.parametrize("masked", [False, True])
def test_ulysses_attention_ranks_reassemble_full_attention(W, masked):
    # Every rank attends its head slice over the whole sequence between the two
    # exchanges; after the reverse exchange rank r holds rows r of full attention.
    B, S, H, D = 2, 30, 6, 4
    q, k, v = _rand((B, S, H, D), 44), _rand((B, S, H, D), 45), _rand((B, S, H, D), 46)
    m = _mask(B, S, 47) if masked else None
    recv, outs = cp_share.ulysses_attention_all(q, k, v, W, m)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), A.attention(q, k, v, m),
                               rtol=1e-12, atol=1e-13)
    # Rank j's send buffer, chunk r, is its heads' output for rows of rank r.
    Sl, Hl = S // W, H // W
    full = A.attention(q, k, v, m)
    for j in range(W):
        snd = cp_share.ulysses_attention_send(recv[j], B, W, m)
        for r in range(W):
            np.testing.assert_allclose(snd[r], full[:, r * Sl:(r + 1) * Sl, j * Hl:(j + 1) * Hl],
                                       rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("U", [2, 3])
@pytest.mark.parametrize("masked", [False, True])
def test_fused_2d_ranks_reassemble_full_attention(U, masked):
    # 2D layout, A = 2: each rank attends its Ulysses group's received rows over its
    # own region plus the other AllGather rank's region (region 0 first); after the
    # reverse exchange the ranks' outputs, in global rank order, are full attention,
    # the same as the gathered-K/V composition.
    B, S, H, D = 2, 24 * U, 2 * U, 4
    q, k, v = _rand((B, S, H, D), 54), _rand((B, S, H, D), 55), _rand((B, S, H, D), 56)
    m = _mask(B, S, 57) if masked else None
    ins, outs = cp_share.composed_2d_fused(q, k, v, U, m)
    full = A.attention(q, k, v, m)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), full, rtol=1e-12, atol=1e-13)
    _, outs_g = cp_share.composed_2d(q, k, v, U, 2, m)
    for a, b in zip(outs, outs_g):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    # the rank of region 1 takes the other region first; a rank of region 0 after
    assert [x[3] for x in ins] == [False] * U + [True] * U


def test_fused_2d_order_and_masks_enter_as_segments():
    # Swapping which range comes first changes nothing but the order of the keys
    # (attention is invariant under key permutation), and a mask part of zeros
    # removes that range: then the result is the own range's attention alone.
    B, W, Sl, Hl, D, So = 1, 2, 6, 2, 4, 9
    rng = np.random.default_rng(58)
    recv = rng.standard_normal((W, B * Sl, Hl, 3 * D))
    ko, vo = rng.standard_normal((B, So, Hl, D)), rng.standard_normal((B, So, Hl, D))
    a0 = cp_share.ulysses_2d_attention_send(recv, ko, vo, B, W, False)
    a1 = cp_share.ulysses_2d_attention_send(recv, ko, vo, B, W, True)
    np.testing.assert_allclose(a0, a1, rtol=1e-12, atol=1e-13)
    none = np.zeros((B, So), dtype=np.uint8)
    got = cp_share.ulysses_2d_attention_send(recv, ko, vo, B, W, True, None, none)
    np.testing.assert_allclose(got, cp_share.ulysses_attention_send(recv, B, W), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("cuts", [(7,), (1, 20), (5, 6, 30)])
def test_chunked_keys_merge_to_full_attention(masked, cuts):
    # attention over disjoint key chunks, merged by their log-sum-exp, is attention
    # over all keys; the lse of the whole equals the logsumexp of the chunks' lses
    B, Sq, Skv, H, D = 2, 9, 33, 2, 8
    q, k, v = _rand((B, Sq, H, D), 50), _rand((B, Skv, H, D), 51), _rand((B, Skv, H, D), 52)
    m = _mask(B, Skv, 53) if masked else None
    edges = [0, *cuts, Skv]
    parts = [A.attention_partial(q, k[:, a:b], v[:, a:b], None if m is None else m[:, a:b])
             for a, b in zip(edges[:-1], edges[1:])]
    o = A.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(o, A.attention(q, k, v, m), rtol=1e-12, atol=1e-13)
    _, lse_all = A.attention_partial(q, k, v, m)
    lses = np.stack([p[1] for p in parts])
    np.testing.assert_allclose(lse_all, np.logaddexp.reduce(lses, axis=0), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("masked", [False, True])
def test_folding_chunks_one_by_one_is_full_attention(masked):
    # state = partial(chunk 0); state = accumulate(state, partial(chunk i)) ... equals
    # attention and log-sum-exp over all keys; a leading fully masked chunk is a no-op
    B, Sq, Skv, H, D = 2, 6, 40, 2, 4
    q, k, v = _rand((B, Sq, H, D), 81), _rand((B, Skv, H, D), 82), _rand((B, Skv, H, D), 83)
    m = _mask(B, Skv, 84) if masked else np.ones((B, Skv), np.uint8)
    m[:, :5] = 0
    edges = [0, 5, 17, 18, 40]
    st_o, st_l = A.attention_partial(q, k[:, :5], v[:, :5], m[:, :5])
    assert np.all(st_l == -np.inf)
    for a, b in zip(edges[1:-1], edges[2:]):
        o_k, l_k = A.attention_partial(q, k[:, a:b], v[:, a:b], m[:, a:b])
        st_o, st_l = A.accumulate_partial(st_o, st_l, o_k, l_k)
    np.testing.assert_allclose(st_o, A.attention(q, k, v, m), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st_l, A.attention_partial(q, k, v, m)[1], rtol=1e-12, atol=1e-12)


def test_partial_lse_closed_forms():
    # Q = 0: every z = 0, so lse = ln(number of valid keys); one valid key: lse = its z
    B, Sq, Skv, H, D = 2, 3, 10, 1, 4
    k, v = _rand((B, Skv, H, D), 54), _rand((B, Skv, H, D), 55)
    m = np.ones((B, Skv), dtype=np.uint8)
    m[0, 4:] = 0
    _, lse = A.attention_partial(np.zeros((B, Sq, H, D)), k, v, m)
    np.testing.assert_allclose(lse[0], math.log(4), rtol=1e-14)
    np.testing.assert_allclose(lse[1], math.log(10), rtol=1e-14)
    q = _rand((B, Sq, H, D), 56)
    one = np.zeros((B, Skv), dtype=np.uint8)
    one[:, 6] = 1
    o, lse = A.attention_partial(q, k, v, one, scale=0.3)
    for b in range(B):
        for i in range(Sq):
            assert lse[b, 0, i] == pytest.approx(0.3 * float(q[b, i, 0] @ k[b, 6, 0]), rel=1e-13)
            np.testing.assert_allclose(o[b, i, 0], v[b, 6, 0], rtol=1e-14)


def test_partial_fully_masked_rows_and_merge():
    # a chunk with no valid key has lse = -inf and zero output, and the merge gives it
    # no weight; with no valid key in any chunk the merged row is zero
    B, Sq, Skv, H, D = 2, 2, 8, 1, 4
    q, k, v = _rand((B, Sq, H, D), 57), _rand((B, Skv, H, D), 58), _rand((B, Skv, H, D), 59)
    m = np.ones((B, Skv), dtype=np.uint8)
    m[0, :4] = 0
    m[1, :] = 0
    p1 = A.attention_partial(q, k[:, :4], v[:, :4], m[:, :4])
    p2 = A.attention_partial(q, k[:, 4:], v[:, 4:], m[:, 4:])
    assert np.all(p1[1][0] == -np.inf) and np.all(p1[0][0] == 0)
    o = A.merge_partials(np.stack([p1[0], p2[0]]), np.stack([p1[1], p2[1]]))
    np.testing.assert_allclose(o[0], p2[0][0], rtol=1e-14)
    assert np.all(o[1] == 0)


@pytest.mark.parametrize("W,H", [(4, 6), (4, 14), (3, 4)])
def test_uaa_padded_ranks_reassemble_full_attention(W, H):
    # zero padding heads attend to zero keys and values; dropping them after the
    # merge leaves every rank with its rows of full attention over the real heads
    B, S, D = 1, 12, 4
    q, k, v = _rand((B, S, H, D), 60), _rand((B, S, H, D), 61), _rand((B, S, H, D), 62)
    ins, outs = cp_share.uaa_attention_all(q, k, v, W)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), A.attention(q, k, v), rtol=1e-12, atol=1e-13)
    H_pad = -(-H // W) * W
    assert sum(x[0].shape[2] for x in ins) == H_pad


@pytest.mark.parametrize("front", [False, True])
def test_joint_segments_equal_attention_over_valid_keys_only(front):
    # masked keys contribute nothing: joint attention equals plain attention over the
    # valid image keys and valid text keys gathered by hand; front and rear agree
    B, Sq, S_img, T, H, D = 2, 5, 11, 6, 2, 4
    q = _rand((B, Sq, H, D), 70)
    ki, vi = _rand((B, S_img, H, D), 71), _rand((B, S_img, H, D), 72)
    kj, vj = _rand((B, T, H, D), 73), _rand((B, T, H, D), 74)
    im = _mask(B, S_img, 75)
    jm = np.ones((B, T), dtype=np.uint8)
    jm[0, 2:] = 0          # batch 0: two valid text tokens
    got = A.joint_attention(q, ki, vi, kj, vj, im, jm, joint_front=front)
    for b in range(B):
        kk = np.concatenate([ki[b][im[b] != 0], kj[b][jm[b] != 0]])[None]
        vv = np.concatenate([vi[b][im[b] != 0], vj[b][jm[b] != 0]])[None]
        np.testing.assert_allclose(got[b:b + 1], A.attention(q[b:b + 1], kk, vv), rtol=1e-12, atol=1e-13)
    other = A.joint_attention(q, ki, vi, kj, vj, im, jm, joint_front=not front)
    np.testing.assert_allclose(got, other, rtol=1e-12, atol=1e-13)


def test_joint_without_text_or_masks():
    B, Sq, S_img, T, H, D = 1, 3, 7, 4, 1, 4
    q, ki, vi = _rand((B, Sq, H, D), 76), _rand((B, S_img, H, D), 77), _rand((B, S_img, H, D), 78)
    np.testing.assert_allclose(A.joint_attention(q, ki, vi, None, None), A.attention(q, ki, vi),
                               rtol=1e-14)
    # all text masked out: only the image keys count
    kj, vj = _rand((B, T, H, D), 79), _rand((B, T, H, D), 80)
    np.testing.assert_allclose(A.joint_attention(q, ki, vi, kj, vj, None, np.zeros((B, T), np.uint8)),
                               A.attention(q, ki, vi), rtol=1e-12, atol=1e-13)


def test_bf16_widening_is_exact():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4049, 0x7F80, 0x0001, 0x7F7F],
                    dtype=np.uint16)
    got = bf16.bits_to_f64(bits)
    want = [0.0, -0.0, 1.0, -1.0, 3.140625, math.inf, 2.0 ** -133, 3.3895313892515355e38]
    assert list(got) == want
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got, t)
    # narrowing round trip and ties-to-even
    assert (bf16.f64_to_bits_rne(got[:6]) == bits[:6]).all()
    assert bf16.f64_to_bits_rne(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80      # tie -> even
    assert bf16.f64_to_bits_rne(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82  # tie -> even
