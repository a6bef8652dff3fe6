"""Pins for the oracle's layout maps (CPU only).

Each map is checked against a hand-worked fixture under tests/golden/, against its
own explicit-loop form, and end to end against the closed form of the pages' unit
test: after pack -> exchange -> unpack, rank j holds the sequence-concatenated
global tensor restricted to head slice j (sglang PR #33667 summary, "Key source
snippets", test_usp_packed_qkv_a2a.py excerpt).
"""

import os

import numpy as np
import pytest

import workloads
from oracle import layout


def _read_golden(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line)
    return rows


# ----------------------------------------------------------------- exchange

@pytest.mark.parametrize("name", ["exchange_w2.txt", "exchange_w3.txt"])
def test_exchange_golden(golden_dir, name):
    sends, recvs = {}, {}
    for line in _read_golden(os.path.join(golden_dir, name)):
        head, vals = line.split(":")
        kind, idx = head.split()
        arr = np.array([int(x) for x in vals.split()], dtype=np.int64)
        (sends if kind == "send" else recvs)[int(idx)] = arr
    W = len(sends)
    got = layout.exchange([sends[r] for r in range(W)])
    for j in range(W):
        np.testing.assert_array_equal(got[j], recvs[j])
    got2 = layout.exchange_loops([sends[r] for r in range(W)])
    for j in range(W):
        np.testing.assert_array_equal(got2[j], recvs[j])


@pytest.mark.parametrize("W,shape", [(2, (2, 3, 4)), (3, (3, 2, 5)), (4, (8, 3))])
def test_exchange_matches_loops(W, shape):
    rng = np.random.default_rng(7)
    sends = [rng.integers(0, 60000, size=shape).astype(np.uint16) for _ in range(W)]
    a = layout.exchange(sends)
    b = layout.exchange_loops(sends)
    for j in range(W):
        np.testing.assert_array_equal(a[j], b[j])


def test_exchange_is_an_involution_on_equal_chunks():
    # Applying the chunk exchange twice returns every rank's buffer.
    rng = np.random.default_rng(3)
    sends = [rng.integers(0, 1000, size=12) for _ in range(4)]
    back = layout.exchange(layout.exchange(sends))
    for r in range(4):
        np.testing.assert_array_equal(back[r], sends[r])


# ----------------------------------------------------------------- pack / unpack goldens

def _coded_inputs(B, Sl, H, D):
    x = []
    for c in range(3):
        t = np.zeros((B, Sl, H, D), dtype=np.int64)
        for b in range(B):
            for s in range(Sl):
                for h in range(H):
                    for d in range(D):
                        t[b, s, h, d] = c * 10000 + b * 1000 + s * 100 + h * 10 + d
        x.append(t)
    return x


def test_pack_golden(golden_dir):
    q, k, v = _coded_inputs(2, 2, 4, 2)
    expect = np.zeros((2, 4, 2, 6), dtype=np.int64)
    for line in _read_golden(os.path.join(golden_dir, "pack_w2_b2.txt")):
        idx, vals = line.split(":")
        j, row, hl = (int(x) for x in idx.split())
        expect[j, row, hl] = [int(x) for x in vals.split()]
    np.testing.assert_array_equal(layout.pack_qkv_dst_major(q, k, v, 2), expect)
    np.testing.assert_array_equal(layout.pack_qkv_dst_major_loops(q, k, v, 2), expect)


def test_unpack_golden(golden_dir):
    W, B, Sl, Hl, D = 2, 2, 2, 2, 2
    recv = np.zeros((W, B * Sl, Hl, 3 * D), dtype=np.int64)
    for r in range(W):
        for row in range(B * Sl):
            for hl in range(Hl):
                for e in range(3 * D):
                    recv[r, row, hl, e] = r * 1000 + row * 100 + hl * 10 + e
    expect = np.zeros((3, B, W * Sl, Hl, D), dtype=np.int64)
    for line in _read_golden(os.path.join(golden_dir, "unpack_w2_b2.txt")):
        idx, vals = line.split(":")
        c, b, t, hl = (int(x) for x in idx.split())
        expect[c, b, t, hl] = [int(x) for x in vals.split()]
    got = layout.unpack_head_sharded(recv, B, W)
    got2 = layout.unpack_head_sharded_loops(recv, B, W)
    for c in range(3):
        np.testing.assert_array_equal(got[c], expect[c])
        np.testing.assert_array_equal(got2[c], expect[c])


def test_reverse_send_golden(golden_dir):
    W, B, Sl, Hl, D = 2, 2, 2, 1, 2
    o = np.zeros((B, W * Sl, Hl, D), dtype=np.int64)
    for b in range(B):
        for t in range(W * Sl):
            for hl in range(Hl):
                for d in range(D):
                    o[b, t, hl, d] = b * 1000 + t * 100 + hl * 10 + d
    expect = np.zeros((W, B, Sl, Hl, D), dtype=np.int64)
    for line in _read_golden(os.path.join(golden_dir, "reverse_send_w2_b2.txt")):
        idx, vals = line.split(":")
        r, b, s = (int(x) for x in idx.split())
        expect[r, b, s, 0] = [int(x) for x in vals.split()]
    np.testing.assert_array_equal(layout.output_reverse_send(o, W), expect)
    np.testing.assert_array_equal(layout.output_reverse_send_loops(o, W), expect)


def test_reverse_merge_golden(golden_dir):
    W, B, Sl, Hl, D = 2, 2, 2, 2, 1
    rcv = np.zeros((W, B, Sl, Hl, D), dtype=np.int64)
    for j in range(W):
        for b in range(B):
            for s in range(Sl):
                for hl in range(Hl):
                    rcv[j, b, s, hl, 0] = j * 1000 + b * 100 + s * 10 + hl
    expect = np.zeros((B, Sl, W * Hl, D), dtype=np.int64)
    for line in _read_golden(os.path.join(golden_dir, "reverse_merge_w2_b2.txt")):
        idx, vals = line.split(":")
        b, s = (int(x) for x in idx.split())
        expect[b, s, :, 0] = [int(x) for x in vals.split()]
    np.testing.assert_array_equal(layout.output_reverse_merge(rcv), expect)
    np.testing.assert_array_equal(layout.output_reverse_merge_loops(rcv), expect)


# ----------------------------------------------------------------- loops vs reshape, random

@pytest.mark.parametrize("W,B,Sl,H,D", [(2, 1, 3, 4, 2), (3, 2, 2, 6, 3), (4, 3, 1, 4, 1)])
def test_pack_unpack_reverse_match_loops(W, B, Sl, H, D):
    rng = np.random.default_rng(11)
    q, k, v = (rng.integers(0, 65535, size=(B, Sl, H, D)).astype(np.uint16) for _ in range(3))
    st = layout.pack_qkv_dst_major(q, k, v, W)
    np.testing.assert_array_equal(st, layout.pack_qkv_dst_major_loops(q, k, v, W))
    a = layout.unpack_head_sharded(st, B, W)
    b = layout.unpack_head_sharded_loops(st, B, W)
    for c in range(3):
        np.testing.assert_array_equal(a[c], b[c])
    o = rng.integers(0, 65535, size=(B, W * Sl, H // W, D)).astype(np.uint16)
    np.testing.assert_array_equal(layout.output_reverse_send(o, W),
                                  layout.output_reverse_send_loops(o, W))
    rcv = rng.integers(0, 65535, size=(W, B, Sl, H // W, D)).astype(np.uint16)
    np.testing.assert_array_equal(layout.output_reverse_merge(rcv),
                                  layout.output_reverse_merge_loops(rcv))


# ----------------------------------------------------------------- end-to-end spec

def _forward_spec_check(full, W):
    B, S, H, D = full[0].shape
    Sl, Hl = S // W, H // W
    shards = [tuple(np.ascontiguousarray(t[:, r * Sl:(r + 1) * Sl]) for t in full)
              for r in range(W)]
    out = layout.ulysses_forward(shards, W)
    for j in range(W):
        for c in range(3):
            spec = full[c][:, :, j * Hl:(j + 1) * Hl]
            np.testing.assert_array_equal(out[j][c], spec)
    return shards, out


@pytest.mark.parametrize("W,B,S,H,D", workloads.PAGE_TEST_SHAPES)
def test_forward_spec_page_shapes(W, B, S, H, D):
    full = workloads.page_test_tensors(B, S, H, D)
    _forward_spec_check(full, W)


@pytest.mark.parametrize("name", ["tiny_w2", "image_cp4", "image_cp8", "joint_cfg_cp4"])
def test_forward_spec_and_round_trip_workloads(name):
    wl = workloads.WORKLOADS[name]
    full = workloads.global_qkv(wl)
    # The Ulysses group of global rank 0 covers rows [0, W*S_l) of all heads.
    span = wl.W * wl.S_local
    full = [np.ascontiguousarray(t[:, :span]) for t in full]
    shards, out = _forward_spec_check(full, wl.W)
    # Reverse applied to each head-sharded tensor returns every rank's shard.
    for c in range(3):
        back = layout.ulysses_reverse([out[j][c] for j in range(wl.W)], wl.W)
        for r in range(wl.W):
            np.testing.assert_array_equal(back[r], shards[r][c])


def test_forward_spec_video_2d_group0():
    wl = workloads.WORKLOADS["video_u2a2"]
    full = workloads.global_qkv(wl)
    span = wl.W * wl.S_local
    full = [np.ascontiguousarray(t[:, :span]) for t in full]
    _forward_spec_check(full, wl.W)


@pytest.mark.parametrize("W,S,H,D", [(2, 8, 4, 4), (4, 16, 8, 2), (8, 16, 8, 8)])
def test_b1_receive_buffer_is_sequence_major(W, S, H, D):
    # For B == 1 the received buffer, read as [1, W*S_l, H_l, 3D], already is the
    # unpacked result: unpack only splits the last axis (usp.py excerpt, B == 1 branch).
    rng = np.random.default_rng(5)
    full = [rng.integers(0, 65535, size=(1, S, H, D)).astype(np.uint16) for _ in range(3)]
    Sl, Hl = S // W, H // W
    shards = [tuple(t[:, r * Sl:(r + 1) * Sl] for t in full) for r in range(W)]
    recv = layout.exchange([layout.pack_qkv_dst_major(*s, W) for s in shards])
    for j in range(W):
        view = recv[j].reshape(1, W * Sl, Hl, 3 * D)
        out = layout.unpack_head_sharded(recv[j], 1, W)
        for c in range(3):
            np.testing.assert_array_equal(out[c], view[..., c * D:(c + 1) * D])


def test_reverse_send_is_identity_layout_for_b1():
    rng = np.random.default_rng(9)
    o = rng.integers(0, 65535, size=(1, 12, 3, 4)).astype(np.uint16)
    np.testing.assert_array_equal(layout.output_reverse_send(o, 3).reshape(-1), o.reshape(-1))


def test_layout_rejects_indivisible_shapes():
    q = np.zeros((1, 2, 3, 4), dtype=np.uint16)
    with pytest.raises(ValueError):
        layout.pack_qkv_dst_major(q, q, q, 2)
    with pytest.raises(ValueError):
        layout.exchange([np.zeros(3), np.zeros(3)])
    with pytest.raises(ValueError):
        layout.output_reverse_send(np.zeros((1, 3, 1, 1)), 2)


# ----------------------------------------------------------------- head padding

def _pack_padded_loops(q, k, v, W, H_pad):
    """The padded pack written element by element from its definition."""
    B, Sl, H, D = q.shape
    Hl = H_pad // W
    out = np.zeros((W, B * Sl, Hl, 3 * D), dtype=q.dtype)
    for j in range(W):
        for b in range(B):
            for s in range(Sl):
                for hl in range(Hl):
                    g = j * Hl + hl
                    if g >= H:
                        continue
                    for c, t in enumerate((q, k, v)):
                        for d in range(D):
                            out[j, b * Sl + s, hl, c * D + d] = t[b, s, g, d]
    return out


@pytest.mark.parametrize("W,B,Sl,H,H_pad,D", [(4, 1, 3, 14, 16, 2), (3, 2, 2, 4, 6, 3), (2, 1, 2, 3, 4, 1)])
def test_padded_pack_matches_loops(W, B, Sl, H, H_pad, D):
    rng = np.random.default_rng(W * 100 + H)
    q, k, v = (rng.integers(1, 65535, size=(B, Sl, H, D)).astype(np.uint16) for _ in range(3))
    np.testing.assert_array_equal(layout.pack_qkv_dst_major_padded(q, k, v, W, H_pad),
                                  _pack_padded_loops(q, k, v, W, H_pad))


def test_padded_pack_without_padding_is_the_plain_pack():
    rng = np.random.default_rng(3)
    q, k, v = (rng.integers(0, 65535, size=(2, 3, 8, 4)).astype(np.uint16) for _ in range(3))
    np.testing.assert_array_equal(layout.pack_qkv_dst_major_padded(q, k, v, 4, 8),
                                  layout.pack_qkv_dst_major(q, k, v, 4))


@pytest.mark.parametrize("W,B,S,H,D", [(4, 1, 16, 14, 4), (4, 2, 8, 6, 2), (3, 2, 12, 4, 3)])
def test_padded_forward_spec_and_cropped_round_trip(W, B, S, H, D):
    # After padded pack -> exchange -> unpack, rank j holds global heads
    # [j*H_l, (j+1)*H_l) of the sequence-concatenated tensor, zeros past H; the
    # reverse with the cropped merge returns every rank's original shard.
    rng = np.random.default_rng(S + H)
    full = [rng.integers(1, 65535, size=(B, S, H, D)).astype(np.uint16) for _ in range(3)]
    H_pad = -(-H // W) * W
    Hl, Sl = H_pad // W, S // W
    shards = [tuple(t[:, r * Sl:(r + 1) * Sl] for t in full) for r in range(W)]
    recv = layout.exchange([layout.pack_qkv_dst_major_padded(*sh, W, H_pad) for sh in shards])
    outs = [layout.unpack_head_sharded(recv[j], B, W) for j in range(W)]
    padded = [np.pad(t, [(0, 0), (0, 0), (0, H_pad - H), (0, 0)]) for t in full]
    for j in range(W):
        for c in range(3):
            np.testing.assert_array_equal(outs[j][c], padded[c][:, :, j * Hl:(j + 1) * Hl])
    for c in range(3):
        rcv = layout.exchange([layout.output_reverse_send(outs[j][c], W) for j in range(W)])
        for r in range(W):
            np.testing.assert_array_equal(layout.output_merge_cropped(rcv[r], H), shards[r][c])
