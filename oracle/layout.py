"""Ulysses layout exchange: pack, chunk exchange, unpack and output reverse.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Each map is written twice: once as a reshape/transpose (``*`` functions, any size)
and once as explicit element loops (``*_loops``, tiny inputs only).  Arrays may be
of any dtype; the tests feed uint16 bf16 bit patterns so equality is bitwise.

Notation: ``W`` ranks in the Ulysses group, ``B`` batch, ``S_l`` rows per rank,
``H = W * H_l`` heads, ``D`` head dim, ``rows = B * S_l``.

Definitions, from [sglang#33667] ("Key source snippets", usp.py excerpt of
``_usp_input_all_to_all_qkv`` and the unit-test excerpt):

* pack: each of Q/K/V is viewed as ``[rows, H, D]`` and written into one staging
  buffer of shape ``[W, rows, H_l, 3D]``; destination rank ``j`` receives head
  slice ``j`` and the last axis is ``[q | k | v]`` (the receiver splits it by ``D``
  in that order);
* exchange: a single all-to-all-single over the flattened staging buffer; the
  unit test reproduces it with a fake collective under which the chunk ``j`` that
  rank ``r`` sends becomes the ``r``-th chunk that rank ``j`` receives;
* unpack: the received ``[W, rows, H_l, 3D]`` buffer is ``[W, B, S_l, H_l, 3D]``;
  moving the source-rank axis next to the sequence axis gives
  ``[B, W*S_l, H_l, 3D]`` (for ``B == 1`` that is a plain view), then the last
  axis is split into q, k, v;
* end to end: rank ``j`` ends with the sequence-concatenated global tensor
  restricted to heads ``[j*H_l, (j+1)*H_l)``.

The output reverse is only named on the pages (``_usp_output_all_to_all`` in the
implementation breakdown of [sglang#33667]; the reverse Ulysses step in the
commit message of [vllm-omni#7641]).  Reading taken: it is the exact inverse of
the forward exchange, with the same flat-chunk collective, so the sender must
lay its head-sharded output out destination-major as ``[W, B, S_l, H_l, D]``
(send phase) and the receiver interleaves the W head groups back into full heads
(merge phase).
"""

from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------- exchange

def exchange(sends):
    """Flat-chunk all-to-all: ``recv[j] = concat_r chunk_j(flatten(send[r]))``.

    ``sends`` is a list of W arrays of equal shape and size N (N % W == 0).  Each
    returned array has the shape of the sends.  [sglang#33667], unit-test excerpt
    (the fake collective's replay rule).
    """
    W = len(sends)
    shape = sends[0].shape
    flat = [np.ascontiguousarray(s).reshape(-1) for s in sends]
    N = flat[0].size
    if any(f.size != N for f in flat) or N % W:
        raise ValueError("exchange needs W equal buffers whose size divides by W")
    c = N // W
    return [np.concatenate([flat[r][j * c:(j + 1) * c] for r in range(W)]).reshape(shape)
            for j in range(W)]


def exchange_loops(sends):
    """Element-by-element form of :func:`exchange` (tiny inputs only)."""
    W = len(sends)
    shape = sends[0].shape
    flat = [list(np.ascontiguousarray(s).reshape(-1)) for s in sends]
    N = len(flat[0])
    c = N // W
    out = []
    for j in range(W):
        buf = [None] * N
        for r in range(W):
            for e in range(c):
                buf[r * c + e] = flat[r][j * c + e]
        out.append(np.array(buf, dtype=sends[0].dtype).reshape(shape))
    return out


# --------------------------------------------------------------------------- pack

def pack_qkv_dst_major(q, k, v, W):
    """``staging[j, b*S_l+s, hl, c*D+d] = X_c[b, s, j*H_l+hl, d]`` for c = q, k, v.

    Inputs ``[B, S_l, H, D]``; output ``[W, B*S_l, H/W, 3D]``.  [sglang#33667],
    implementation breakdown item 3 and the usp.py excerpt.
    """
    B, Sl, H, D = q.shape
    if H % W:
        raise ValueError("H must divide by W")
    Hl = H // W
    rows = B * Sl
    x = np.stack([np.asarray(t).reshape(rows, W, Hl, D) for t in (q, k, v)])  # [3,rows,W,Hl,D]
    return np.ascontiguousarray(x.transpose(2, 1, 3, 0, 4)).reshape(W, rows, Hl, 3 * D)


def pack_qkv_dst_major_loops(q, k, v, W):
    B, Sl, H, D = q.shape
    Hl = H // W
    out = np.zeros((W, B * Sl, Hl, 3 * D), dtype=q.dtype)
    src = (q, k, v)
    for j in range(W):
        for b in range(B):
            for s in range(Sl):
                for hl in range(Hl):
                    for c in range(3):
                        for d in range(D):
                            out[j, b * Sl + s, hl, c * D + d] = src[c][b, s, j * Hl + hl, d]
    return out


# --------------------------------------------------------------------------- unpack

def unpack_head_sharded(recv, B, W):
    """``out_c[b, r*S_l+s, hl, d] = recv[r, b*S_l+s, hl, c*D+d]``; returns (q, k, v).

    ``recv`` is ``[W, B*S_l, H_l, 3D]``; each output is ``[B, W*S_l, H_l, D]``.
    [sglang#33667], usp.py excerpt (view for B == 1, source-rank/batch permute for
    B > 1, then a split of the last axis by D).
    """
    W_, rows, Hl, D3 = recv.shape
    if W_ != W or rows % B or D3 % 3:
        raise ValueError("recv shape does not match W/B")
    Sl, D = rows // B, D3 // 3
    x = np.asarray(recv).reshape(W, B, Sl, Hl, 3, D).transpose(4, 1, 0, 2, 3, 5)
    x = np.ascontiguousarray(x).reshape(3, B, W * Sl, Hl, D)
    return x[0].copy(), x[1].copy(), x[2].copy()


def unpack_head_sharded_loops(recv, B, W):
    _, rows, Hl, D3 = recv.shape
    Sl, D = rows // B, D3 // 3
    outs = [np.zeros((B, W * Sl, Hl, D), dtype=recv.dtype) for _ in range(3)]
    for r in range(W):
        for b in range(B):
            for s in range(Sl):
                for hl in range(Hl):
                    for c in range(3):
                        for d in range(D):
                            outs[c][b, r * Sl + s, hl, d] = recv[r, b * Sl + s, hl, c * D + d]
    return tuple(outs)


# --------------------------------------------------------------------------- output reverse

def output_reverse_send(o, W):
    """Send layout ``snd[r, b, s, hl, d] = O[b, r*S_l+s, hl, d]``.

    ``o`` is the head-sharded output ``[B, W*S_l, H_l, D]``; result
    ``[W, B, S_l, H_l, D]``.  For B == 1 this is the identity on memory.
    """
    B, S, Hl, D = o.shape
    if S % W:
        raise ValueError("sequence must divide by W")
    Sl = S // W
    return np.ascontiguousarray(np.asarray(o).reshape(B, W, Sl, Hl, D).transpose(1, 0, 2, 3, 4))


def output_reverse_merge(rcv):
    """Merge ``out[b, s, j*H_l+hl, d] = rcv[j, b, s, hl, d]``: ``[W,B,S_l,H_l,D] -> [B,S_l,W*H_l,D]``."""
    W, B, Sl, Hl, D = rcv.shape
    return np.ascontiguousarray(np.asarray(rcv).transpose(1, 2, 0, 3, 4)).reshape(B, Sl, W * Hl, D)


def output_reverse_send_loops(o, W):
    B, S, Hl, D = o.shape
    Sl = S // W
    out = np.zeros((W, B, Sl, Hl, D), dtype=o.dtype)
    for r in range(W):
        for b in range(B):
            for s in range(Sl):
                for hl in range(Hl):
                    for d in range(D):
                        out[r, b, s, hl, d] = o[b, r * Sl + s, hl, d]
    return out


def output_reverse_merge_loops(rcv):
    W, B, Sl, Hl, D = rcv.shape
    out = np.zeros((B, Sl, W * Hl, D), dtype=rcv.dtype)
    for j in range(W):
        for b in range(B):
            for s in range(Sl):
                for hl in range(Hl):
                    for d in range(D):
                        out[b, s, j * Hl + hl, d] = rcv[j, b, s, hl, d]
    return out


# ------------------------------------------------------------------ head padding
#
# Head counts the Ulysses degree does not divide ([vllm-omni#7641], attention
# benchmark: 14 heads over 4 ranks run as 16, "+14.3% attention work"): the head
# axis is padded with zero heads to a multiple of W before the pack, and the
# padding heads are dropped after the merge.


def pack_qkv_dst_major_padded(q, k, v, W, H_pad):
    """Pack of Q/K/V whose head axis is first padded with zero heads up to ``H_pad``."""
    H = q.shape[2]
    if H_pad < H or H_pad % W:
        raise ValueError("H_pad must be >= H and divide by W")
    pad = [(0, 0), (0, 0), (0, H_pad - H), (0, 0)]
    return pack_qkv_dst_major(*(np.pad(t, pad) for t in (q, k, v)), W)


def output_merge_cropped(rcv, H):
    """Merge of the received output chunks, keeping the first ``H`` heads."""
    return output_reverse_merge(rcv)[:, :, :H, :]


# --------------------------------------------------------------------------- composed

def ulysses_forward(shards, W):
    """All W ranks: pack -> exchange -> unpack.

    ``shards[r] = (q, k, v)``, each ``[B, S_l, H, D]``; returns per-rank head-sharded
    ``(q, k, v)``, each ``[B, W*S_l, H/W, D]``.
    """
    B = shards[0][0].shape[0]
    staged = [pack_qkv_dst_major(*shards[r], W) for r in range(W)]
    recv = exchange(staged)
    return [unpack_head_sharded(recv[j], B, W) for j in range(W)]


def ulysses_reverse(outs, W):
    """All W ranks: send layout -> exchange -> merge.  ``outs[r]`` is ``[B, W*S_l, H_l, D]``."""
    snd = [output_reverse_send(o, W) for o in outs]
    rcv = exchange(snd)
    return [output_reverse_merge(x) for x in rcv]
