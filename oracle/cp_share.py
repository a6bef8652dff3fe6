"""Per-rank shares of context-parallel attention, composed from the oracle's steps.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Two layouts, from [vllm-omni#7641] (commit message):

* AllGather-KV over A ranks: rank r keeps query rows ``[r*S/A, (r+1)*S/A)`` and
  attends to the gathered global K/V of all heads.
* 2D, Ulysses degree U times AllGather-KV degree A (ring degree 1): global rank
  ``g = a*U + u``.  Ulysses groups are contiguous blocks of U ranks
  (group a = ranks ``a*U .. a*U+U-1``); AllGather-KV groups stride by U
  (group u = ranks ``u, u+U, u+2U, ...``).  Rank g starts with rows
  ``[g*S_l, (g+1)*S_l)``, ``S_l = S/(U*A)``, of all heads.  The Ulysses exchange
  inside group a leaves rank (a, u) with region a (rows ``[a*S/A, (a+1)*S/A)``) of
  heads ``[u*H/U, (u+1)*H/U)``; the K/V all-gather inside group u, in rank order,
  rebuilds every region of those heads in sequence order; attention is then a
  plain local-Q/global-KV problem; the reverse Ulysses step returns rank g's own
  rows with all heads.

The functions return every rank's result so that tests can check that the ranks'
outputs, concatenated in global rank order, equal single-rank attention.

A Ulysses rank's attention sits between its two exchanges ([sglang#33667],
usp.py excerpt and implementation breakdown): it unpacks the received staging
buffer into head-sharded Q/K/V, attends over the whole sequence for its H/W
heads, and lays the output out for the reverse exchange.  ``ulysses_attention_send``
is that composition, one step after the other.
"""

from __future__ import annotations

import numpy as np

from . import attention as _attn
from . import layout as _layout


def agkv_outputs(q_full, k_full, v_full, A, key_mask=None, scale=None):
    """Rank r of A: ``attention(Q rows of region r, all K, all V)``; list over ranks."""
    S = q_full.shape[1]
    if S % A:
        raise ValueError("S must divide by A")
    Sl = S // A
    return [_attn.attention(q_full[:, r * Sl:(r + 1) * Sl], k_full, v_full, key_mask, scale)
            for r in range(A)]


def ulysses_groups(U, A):
    return [[a * U + u for u in range(U)] for a in range(A)]


def agkv_groups(U, A):
    return [[u + k * U for k in range(A)] for u in range(U)]


def composed_2d(q_full, k_full, v_full, U, A, key_mask=None, scale=None):
    """Run the 2D layout on every rank.

    Returns ``(attn_inputs, outputs)``: ``attn_inputs[g] = (q, k, v)`` is the
    local-Q/global-KV problem rank g hands to attention, and ``outputs[g]`` is rank
    g's final ``[B, S_l, H, D]`` output after the reverse exchange.
    """
    B, S, H, D = q_full.shape
    P = U * A
    if S % P or H % U:
        raise ValueError("S must divide by U*A and H by U")
    Sl = S // P
    shard = [tuple(t[:, g * Sl:(g + 1) * Sl] for t in (q_full, k_full, v_full))
             for g in range(P)]

    after_ulysses = [None] * P
    for group in ulysses_groups(U, A):
        res = _layout.ulysses_forward([shard[g] for g in group], U)
        for u, g in enumerate(group):
            after_ulysses[g] = res[u]

    attn_inputs = [None] * P
    for group in agkv_groups(U, A):
        k_all = np.concatenate([after_ulysses[g][1] for g in group], axis=1)
        v_all = np.concatenate([after_ulysses[g][2] for g in group], axis=1)
        for g in group:
            attn_inputs[g] = (after_ulysses[g][0], k_all, v_all)

    o_hs = [_attn.attention(*attn_inputs[g], key_mask=key_mask, scale=scale) for g in range(P)]

    outputs = [None] * P
    for group in ulysses_groups(U, A):
        res = _layout.ulysses_reverse([o_hs[g] for g in group], U)
        for u, g in enumerate(group):
            outputs[g] = res[u]
    return attn_inputs, outputs


def ulysses_attention_send(recv, B, W, key_mask=None, scale=None):
    """One Ulysses rank between its exchanges: received ``[W, B*S_l, H_l, 3D]`` ->
    send layout ``[W, B, S_l, H_l, D]`` of the attention over all ``W*S_l`` rows
    (unpack, then attention, then the send step of the output reverse)."""
    q, k, v = _layout.unpack_head_sharded(recv, B, W)
    o = _attn.attention(q, k, v, key_mask=key_mask, scale=scale)
    return _layout.output_reverse_send(o, W)


def ulysses_2d_attention_send(recv, k_other, v_other, B, W, other_first=False, own_mask=None,
                              other_mask=None, scale=None):
    """One rank of the 2D layout with A = 2 between its Ulysses exchanges: the
    received ``[W, B*S_l, H_l, 3D]`` buffer of its own Ulysses group and the other
    AllGather rank's head-sharded ``k_other`` / ``v_other`` ``[B, S_o, H_l, D]`` ->
    send layout ``[W, B, S_l, H_l, D]`` of the attention of the rank's rows over
    both key ranges in sequence order (the other rank's region first when it holds
    the earlier one).  Masks: ``[B, W*S_l]`` over the own keys, ``[B, S_o]`` over
    the other rank's, None = attend."""
    q, k, v = _layout.unpack_head_sharded(recv, B, W)
    S, So = k.shape[1], k_other.shape[1]
    own = (k, v, own_mask, S)
    oth = (k_other, v_other, other_mask, So)
    first, second = (oth, own) if other_first else (own, oth)
    kk = np.concatenate([first[0], second[0]], axis=1)
    vv = np.concatenate([first[1], second[1]], axis=1)
    mask = None
    if own_mask is not None or other_mask is not None:
        parts = [np.ones((B, n), dtype=np.uint8) if m is None else np.asarray(m, dtype=np.uint8)
                 for (_, _, m, n) in (first, second)]
        mask = np.concatenate(parts, axis=1)
    o = _attn.attention(q, kk, vv, key_mask=mask, scale=scale)
    return _layout.output_reverse_send(o, W)


def composed_2d_fused(q_full, k_full, v_full, U, key_mask=None, scale=None):
    """The 2D layout with A = 2, every rank through ``ulysses_2d_attention_send``.

    Rank (a, u) receives its Ulysses group's exchange (region a, head slice u); the
    other AllGather rank of its group u is (1 - a, u), whose unpacked K/V (region
    1 - a, the same heads) it attends as well, region 0 first.  Returns
    ``(fused_inputs, outputs)``: ``fused_inputs[g] = (recv, k_other, v_other,
    other_first, own_mask, other_mask)`` and rank g's final ``[B, S_l, H, D]``."""
    A = 2
    B, S, H, D = q_full.shape
    P = U * A
    if S % P or H % U:
        raise ValueError("S must divide by 2U and H by U")
    Sl, Sr = S // P, S // A
    shard = [tuple(t[:, g * Sl:(g + 1) * Sl] for t in (q_full, k_full, v_full)) for g in range(P)]
    recv = [None] * P
    for group in ulysses_groups(U, A):
        r = _layout.exchange([_layout.pack_qkv_dst_major(*shard[g], U) for g in group])
        for u, g in enumerate(group):
            recv[g] = r[u]
    inputs, snd = [None] * P, [None] * P
    for a in range(A):
        for u in range(U):
            g, go = a * U + u, (1 - a) * U + u
            _, k_o, v_o = _layout.unpack_head_sharded(recv[go], B, U)
            own_m = None if key_mask is None else key_mask[:, a * Sr:(a + 1) * Sr]
            oth_m = None if key_mask is None else key_mask[:, (1 - a) * Sr:(2 - a) * Sr]
            inputs[g] = (recv[g], k_o, v_o, a == 1, own_m, oth_m)
            snd[g] = ulysses_2d_attention_send(recv[g], k_o, v_o, B, U, a == 1, own_m, oth_m, scale)
    outputs = [None] * P
    for group in ulysses_groups(U, A):
        rcv = _layout.exchange([snd[g] for g in group])
        for u, g in enumerate(group):
            outputs[g] = _layout.output_reverse_merge(rcv[u])
    return inputs, outputs


def ulysses_attention_all(q_full, k_full, v_full, W, key_mask=None, scale=None):
    """Every rank of one Ulysses group: pack, exchange, ``ulysses_attention_send``,
    exchange, merge.  Returns ``(recv, outputs)``: each rank's received staging
    buffer and its final ``[B, S_l, H, D]`` output (its own rows, all heads)."""
    B, S, H, D = q_full.shape
    if S % W or H % W:
        raise ValueError("S and H must divide by W")
    Sl = S // W
    shards = [tuple(t[:, r * Sl:(r + 1) * Sl] for t in (q_full, k_full, v_full)) for r in range(W)]
    recv = _layout.exchange([_layout.pack_qkv_dst_major(*shards[r], W) for r in range(W)])
    snd = [ulysses_attention_send(recv[j], B, W, key_mask, scale) for j in range(W)]
    rcv = _layout.exchange(snd)
    return recv, [_layout.output_reverse_merge(x) for x in rcv]


def uaa_attention_all(q_full, k_full, v_full, W, key_mask=None, scale=None):
    """Every rank of a Ulysses group whose degree W does not divide the head count:
    zero heads pad H up to a multiple of W before the pack, each rank attends its
    padded head slice, and the merge drops the padding.  Returns
    ``(per-rank attention inputs, per-rank outputs [B, S_l, H, D])``."""
    B, S, H, D = q_full.shape
    if S % W:
        raise ValueError("S must divide by W")
    H_pad = -(-H // W) * W
    Sl = S // W
    shards = [tuple(t[:, r * Sl:(r + 1) * Sl] for t in (q_full, k_full, v_full)) for r in range(W)]
    recv = _layout.exchange([_layout.pack_qkv_dst_major_padded(*shards[r], W, H_pad) for r in range(W)])
    ins = [_layout.unpack_head_sharded(recv[j], B, W) for j in range(W)]
    outs = [_attn.attention(q, k, v, key_mask=key_mask, scale=scale) for q, k, v in ins]
    rcv = _layout.exchange([_layout.output_reverse_send(o, W) for o in outs])
    return ins, [_layout.output_merge_cropped(x, H) for x in rcv]
