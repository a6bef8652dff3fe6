"""Packed variable-length attention on an AllGather-KV rank.  float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Packed metadata ([vllm-omni#7641], review-fix commit on packed query metadata):
several documents (requests) are concatenated along the sequence axis of one
batch row; ``cu_seqlens`` holds the n+1 cumulative boundaries, document i taking
rows ``[cu[i], cu[i+1])``.  Query document i attends to key document i only,
non-causally.

After the K/V all-gather each of the A ranks keeps the query rows
``[r*S/A, (r+1)*S/A)`` while the keys stay global.  The global query boundaries
are remapped by intersecting every document with the rank's span; each document
keeps exactly one (possibly empty) local entry so that query document i still
pairs with key document i, and the key boundaries are left global.

``remap_cu_seqlens_q`` is that intersection, written per document;
``varlen_attention`` is per-document softmax attention (one call of the plain
oracle per document and head group).

Readings where the pages are silent:
* query rows outside every document are left at zero;
* a document with query rows but no key rows gets zero outputs (the plain
  oracle's reading of a row without a valid key).
"""

from __future__ import annotations

import numpy as np

from . import attention as _attn


def remap_cu_seqlens_q(cu_q_global, rank, S_local):
    """Local query boundaries of AllGather-KV rank ``rank`` whose span is
    ``[s0, s1) = [rank*S_local, (rank+1)*S_local)``.  Document i, global rows
    ``[lo_i, hi_i)``, keeps the local rows ``[max(lo_i, s0), min(hi_i, s1)) - s0``,
    an empty range placed at the clamped position when the two do not meet, so
    every document keeps one entry and document i's local rows are exactly its
    rows inside the span."""
    cu = [int(x) for x in cu_q_global]
    s0, s1 = rank * S_local, (rank + 1) * S_local
    starts, ends = [], []
    for i in range(len(cu) - 1):
        lo, hi = cu[i], cu[i + 1]
        a = min(max(lo, s0), s1)          # intersection [a, b) of [lo, hi) with [s0, s1)
        b = max(min(hi, s1), a)
        starts.append(a - s0)
        ends.append(b - s0)
    # consecutive documents share a boundary: document i ends where i + 1 starts
    for i in range(len(starts) - 1):
        assert ends[i] == starts[i + 1]
    return np.asarray(starts + ends[-1:], dtype=np.int64)


def _check_cu(cu, total, name):
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] < 0 or (np.diff(cu) < 0).any() or cu[-1] > total:
        raise ValueError(f"{name}: expected non-decreasing boundaries within [0, {total}]")
    return cu


def varlen_attention(q, k, v, cu_q, cu_k, scale=None):
    """q ``[Sq, H, D]``, k and v ``[Skv, H, D]`` (one packed batch row); document i:
    queries ``[cu_q[i], cu_q[i+1])`` against keys ``[cu_k[i], cu_k[i+1])``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 3 or k.shape != v.shape or k.ndim != 3 or q.shape[1:] != k.shape[1:]:
        raise ValueError("expected q [Sq,H,D] and k, v [Skv,H,D]")
    cu_q = _check_cu(cu_q, q.shape[0], "cu_q")
    cu_k = _check_cu(cu_k, k.shape[0], "cu_k")
    if cu_q.size != cu_k.size:
        raise ValueError("cu_q and cu_k must describe the same documents")
    out = np.zeros_like(q)
    for i in range(cu_q.size - 1):
        q0, q1, k0, k1 = cu_q[i], cu_q[i + 1], cu_k[i], cu_k[i + 1]
        if q1 == q0 or k1 == k0:
            continue
        out[q0:q1] = _attn.attention(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], scale=scale)[0]
    return out


def agkv_varlen_outputs(q_full, k_full, v_full, cu_global, A, scale=None):
    """Every AllGather-KV rank's packed attention: rank r remaps the query
    boundaries to its span and attends its local rows over the global keys."""
    S = q_full.shape[0]
    if S % A:
        raise ValueError("S must divide by A")
    Sl = S // A
    outs = []
    for r in range(A):
        cu_l = remap_cu_seqlens_q(cu_global, r, Sl)
        outs.append(varlen_attention(q_full[r * Sl:(r + 1) * Sl], k_full, v_full, cu_l, cu_global, scale))
    return outs
