"""Non-causal multi-head attention, local queries against global keys.  float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed, per batch b, head h and query row i (inputs ``[B, S, H, D]``):

    z_ij  = scale * sum_d q[b,i,h,d] * k[b,j,h,d]
    V_b   = { j : key_mask[b, j] != 0 }          (all keys when there is no mask)
    o_i   = sum_{j in V_b} exp(z_ij - m_i) v[b,j,h,:] / sum_{j in V_b} exp(z_ij - m_i),
    m_i   = max_{j in V_b} z_ij.

The attention form is the one the AllGather-KV path hands to its backend: every
rank keeps its own query rows and attends, non-causally, over the gathered
global K/V of the same heads ([vllm-omni#7641], commit message; MHA only,
[chitu-fastcp] "Support scope").  The key mask is the 2D ``[B, K]``
key-validity mask of [vllm-omni#7641]'s review-fix commits, where True means
"attend"; here it is uint8 with nonzero meaning valid.

Readings where the pages are silent:
* ``scale`` defaults to 1/sqrt(D);
* a query whose batch has no valid key gets an all-zero output row (the pages
  never produce one; the synthetic workloads never do either).

The oracle subtracts the row maximum before exponentiating (a rounding device
only: the quotient is unchanged in exact arithmetic) and works on row chunks so
that large shapes fit in memory.  There is no other blocking or reordering.
"""

from __future__ import annotations

import math

import numpy as np


def _check(q, k, v, key_mask):
    if q.ndim != 4 or k.shape != v.shape or q.shape[0] != k.shape[0] \
            or q.shape[2:] != k.shape[2:]:
        raise ValueError("expected q [B,Sq,H,D] and k, v [B,Skv,H,D]")
    if key_mask is not None and key_mask.shape != (k.shape[0], k.shape[1]):
        raise ValueError("key_mask must be [B, Skv]")


def attention(q, k, v, key_mask=None, scale=None, chunk=256):
    """softmax(scale * Q K^T) V over valid keys; float64 in and out, ``[B, Sq, H, D]``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _check(q, k, v, key_mask)
    B, Sq, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Sq, H, D), dtype=np.float64)
    for b in range(B):
        valid = np.ones(k.shape[1], dtype=bool) if key_mask is None else (key_mask[b] != 0)
        if not valid.any():
            continue
        for h in range(H):
            kb = k[b][valid, h, :]            # [Kv, D]
            vb = v[b][valid, h, :]
            for i0 in range(0, Sq, chunk):
                z = scale * (q[b, i0:i0 + chunk, h, :] @ kb.T)   # [chunk, Kv]
                z -= z.max(axis=1, keepdims=True)
                e = np.exp(z)
                out[b, i0:i0 + chunk, h, :] = (e @ vb) / e.sum(axis=1, keepdims=True)
    return out


def attention_rows(q, k, v, rows, key_mask=None, scale=None):
    """Selected outputs one by one: ``rows`` is a list of (b, i, h); returns ``[n, D]``.

    Used at full workload sizes where the whole output is too costly on the CPU.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    D = q.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    res = np.zeros((len(rows), D), dtype=np.float64)
    for n, (b, i, h) in enumerate(rows):
        valid = np.ones(k.shape[1], dtype=bool) if key_mask is None else (key_mask[b] != 0)
        if not valid.any():
            continue
        kb = np.asarray(k[b][valid, h, :], dtype=np.float64)
        vb = np.asarray(v[b][valid, h, :], dtype=np.float64)
        z = scale * (kb @ np.asarray(q[b, i, h, :], dtype=np.float64))
        e = np.exp(z - z.max())
        res[n] = (e @ vb) / e.sum()
    return res


def attention_loops(q, k, v, key_mask=None, scale=None):
    """Pure-Python triple loop of the definition above (tiny inputs only)."""
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Sq, H, D), dtype=np.float64)
    for b in range(B):
        keys = [j for j in range(Skv) if key_mask is None or key_mask[b, j] != 0]
        for h in range(H):
            for i in range(Sq):
                if not keys:
                    continue
                z = []
                for j in keys:
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[b, i, h, d]) * float(k[b, j, h, d])
                    z.append(scale * acc)
                m = max(z)
                w = [math.exp(x - m) for x in z]
                den = sum(w)
                for d in range(D):
                    num = 0.0
                    for wj, j in zip(w, keys):
                        num += wj * float(v[b, j, h, d])
                    out[b, i, h, d] = num / den
    return out


# ------------------------------------------------ attention over key chunks, merged
#
# Attention over keys that arrive in chunks ([chitu-fastcp] FAQ and section 5: a
# forward over each K/V chunk that also returns the log-sum-exp, then a merge;
# [vllm-omni#7641]'s follow-up note on overlapping the K/V gather the same way):
#
#   lse_i  = ln sum_{j in V_b} exp(z_ij)                (-inf when V_b is empty)
#   o_i    = sum_{j in V_b} exp(z_ij - lse_i) v_j        (zeros when V_b is empty)
#
# and for parts k = 1..N over disjoint key sets, with L_i = ln sum_k exp(lse_k,i):
#
#   o_i    = sum_k exp(lse_k,i - L_i) o_k,i              (zeros when every lse_k,i = -inf)
#
# which equals attention over the union of the keys.


def attention_partial(q, k, v, key_mask=None, scale=None, chunk=256):
    """Normalised output ``[B, Sq, H, D]`` and ``lse`` ``[B, H, Sq]`` (natural log) over these keys."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _check(q, k, v, key_mask)
    B, Sq, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Sq, H, D), dtype=np.float64)
    lse = np.full((B, H, Sq), -np.inf, dtype=np.float64)
    for b in range(B):
        valid = np.ones(k.shape[1], dtype=bool) if key_mask is None else (key_mask[b] != 0)
        if not valid.any():
            continue
        for h in range(H):
            kb = k[b][valid, h, :]
            vb = v[b][valid, h, :]
            for i0 in range(0, Sq, chunk):
                z = scale * (q[b, i0:i0 + chunk, h, :] @ kb.T)
                m = z.max(axis=1, keepdims=True)
                e = np.exp(z - m)
                s = e.sum(axis=1, keepdims=True)
                out[b, i0:i0 + chunk, h, :] = (e @ vb) / s
                lse[b, h, i0:i0 + chunk] = (m + np.log(s))[:, 0]
    return out, lse


def accumulate_partial(state_o, state_lse, o_k, lse_k):
    """Running state after one more key chunk: the merge of two partial results, as
    ``(o, lse)`` with ``lse = ln(e^state_lse + e^lse_k)`` (rows with both -inf stay
    -inf with zero output)."""
    state_o, o_k = np.asarray(state_o, np.float64), np.asarray(o_k, np.float64)
    state_lse, lse_k = np.asarray(state_lse, np.float64), np.asarray(lse_k, np.float64)
    lse = np.logaddexp(state_lse, lse_k)
    B, Sq, H, D = o_k.shape
    out = np.zeros_like(o_k)
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                if lse[b, h, i] == -np.inf:
                    continue
                ws = 0.0 if state_lse[b, h, i] == -np.inf else np.exp(state_lse[b, h, i] - lse[b, h, i])
                wk = 0.0 if lse_k[b, h, i] == -np.inf else np.exp(lse_k[b, h, i] - lse[b, h, i])
                out[b, i, h] = ws * state_o[b, i, h] + wk * o_k[b, i, h]
    return out, lse


def merge_partials(o_parts, lses):
    """``o_parts`` ``[N, B, Sq, H, D]`` and ``lses`` ``[N, B, H, Sq]`` -> merged ``[B, Sq, H, D]``."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    N, B, Sq, H, D = o_parts.shape
    if lses.shape != (N, B, H, Sq):
        raise ValueError("lses must be [N, B, H, Sq]")
    out = np.zeros((B, Sq, H, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                lk = lses[:, b, h, i]
                if np.all(lk == -np.inf):
                    continue
                m = lk.max()
                w = np.exp(lk - m)
                out[b, i, h, :] = (w[:, None] * o_parts[:, b, i, h, :]).sum(axis=0) / w.sum()
    return out


# ------------------------------------------------ joint text/image key segments
#
# The composed Ulysses x AllGather-KV path of [vllm-omni#7641] re-attaches the
# head-sliced joint (text) K/V to the gathered image K/V, in front or behind,
# and merges the 2D key masks against that final layout: a missing side is
# filled with "attend" and the result is a [B, K_final] mask.  Attention then
# runs over the concatenation.


def joint_attention(q, k_img, v_img, k_joint, v_joint, img_mask=None, joint_mask=None,
                    joint_front=False, scale=None):
    """Attention over keys ``[joint | image]`` (front) or ``[image | joint]`` (rear)."""
    B, S_img = k_img.shape[:2]
    T = 0 if k_joint is None else k_joint.shape[1]
    im = np.ones((B, S_img), dtype=np.uint8) if img_mask is None else np.asarray(img_mask, dtype=np.uint8)
    if T == 0:
        return attention(q, k_img, v_img, im, scale)
    jm = np.ones((B, T), dtype=np.uint8) if joint_mask is None else np.asarray(joint_mask, dtype=np.uint8)
    if joint_front:
        k, v, m = (np.concatenate(x, axis=1) for x in ((k_joint, k_img), (v_joint, v_img), (jm, im)))
    else:
        k, v, m = (np.concatenate(x, axis=1) for x in ((k_img, k_joint), (v_img, v_joint), (im, jm)))
    return attention(q, k, v, m, scale)
