"""Pins of the packed variable-length oracle (``oracle/varlen.py``).

* the query-boundary remap against the hand-worked fixture (the pages' own case
  and three more worked from the same rule) and against its invariants on random
  boundaries;
* per-document attention against a brute-force element loop with an explicit
  document lookup (a wrong pairing of query and key documents, or a missed
  boundary, changes rows);
* one document covering everything reduces to the plain (pinned) attention oracle;
* the ranks' remapped outputs, concatenated, equal the unsplit packed attention
  (the equivalence the pages test on two AllGather-KV ranks).
"""

import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import varlen as V


def _fixture(golden_dir):
    cases, cur = [], None
    for line in open(os.path.join(golden_dir, "varlen_remap.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("global"):
            g, a, s = line.split("|")
            cur = {"cu": [int(x) for x in g.split()[1:]], "A": int(a.split()[1]), "S": int(s.split()[1]),
                   "ranks": {}}
            cases.append(cur)
        else:
            head, vals = line.split(":")
            cur["ranks"][int(head.split()[1])] = [int(x) for x in vals.split()]
    return cases


def test_remap_golden(golden_dir):
    cases = _fixture(golden_dir)
    assert len(cases) == 4
    for c in cases:
        assert sorted(c["ranks"]) == list(range(c["A"]))
        for r, want in c["ranks"].items():
            got = V.remap_cu_seqlens_q(c["cu"], r, c["S"] // c["A"])
            assert got.tolist() == want, (c["cu"], r)


@pytest.mark.parametrize("seed", range(6))
def test_remap_invariants(seed):
    rng = np.random.default_rng(seed)
    A = int(rng.integers(1, 5))
    Sl = int(rng.integers(1, 9))
    S = A * Sl
    n = int(rng.integers(1, 7))
    cu = np.sort(rng.integers(0, S + 1, size=n + 1))
    if seed % 2 == 0:
        cu[0] = 0                       # the usual packing; odd seeds leave rows before document 0
    lens = np.zeros(n, dtype=np.int64)
    for r in range(A):
        loc = V.remap_cu_seqlens_q(cu, r, Sl)
        assert loc.size == n + 1 and loc[0] >= 0 and (np.diff(loc) >= 0).all() and loc[-1] <= Sl
        # local row j of document i is global row r*Sl + j, and lies inside document i
        for i in range(n):
            for j in range(loc[i], loc[i + 1]):
                assert cu[i] <= r * Sl + j < cu[i + 1]
        lens += np.diff(loc)
    np.testing.assert_array_equal(lens, np.diff(cu))


def _brute(q, k, v, cu_q, cu_k, scale):
    Sq, H, D = q.shape
    out = np.zeros((Sq, H, D))
    for i in range(Sq):
        doc = [d for d in range(len(cu_q) - 1) if cu_q[d] <= i < cu_q[d + 1]]
        if not doc:
            continue
        keys = range(cu_k[doc[0]], cu_k[doc[0] + 1])
        for h in range(H):
            w = {j: math.exp(scale * sum(q[i, h, t] * k[j, h, t] for t in range(D))) for j in keys}
            tot = sum(w.values())
            for t in range(D):
                out[i, h, t] = sum(w[j] * v[j, h, t] for j in keys) / tot if keys else 0.0
    return out


@pytest.mark.parametrize("cu_q,cu_k", [
    ([0, 3, 7], [0, 5, 9]),
    ([0, 2, 2, 6], [0, 3, 4, 9]),      # an empty query document keeps its entry
    ([1, 4, 6], [0, 0, 9]),            # a document without keys; row 0 outside every document
    ([0, 7], [2, 8]),
])
def test_varlen_brute_force(cu_q, cu_k):
    rng = np.random.default_rng(len(cu_q) * 10 + cu_k[-1])
    q = rng.standard_normal((7, 2, 4))
    k = rng.standard_normal((9, 2, 4))
    v = rng.standard_normal((9, 2, 4))
    got = V.varlen_attention(q, k, v, cu_q, cu_k, scale=0.7)
    np.testing.assert_allclose(got, _brute(q, k, v, cu_q, cu_k, 0.7), rtol=1e-12, atol=1e-12)


def test_one_document_is_plain_attention():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((10, 3, 8))
    k = rng.standard_normal((13, 3, 8))
    v = rng.standard_normal((13, 3, 8))
    got = V.varlen_attention(q, k, v, [0, 10], [0, 13])
    np.testing.assert_allclose(got, A.attention(q[None], k[None], v[None])[0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("A_deg,cu", [(2, [0, 8, 12]), (2, [0, 3, 5, 12]), (3, [0, 2, 2, 9, 12]), (4, [0, 12])])
def test_ranks_reassemble_unsplit_packed_attention(A_deg, cu):
    rng = np.random.default_rng(A_deg * 7 + len(cu))
    S = cu[-1]
    q, k, v = (rng.standard_normal((S, 2, 8)) for _ in range(3))
    full = V.varlen_attention(q, k, v, cu, cu)
    outs = V.agkv_varlen_outputs(q, k, v, cu, A_deg)
    np.testing.assert_allclose(np.concatenate(outs, axis=0), full, rtol=1e-12, atol=1e-12)


def test_rejects_bad_boundaries():
    q = np.zeros((4, 1, 2))
    k = np.zeros((4, 1, 2))
    with pytest.raises(ValueError):
        V.varlen_attention(q, k, k, [0, 3, 2], [0, 1, 4])
    with pytest.raises(ValueError):
        V.varlen_attention(q, k, k, [0, 5], [0, 4])
    with pytest.raises(ValueError):
        V.varlen_attention(q, k, k, [0, 2, 4], [0, 4])
