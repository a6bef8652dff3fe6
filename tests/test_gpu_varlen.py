"""GPU parity of packed variable-length attention and of the per-rank remap of
packed query boundaries.

* remap: bit-exact (integers) against the oracle on the hand-worked fixture and
  on random boundaries;
* varlen attention: element by element against the fp64 oracle, max|err| <= 2e-2
  and mean|err| <= 2e-3, on documents that span several 128-row query blocks and
  64-key tiles with ragged tails, empty query documents, documents without keys and
  rows outside every document (which stay untouched);
* the pages' two-rank equivalence: every AllGather-KV rank remaps the global
  boundaries on the device and attends its local rows; the outputs, concatenated,
  equal the unsplit packed call bit for bit (a query row's result does not depend
  on the block it sits in) and the oracle within the bar;
* one document covering everything is the dense call, bit for bit.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import bf16
from oracle import varlen as OV

pytestmark = pytest.mark.gpu

MAX_ERR = 2e-2
MEAN_ERR = 2e-3


@pytest.fixture(scope="module")
def gu():
    import gpu_util
    return gpu_util


def _bits(shape, seed):
    return bf16.f64_to_bits_rne(np.random.default_rng(seed).standard_normal(shape))


def _cu(gu, c):
    return torch.tensor(list(c), dtype=torch.int32, device=gu.DEV)


def _close(got, ref, what):
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    print(f"  {what}: max|err| {mx:.3e} mean|err| {mean:.3e}", flush=True)
    assert mx <= MAX_ERR and mean <= MEAN_ERR, f"{what}: max {mx} mean {mean}"


def test_remap_golden_and_random(gu):
    import context_attention_diffusion_amd as cp
    cases = [([0, 8, 12], 2, 12), ([0, 3, 5, 12], 2, 12), ([0, 12], 3, 12), ([0, 2, 2, 9, 12], 3, 12)]
    rng = np.random.default_rng(5)
    for _ in range(6):
        A = int(rng.integers(1, 9))
        Sl = int(rng.integers(1, 5000))
        cu = np.sort(rng.integers(0, A * Sl + 1, size=int(rng.integers(2, 40))))
        cases.append((cu.tolist(), A, A * Sl))
    for cu, A, S in cases:
        print(f"[varlen] remap n_docs={len(cu) - 1} A={A} S={S}", flush=True)
        g = _cu(gu, cu)
        for r in range(A):
            got = cp.cp_varlen_remap_cu_seqlens_q(g, r, S // A)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(got.cpu().numpy(), OV.remap_cu_seqlens_q(cu, r, S // A),
                                          err_msg=f"cu {cu} rank {r}")


CASES = [
    # (D, H, Sq, Skv, cu_q, cu_k)
    (128, 3, 700, 900, [0, 300, 301, 700], [0, 450, 451, 900]),        # ragged documents, one of one row
    (128, 2, 600, 640, [0, 0, 250, 600], [0, 100, 300, 640]),         # an empty query document
    (64, 4, 520, 700, [10, 200, 200, 500], [0, 130, 130, 700]),       # rows outside every document, no keys
    (128, 2, 1100, 1000, [0, 1100], [0, 1000]),                      # one long document, 9 query blocks
    (64, 1, 300, 300, [0, 64, 128, 192, 256, 300], [0, 64, 128, 192, 256, 300]),  # tile-aligned
    # several documents inside one 128-row tile, run one after the other by its block
    (128, 2, 400, 500, [0, 5, 17, 18, 40, 77, 128, 129, 300, 400], [0, 50, 60, 61, 100, 200, 300, 310, 420, 500]),
]


@pytest.mark.parametrize("D,H,Sq,Skv,cu_q,cu_k", CASES)
def test_varlen_matches_oracle(gu, D, H, Sq, Skv, cu_q, cu_k):
    import context_attention_diffusion_amd as cp
    print(f"[varlen] attention D={D} H={H} Sq={Sq} Skv={Skv} cu_q={cu_q} cu_k={cu_k}", flush=True)
    seed = D + H + Sq
    q, k, v = _bits((Sq, H, D), seed), _bits((Skv, H, D), seed + 1), _bits((Skv, H, D), seed + 2)
    scale = 1.0 / math.sqrt(D)
    out = torch.zeros((Sq, H, D), dtype=torch.bfloat16, device=gu.DEV)
    out.fill_(7.0)   # rows outside every document must keep this value
    cp.cp_attn_varlen(gu.to_dev(q), gu.to_dev(k), gu.to_dev(v), _cu(gu, cu_q), _cu(gu, cu_k), out=out)
    torch.cuda.synchronize()
    got = gu.to_f64(out)
    ref = OV.varlen_attention(bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v), cu_q, cu_k, scale)
    covered = np.zeros(Sq, dtype=bool)
    for i in range(len(cu_q) - 1):
        covered[cu_q[i]:cu_q[i + 1]] = True
    assert (got[~covered] == 7.0).all(), "rows outside every document were written"
    _close(got[covered], ref[covered], "varlen")


def test_varlen_one_document_is_dense_call(gu):
    import context_attention_diffusion_amd as cp
    Sq, Skv, H, D = 333, 517, 2, 128
    q, k, v = _bits((Sq, H, D), 1), _bits((Skv, H, D), 2), _bits((Skv, H, D), 3)
    qd, kd, vd = gu.to_dev(q), gu.to_dev(k), gu.to_dev(v)
    vo = cp.cp_attn_varlen(qd, kd, vd, _cu(gu, [0, Sq]), _cu(gu, [0, Skv]))
    do = cp.cp_attn_localq_globalkv(qd[None], kd[None], vd[None], None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.to_bits(vo), gu.to_bits(do[0]))


@pytest.mark.parametrize("A,S,H,D,cu", [
    (2, 12, 2, 64, [0, 8, 12]),                                   # the pages' worked case
    (2, 2048, 3, 128, [0, 700, 701, 1500, 2048]),
    (4, 4352, 2, 128, [0, 1000, 2200, 2201, 4100, 4352]),
    (3, 1536, 2, 64, [0, 0, 600, 1536]),
])
def test_agkv_ranks_reassemble_unsplit(gu, A, S, H, D, cu):
    import context_attention_diffusion_amd as cp
    print(f"[varlen] AllGather-KV A={A} S={S} H={H} D={D} cu={cu}", flush=True)
    q, k, v = _bits((S, H, D), S + 1), _bits((S, H, D), S + 2), _bits((S, H, D), S + 3)
    qd, kd, vd = gu.to_dev(q), gu.to_dev(k), gu.to_dev(v)
    g = _cu(gu, cu)
    full = cp.cp_attn_varlen(qd, kd, vd, g, g)
    Sl = S // A
    parts = []
    for r in range(A):
        loc = cp.cp_varlen_remap_cu_seqlens_q(g, r, Sl)
        parts.append(cp.cp_attn_varlen(qd[r * Sl:(r + 1) * Sl].contiguous(), kd, vd, loc, g))
    torch.cuda.synchronize()
    cat = torch.cat(parts, dim=0)
    np.testing.assert_array_equal(gu.to_bits(cat), gu.to_bits(full))
    ref = np.concatenate(OV.agkv_varlen_outputs(bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v),
                                                cu, A, 1.0 / math.sqrt(D)), axis=0)
    _close(gu.to_f64(cat), ref, "AllGather-KV varlen")


def test_full_size_image_share_all_ranks(gu):
    """The bench's packed workload at full size: the image CP4 sequence (4352 rows, 24
    heads, D 128) cut into 4 seeded documents, every AllGather-KV rank's remap and
    packed attention of its 1088 rows, against the oracle over every output."""
    import context_attention_diffusion_amd as cp
    import workloads
    wl = workloads.WORKLOADS["image_cp4"]
    cu = workloads.packed_boundaries(wl, 4)
    print(f"[varlen] full size image_cp4, documents {cu}", flush=True)
    q, k, v = (np.ascontiguousarray(t[0]) for t in workloads.global_qkv(wl))
    qd, kd, vd = gu.to_dev(q), gu.to_dev(k), gu.to_dev(v)
    g = _cu(gu, cu)
    Sl = wl.attn_rows
    A = wl.S // Sl
    parts = []
    for r in range(A):
        loc = cp.cp_varlen_remap_cu_seqlens_q(g, r, Sl)
        parts.append(cp.cp_attn_varlen(qd[r * Sl:(r + 1) * Sl].contiguous(), kd, vd, loc, g))
    torch.cuda.synchronize()
    got = gu.to_f64(torch.cat(parts, dim=0))
    ref = np.concatenate(OV.agkv_varlen_outputs(bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v),
                                                cu, A, 1.0 / math.sqrt(wl.D)), axis=0)
    _close(got, ref, "image_cp4 packed, 4 ranks")
