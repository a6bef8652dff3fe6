"""The allocation-free attention entry point against the workspace one.

cp_attn_localq_globalkv_noalloc keeps the split-KV partial states in the
library's static scratch array; its output must equal that of
cp_attn_localq_globalkv_ws (same kernels, same split plan) bit for bit, and be
within the attention tolerance of the fp64 oracle.  Two calls in a row, the
second on a smaller input, so the second reads scratch that the first left
behind only where it wrote it again.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import bf16

pytestmark = pytest.mark.gpu


def _rand_bits(shape, seed):
    return bf16.f64_to_bits_rne(np.random.default_rng(seed).standard_normal(shape))


@pytest.mark.parametrize("first,second", [
    # (B, H, Sq, Skv, D, masked): both shapes split their key range over several
    # workgroups (few query blocks), the second one smaller and masked
    ((1, 2, 130, 4096, 128, False), (2, 1, 70, 2000, 64, True)),
    ((1, 24, 512, 4096, 128, False), (1, 3, 100, 2000, 128, True)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    import context_attention_diffusion_amd as cp
    import gpu_util as gu
    for n, (B, H, Sq, Skv, D, masked) in enumerate((first, second)):
        seed = 4200 + 10 * n + Sq + Skv + D
        q = _rand_bits((B, Sq, H, D), seed)
        k = _rand_bits((B, Skv, H, D), seed + 1)
        v = _rand_bits((B, Skv, H, D), seed + 2)
        mask = None
        if masked:
            mask = (np.random.default_rng(seed + 3).random((B, Skv)) > 0.4).astype(np.uint8)
            mask[:, 0] = 1
        print(f"[noalloc] call {n}: B={B} H={H} Sq={Sq} Skv={Skv} D={D} masked={masked}", flush=True)
        qd, kd, vd = gu.to_dev(q), gu.to_dev(k), gu.to_dev(v)
        md = None if mask is None else torch.from_numpy(mask).to(gu.DEV)
        out = torch.empty_like(qd)
        cp.cp_attn_localq_globalkv_noalloc(qd, kd, vd, md, out=out)
        ref_ws = cp.cp_attn_localq_globalkv(qd, kd, vd, md, split=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_ws), f"call {n}: differs from the workspace entry point"
        got = gu.to_f64(out)
        ref = OA.attention(bf16.bits_to_f64(q), bf16.bits_to_f64(k), bf16.bits_to_f64(v), mask,
                           1.0 / math.sqrt(D))
        err = np.abs(got - ref)
        print(f"  max|err| {err.max():.3e} mean|err| {err.mean():.3e}", flush=True)
        assert np.isfinite(got).all() and err.max() <= 2e-2 and err.mean() <= 2e-3
