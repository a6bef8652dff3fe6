"""Seeded synthetic workloads shared by the tests, the oracle checks and the benchmark.

This module holds shapes and random draws only.  It computes no step of the
method (no packing, no exchange, no attention), so the oracle and the HIP path
can both take their inputs from here without sharing any arithmetic.

Shapes follow the per-rank shares of context-parallel diffusion attention:

* image-DiT shapes: 24 heads, head dim 128, 4096 image tokens plus text tokens
  (the Wan / Qwen-Image / Z-Image class of models that the ChituDiffusion
  "Install and enable Fast CP" page validates its wrapper on, section
  "Support scope": CP2/4/8, batch 1, BF16, D 128, even shards, no mask);
* a video-DiT shape with 12 heads and 32760 tokens, sharded over a 2 x 2
  Ulysses x AllGather-KV grid as in vllm-omni PR #7641 ("Compose Ulysses with
  AllGather-KV as a 2D diffusion SP", commit message);
* a batch-2 joint text+image share with a per-batch key-padding mask, the
  2D key-validity mask of that PR's review-fix commits (True = attend).

Every tensor is bf16 drawn as N(0, 1) on the CPU by ``torch.randn`` with a
seeded ``torch.Generator`` -- the recipe of the unit test in the sglang PR
#33667 summary ("Key source snippets", test_usp_packed_qkv_a2a.py excerpt,
seed 1234) -- and handed out as raw ``uint16`` bit patterns so that both sides
see identical bits.
"""

from __future__ import annotations

import dataclasses
import hashlib

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """One rank's share of a context-parallel attention layer.

    Global tensors are ``[B, S, H, D]``.  The Ulysses exchange runs over ``W``
    ranks, each holding ``S_local = S / (W * A)`` consecutive rows of all heads
    (ranks 0..W-1 of Ulysses group 0).  ``attn_rows`` / ``attn_heads`` give the
    attention problem of global rank 0: its query rows ``[0, attn_rows)`` and
    heads ``[0, attn_heads)`` against every key row of the same heads.
    """

    name: str
    seed: int
    B: int
    S: int
    H: int
    D: int
    W: int
    A: int
    attn_rows: int
    attn_heads: int
    text_tokens: int = 0        # > 0: the last text_tokens keys are padded text
    text_len_min: int = 64
    text_len_max: int = 512

    @property
    def S_local(self) -> int:
        return self.S // (self.W * self.A)

    @property
    def H_local(self) -> int:
        return self.H // self.W

    @property
    def masked(self) -> bool:
        return self.text_tokens > 0

    def pack_bytes(self) -> int:
        """Algorithmic bytes of one pack (or unpack): 3 tensors read + written once."""
        return 2 * 3 * self.B * self.S_local * self.H * self.D * 2

    def merge_bytes(self) -> int:
        """Algorithmic bytes of one output-reverse merge: one tensor read + written."""
        return 2 * self.B * self.S_local * self.H * self.D * 2

    def attn_flops_dense(self) -> int:
        """4*B*H*Sq*Skv*D: the two GEMMs of non-causal attention, softmax not counted."""
        return 4 * self.B * self.attn_heads * self.attn_rows * self.S * self.D


# Seed rule: 1234 (the pages' test seed) + a per-workload id.
WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in (
        # B=1, S=256, H=4, D=64, W=2: a correctness-sized case.
        Workload("tiny_w2", 1235, B=1, S=256, H=4, D=64, W=2, A=1,
                 attn_rows=128, attn_heads=4),
        # Image DiT, CP4 share: 4096 image + 256 text tokens.
        Workload("image_cp4", 1236, B=1, S=4352, H=24, D=128, W=4, A=1,
                 attn_rows=1088, attn_heads=24),
        # Image DiT, CP8 share.
        Workload("image_cp8", 1237, B=1, S=4096, H=24, D=128, W=8, A=1,
                 attn_rows=512, attn_heads=24),
        # Video DiT, Ulysses U=2 x AllGather-KV A=2: rank (0,0) after the exchange
        # holds rows [0, 16380) of heads [0, 6) and attends to all 32760 keys.
        Workload("video_u2a2", 1238, B=1, S=32760, H=12, D=128, W=2, A=2,
                 attn_rows=16380, attn_heads=6),
        # Joint text+image with a CFG pair (B=2) and a per-batch text padding mask.
        Workload("joint_cfg_cp4", 1239, B=2, S=4608, H=24, D=128, W=4, A=1,
                 attn_rows=1152, attn_heads=24, text_tokens=512),
    )
}

# The two shapes of the pages' own single-GPU unit test, (W, B, S, H, D), seed 1234.
PAGE_TEST_SHAPES = ((4, 1, 128, 8, 64), (2, 2, 48, 6, 32))
PAGE_TEST_SEED = 1234


def randn_bf16_bits(shape, seed: int, stream: int = 0) -> np.ndarray:
    """bf16 N(0,1) draws as uint16 bits.  ``stream`` separates tensors of one seed."""
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) * 16 + int(stream))
    t = torch.randn(tuple(int(s) for s in shape), dtype=torch.bfloat16, generator=g)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def page_test_tensors(B: int, S: int, H: int, D: int, seed: int = PAGE_TEST_SEED):
    """Three global [B,S,H,D] bf16 tensors drawn in sequence from one seeded generator,
    as the pages' unit test does for Q, K and V."""
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    out = []
    for _ in range(3):
        t = torch.randn((B, S, H, D), dtype=torch.bfloat16, generator=g)
        out.append(t.view(torch.int16).numpy().view(np.uint16).copy())
    return out


def global_qkv(wl: Workload, heads: int | None = None):
    """Global Q, K, V ``[B, S, H, D]`` as uint16 bf16 bits (optionally only the first heads)."""
    H = wl.H if heads is None else heads
    out = []
    for c in range(3):
        full = randn_bf16_bits((wl.B, wl.S, wl.H, wl.D), wl.seed, stream=c)
        out.append(np.ascontiguousarray(full[:, :, :H, :]))
    return out


def text_lengths(wl: Workload) -> np.ndarray:
    """Per-batch valid text length L_b ~ Uniform{text_len_min..text_len_max} (inclusive)."""
    rng = np.random.default_rng(wl.seed)
    return rng.integers(wl.text_len_min, wl.text_len_max + 1, size=wl.B)


def packed_boundaries(wl, n_docs):
    """Seeded boundaries of ``n_docs`` documents packed into the ``wl.S`` rows of one
    batch row: ``[0, c_1, ..., wl.S]`` with distinct cut points drawn uniformly."""
    rng = np.random.default_rng(wl.seed + 31)
    cuts = np.sort(rng.choice(np.arange(1, wl.S), size=n_docs - 1, replace=False))
    return [0] + [int(c) for c in cuts] + [wl.S]


def key_mask(wl: Workload, text_front: bool = False) -> np.ndarray | None:
    """uint8 ``[B, S]`` key-validity mask (nonzero = attend), or None when unmasked.

    Rear layout (default): image keys ``[0, S-T)`` then text ``[S-T, S)``; key j is
    padding iff ``j >= S - T + L_b``.  Front layout: text ``[0, T)`` first; key j is
    padding iff ``L_b <= j < T``.
    """
    if not wl.masked:
        return None
    T = wl.text_tokens
    L = text_lengths(wl)
    m = np.ones((wl.B, wl.S), dtype=np.uint8)
    for b in range(wl.B):
        if text_front:
            m[b, int(L[b]):T] = 0
        else:
            m[b, wl.S - T + int(L[b]):] = 0
    return m


def rank_shards(full: np.ndarray, wl: Workload):
    """Sequence shards ``[B, S_local, H, D]`` of Ulysses group 0 (ranks 0..W-1)."""
    Sl = wl.S_local
    return [np.ascontiguousarray(full[:, r * Sl:(r + 1) * Sl]) for r in range(wl.W)]


def sha256_of(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
