"""Helpers for the GPU parity tests: bit-exact host <-> device transfer and the
simulated W-rank exchange driven through the C ABI."""

import numpy as np
import torch

import context_attention_diffusion_amd as cp

DEV = "cuda:0"


def to_dev(bits: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """uint16 bit patterns -> device tensor of a 2-byte dtype (bits unchanged)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype)
    return t.to(DEV)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def forward_all_ranks(shards, W, dtype=torch.bfloat16):
    """Every rank of one Ulysses group: pack -> simulated exchange -> unpack.

    ``shards[r] = (q, k, v)`` as uint16 bits ``[B, S_l, H, D]``.  Returns
    ``(staging, recv, outs)``: per-rank device tensors.
    """
    B = shards[0][0].shape[0]
    staging = []
    for r in range(W):
        q, k, v = (to_dev(x, dtype) for x in shards[r])
        staging.append(cp.cp_pack_qkv_dst_major(q, k, v, W, staging=torch.empty(
            (W, q.shape[0] * q.shape[1], q.shape[2] // W, 3 * q.shape[3]), dtype=dtype, device=DEV)))
    recv = [cp.cp_sim_exchange(staging, j) for j in range(W)]
    outs = [cp.cp_unpack_head_sharded(recv[j], B, W) for j in range(W)]
    return staging, recv, outs


def reverse_all_ranks(o_hs, W, B):
    """Every rank: send layout -> simulated exchange -> merge.  ``o_hs[r]`` on device."""
    if B == 1:
        snd = [o for o in o_hs]  # the send layout is the identity for B == 1
    else:
        snd = [cp.cp_output_reverse(0, o, W, B) for o in o_hs]
    snd = [s.reshape(W, B, -1, s.shape[-2], s.shape[-1]) for s in snd]
    rcv = [cp.cp_sim_exchange(snd, j) for j in range(W)]
    return snd, rcv, [cp.cp_output_reverse(1, x, W, B) for x in rcv]
