"""Torch-facing wrappers of the libcpattn C ABI (argument marshalling only).

Each function checks that tensors are on a GPU, contiguous and of the right
dtype, allocates outputs the caller did not supply, and calls the entry point of
the same name on the current HIP stream.  Every step of the computation runs in
the library's kernels; nothing here computes on tensor data.
"""

from __future__ import annotations

import ctypes
import math

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.CP_DTYPE_BF16, torch.float16: _lib.CP_DTYPE_FP16}


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"dtype {t.dtype} not supported; use bfloat16 or float16") from None


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ---------------------------------------------------------------- staging cache

_STAGING: dict[tuple, torch.Tensor] = {}


def staging_buffer(role: str, shape, dtype, device) -> torch.Tensor:
    """Reusable staging buffer keyed by (role, shape, dtype, device index).

    Same contract as the staging cache of the sglang PR #33667 summary
    (implementation breakdown item 1): a role's buffer is fully consumed, in
    stream order, before the next call with that role overwrites it, so reuse is
    safe on one stream; use from several streams needs explicit events.  During
    stream capture a fresh buffer is returned instead, so that a graph never
    shares memory with eager calls.
    """
    device = torch.device(device)
    shape = tuple(int(s) for s in shape)
    if torch.cuda.is_current_stream_capturing():
        return torch.empty(shape, dtype=dtype, device=device)
    key = (role, shape, dtype, device.index)
    buf = _STAGING.get(key)
    if buf is None:
        buf = torch.empty(shape, dtype=dtype, device=device)
        _STAGING[key] = buf
    return buf


def clear_staging() -> None:
    _STAGING.clear()


# ---------------------------------------------------------------- entry points

def cp_pack_qkv_dst_major(q, k, v, W: int, staging=None, stream=None) -> torch.Tensor:
    """[B,S_l,H,D] x3 -> staging [W, B*S_l, H/W, 3D] (destination-major, last axis q|k|v)."""
    lib = _lib.load()
    B, Sl, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if H % W:
        raise ValueError("H must divide by W")
    shape = (W, B * Sl, H // W, 3 * D)
    if staging is None:
        staging = staging_buffer("cp_pack_send", shape, q.dtype, q.device)
    if tuple(staging.shape) != shape or staging.dtype != q.dtype:
        raise ValueError(f"staging must be {shape} {q.dtype}")
    _lib.check("cp_pack_qkv_dst_major", lib.cp_pack_qkv_dst_major(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(staging, "staging"),
        B, Sl, H, D, W, _dtype_code(q), _stream(stream)))
    return staging


def cp_pack_qkv_dst_major_padded(q, k, v, W: int, H_pad: int, staging=None, stream=None) -> torch.Tensor:
    """[B,S_l,H,D] x3 -> staging [W, B*S_l, H_pad/W, 3D], heads >= H zero (head padding)."""
    lib = _lib.load()
    B, Sl, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if H_pad < H or H_pad % W:
        raise ValueError("H_pad must be >= H and divide by W")
    shape = (W, B * Sl, H_pad // W, 3 * D)
    if staging is None:
        staging = staging_buffer("cp_pack_send", shape, q.dtype, q.device)
    if tuple(staging.shape) != shape or staging.dtype != q.dtype:
        raise ValueError(f"staging must be {shape} {q.dtype}")
    _lib.check("cp_pack_qkv_dst_major_padded", lib.cp_pack_qkv_dst_major_padded(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(staging, "staging"),
        B, Sl, H, H_pad, D, W, _dtype_code(q), _stream(stream)))
    return staging


def cp_output_merge_cropped(src, H: int, out=None, stream=None) -> torch.Tensor:
    """[W, B, S_l, H_l, D] -> [B, S_l, H, D]: the merge keeping the first H of W*H_l heads."""
    lib = _lib.load()
    W, B, Sl, Hl, D = src.shape
    if not 1 <= H <= W * Hl:
        raise ValueError("H must be in [1, W*H_l]")
    shape = (B, Sl, H, D)
    if out is None:
        out = torch.empty(shape, dtype=src.dtype, device=src.device)
    if tuple(out.shape) != shape or out.dtype != src.dtype:
        raise ValueError(f"out must be {shape} {src.dtype}")
    _lib.check("cp_output_merge_cropped", lib.cp_output_merge_cropped(
        _dev(src, "src"), _dev(out, "dst"), B, Sl, Hl, H, D, W, _dtype_code(src), _stream(stream)))
    return out


def cp_sim_exchange(sends, rank: int, recv=None, stream=None) -> torch.Tensor:
    """Single-GPU stand-in for the all-to-all: ``recv`` chunk r = chunk ``rank`` of ``sends[r]``."""
    lib = _lib.load()
    W = len(sends)
    nbytes = sends[0].numel() * sends[0].element_size()
    for s in sends:
        if s.shape != sends[0].shape or s.dtype != sends[0].dtype:
            raise ValueError("send buffers must share shape and dtype")
    if recv is None:
        recv = torch.empty_like(sends[0])
    if recv.numel() * recv.element_size() != nbytes:
        raise ValueError("recv must have the size of one send buffer")
    arr = (ctypes.c_void_p * W)(*[_dev(s, f"sends[{i}]") for i, s in enumerate(sends)])
    _lib.check("cp_sim_exchange", lib.cp_sim_exchange(
        arr, _dev(recv, "recv"), W, rank, nbytes, _stream(stream)))
    return recv


def cp_unpack_head_sharded(recv, B: int, W: int, out=None, stream=None):
    """recv [W, B*S_l, H_l, 3D] -> (q, k, v), each [B, W*S_l, H_l, D]."""
    lib = _lib.load()
    W_, rows, Hl, D3 = recv.shape
    if W_ != W or rows % B or D3 % 3:
        raise ValueError("recv shape does not match W / B")
    Sl, D = rows // B, D3 // 3
    shape = (B, W * Sl, Hl, D)
    if out is None:
        out = tuple(torch.empty(shape, dtype=recv.dtype, device=recv.device) for _ in range(3))
    for t in out:
        if tuple(t.shape) != shape or t.dtype != recv.dtype:
            raise ValueError(f"outputs must be {shape} {recv.dtype}")
    _lib.check("cp_unpack_head_sharded", lib.cp_unpack_head_sharded(
        _dev(recv, "recv"), _dev(out[0], "q_out"), _dev(out[1], "k_out"), _dev(out[2], "v_out"),
        B, Sl, Hl, D, W, _dtype_code(recv), _stream(stream)))
    return out


def cp_attn_localq_globalkv(q, k, v, key_mask=None, scale=None, out=None,
                            stream=None, split=True, workspace=None) -> torch.Tensor:
    """Non-causal attention: q [B,Sq,H,D] vs k, v [B,Skv,H,D] (bf16), optional uint8 mask [B,Skv].

    split=True lets the library split the key range of query blocks over
    workgroups when the problem has too few query blocks to fill the GPU; the
    workspace (a uint8 tensor of at least cp_attn_workspace_bytes bytes) comes
    from the staging cache unless given.  split=False uses the entry point
    without a workspace (one workgroup per query block).
    """
    lib = _lib.load()
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if k.shape != (B, Skv, H, D) or v.shape != k.shape:
        raise ValueError("k, v must be [B, Skv, H, D] matching q")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("attention takes bfloat16 q, k, v")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    mask_ptr = None
    if key_mask is not None:
        if key_mask.dtype not in (torch.uint8, torch.bool) or tuple(key_mask.shape) != (B, Skv):
            raise ValueError("key_mask must be uint8/bool [B, Skv]")
        mask_ptr = _dev(key_mask, "key_mask")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if not split:
        _lib.check("cp_attn_localq_globalkv", lib.cp_attn_localq_globalkv(
            _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), mask_ptr, _dev(out, "o"),
            B, Sq, Skv, H, D, float(scale), _stream(stream)))
        return out
    need = int(lib.cp_attn_workspace_bytes(B, Sq, Skv, H, D))
    if workspace is None:
        workspace = staging_buffer("attn_workspace", (max(need, 16),), torch.uint8, q.device)
    elif workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    _lib.check("cp_attn_localq_globalkv_ws", lib.cp_attn_localq_globalkv_ws(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), mask_ptr, _dev(out, "o"),
        B, Sq, Skv, H, D, float(scale), _dev(workspace, "workspace"),
        workspace.numel(), _stream(stream)))
    return out


def cp_attn_localq_globalkv_noalloc(q, k, v, key_mask=None, scale=None, out=None, stream=None) -> torch.Tensor:
    """The split-KV attention with its partial states in the library's static scratch
    array (no workspace, no allocation inside the call; out must be given by callers
    that cannot allocate).  Same arguments and result as cp_attn_localq_globalkv."""
    lib = _lib.load()
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if k.shape != (B, Skv, H, D) or v.shape != k.shape:
        raise ValueError("k, v must be [B, Skv, H, D] matching q")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("attention takes bfloat16 q, k, v")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    mask_ptr = None
    if key_mask is not None:
        if key_mask.dtype not in (torch.uint8, torch.bool) or tuple(key_mask.shape) != (B, Skv):
            raise ValueError("key_mask must be uint8/bool [B, Skv]")
        mask_ptr = _dev(key_mask, "key_mask")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    _lib.check("cp_attn_localq_globalkv_noalloc", lib.cp_attn_localq_globalkv_noalloc(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), mask_ptr, _dev(out, "o"),
        B, Sq, Skv, H, D, float(scale), _stream(stream)))
    return out


def cp_attn_joint(q, k_img, v_img, k_joint=None, v_joint=None, img_mask=None, joint_mask=None,
                  joint_front=False, scale=None, out=None, stream=None, split=True,
                  workspace=None) -> torch.Tensor:
    """Attention of q [B,Sq,H,D] over two key segments, image [B,S_img,H,D] and joint
    [B,T,H,D] (None: T = 0), in the order joint_front selects, with per-segment uint8
    masks (None = all valid)."""
    lib = _lib.load()
    B, Sq, H, D = q.shape
    S_img = k_img.shape[1]
    if k_img.shape != (B, S_img, H, D) or v_img.shape != k_img.shape:
        raise ValueError("k_img, v_img must be [B, S_img, H, D] matching q")
    T = 0 if k_joint is None else k_joint.shape[1]
    if T and (k_joint.shape != (B, T, H, D) or v_joint is None or v_joint.shape != k_joint.shape):
        raise ValueError("k_joint, v_joint must be [B, T, H, D] matching q")
    for t in (q, k_img, v_img) + ((k_joint, v_joint) if T else ()):
        if t.dtype != torch.bfloat16:
            raise TypeError("attention takes bfloat16")
    if scale is None:
        scale = 1.0 / math.sqrt(D)

    def mask_ptr(m, n, name):
        if m is None:
            return None
        if m.dtype not in (torch.uint8, torch.bool) or tuple(m.shape) != (B, n):
            raise ValueError(f"{name} must be uint8/bool [B, {n}]")
        return _dev(m, name)

    im = mask_ptr(img_mask, S_img, "img_mask")
    jm = mask_ptr(joint_mask, T, "joint_mask") if T else None
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    ws_ptr, ws_bytes = None, 0
    if split:
        need = int(lib.cp_attn_workspace_bytes(B, Sq, S_img + T, H, D))
        if workspace is None:
            workspace = staging_buffer("attn_workspace", (max(need, 16),), torch.uint8, q.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel()
    _lib.check("cp_attn_joint", lib.cp_attn_joint(
        _dev(q, "q"), _dev(k_img, "k_img"), _dev(v_img, "v_img"), im,
        _dev(k_joint, "k_joint") if T else None, _dev(v_joint, "v_joint") if T else None, jm,
        int(bool(joint_front)), _dev(out, "o"), B, Sq, S_img, T, H, D, float(scale),
        ws_ptr, ws_bytes, _stream(stream)))
    return out


def cp_attn_partial(q, k, v, key_mask=None, scale=None, out=None, lse=None,
                    stream=None):
    """Attention over one K/V chunk: (o_part fp32 [B,Sq,H,D], lse fp32 [B,H,Sq], natural log).

    Merge the partial results of disjoint key chunks with cp_attn_merge."""
    lib = _lib.load()
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if k.shape != (B, Skv, H, D) or v.shape != k.shape:
        raise ValueError("k, v must be [B, Skv, H, D] matching q")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("attention takes bfloat16 q, k, v")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    mask_ptr = None
    if key_mask is not None:
        if key_mask.dtype not in (torch.uint8, torch.bool) or tuple(key_mask.shape) != (B, Skv):
            raise ValueError("key_mask must be uint8/bool [B, Skv]")
        mask_ptr = _dev(key_mask, "key_mask")
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, Sq, H, D) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [B, Sq, H, D]")
    if tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, Sq]")
    _lib.check("cp_attn_partial", lib.cp_attn_partial(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), mask_ptr, _dev(out, "o_part"), _dev(lse, "lse"),
        B, Sq, Skv, H, D, float(scale), _stream(stream)))
    return out, lse


def cp_attn_partial_accum(q, k, v, state_o, state_lse, key_mask=None, scale=None, final=False, out=None,
                          stream=None):
    """Fold attention over one more K/V chunk into a running state (fp32 state_o [B,Sq,H,D],
    state_lse [B,H,Sq], as cp_attn_partial writes them).  final=False updates the state in
    place and returns (state_o, state_lse); final=True returns the merged bf16 output."""
    lib = _lib.load()
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if k.shape != (B, Skv, H, D) or v.shape != k.shape:
        raise ValueError("k, v must be [B, Skv, H, D] matching q")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("attention takes bfloat16 q, k, v")
    if tuple(state_o.shape) != (B, Sq, H, D) or state_o.dtype != torch.float32:
        raise ValueError("state_o must be float32 [B, Sq, H, D]")
    if tuple(state_lse.shape) != (B, H, Sq) or state_lse.dtype != torch.float32:
        raise ValueError("state_lse must be float32 [B, H, Sq]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    mask_ptr = None
    if key_mask is not None:
        if key_mask.dtype not in (torch.uint8, torch.bool) or tuple(key_mask.shape) != (B, Skv):
            raise ValueError("key_mask must be uint8/bool [B, Skv]")
        mask_ptr = _dev(key_mask, "key_mask")
    o_ptr = None
    if final:
        if out is None:
            out = torch.empty_like(q)
        if out.shape != q.shape or out.dtype != torch.bfloat16:
            raise ValueError("out must match q")
        o_ptr = _dev(out, "o_final")
    _lib.check("cp_attn_partial_accum", lib.cp_attn_partial_accum(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), mask_ptr, _dev(state_o, "state_o"),
        _dev(state_lse, "state_lse"), o_ptr, B, Sq, Skv, H, D, float(scale),
        _stream(stream)))
    return out if final else (state_o, state_lse)


def cp_attn_merge(o_parts, lses, out=None, stream=None) -> torch.Tensor:
    """Merge partial results: o_parts fp32 [N,B,Sq,H,D], lses fp32 [N,B,H,Sq] -> bf16 [B,Sq,H,D]."""
    lib = _lib.load()
    N, B, Sq, H, D = o_parts.shape
    if o_parts.dtype != torch.float32 or lses.dtype != torch.float32 or tuple(lses.shape) != (N, B, H, Sq):
        raise ValueError("o_parts must be float32 [N,B,Sq,H,D] and lses float32 [N,B,H,Sq]")
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device=o_parts.device)
    if tuple(out.shape) != (B, Sq, H, D) or out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16 [B, Sq, H, D]")
    _lib.check("cp_attn_merge", lib.cp_attn_merge(
        _dev(o_parts, "o_parts"), _dev(lses, "lses"), N, _dev(out, "o"), B, Sq, H, D, _stream(stream)))
    return out


def cp_attn_recv_to_send(recv, B: int, W: int, key_mask=None, scale=None, out=None,
                         stream=None, split=True, workspace=None) -> torch.Tensor:
    """Ulysses attention straight from the received staging buffer into the send layout.

    recv [W, B*S_l, H_l, 3D] bf16 -> send [W, B, S_l, H_l, D]: the attention of the
    H_l heads over the whole sequence S = W*S_l, equal bit for bit to
    unpack -> cp_attn_localq_globalkv -> cp_output_reverse(0).  key_mask: uint8/bool
    [B, S] or None.  split / workspace as for cp_attn_localq_globalkv.
    """
    lib = _lib.load()
    W_, rows, Hl, D3 = recv.shape
    if W_ != W or rows % B or D3 % 3:
        raise ValueError("recv shape does not match W / B")
    if recv.dtype != torch.bfloat16:
        raise TypeError("attention takes bfloat16")
    Sl, D = rows // B, D3 // 3
    S = W * Sl
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    mask_ptr = None
    if key_mask is not None:
        if key_mask.dtype not in (torch.uint8, torch.bool) or tuple(key_mask.shape) != (B, S):
            raise ValueError("key_mask must be uint8/bool [B, W*S_l]")
        mask_ptr = _dev(key_mask, "key_mask")
    shape = (W, B, Sl, Hl, D)
    if out is None:
        out = torch.empty(shape, dtype=recv.dtype, device=recv.device)
    if tuple(out.shape) != shape or out.dtype != recv.dtype:
        raise ValueError(f"out must be {shape} {recv.dtype}")
    ws_ptr, ws_bytes = None, 0
    if split:
        need = int(lib.cp_attn_workspace_bytes(B, S, S, Hl, D))
        if workspace is None:
            workspace = staging_buffer("attn_workspace", (max(need, 16),), torch.uint8, recv.device)
        elif workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel()
    _lib.check("cp_attn_recv_to_send", lib.cp_attn_recv_to_send(
        _dev(recv, "recv"), mask_ptr, _dev(out, "send"), B, Sl, Hl, D, W, float(scale),
        ws_ptr, ws_bytes, _stream(stream)))
    return out


def cp_attn_recv_to_send_2d(recv, k_other, v_other, B: int, W: int, other_first: bool = False,
                            own_mask=None, other_mask=None, scale=None, out=None,
                            stream=None, split=True, workspace=None) -> torch.Tensor:
    """2D-layout Ulysses attention from the received staging buffer into the send layout.

    recv [W, B*S_l, H_l, 3D] bf16 (this rank's Ulysses group) and the other
    AllGather rank's head-sharded k_other / v_other [B, S_other, H_l, D] ->
    send [W, B, S_l, H_l, D]: the attention of the H_l heads of the rank's
    W*S_l rows over both key ranges (the other rank's first when other_first),
    equal bit for bit to unpack -> cp_attn_joint -> cp_output_reverse(0).
    own_mask: uint8/bool [B, W*S_l] or None; other_mask: [B, S_other] or None.
    split / workspace as for cp_attn_localq_globalkv.
    """
    lib = _lib.load()
    W_, rows, Hl, D3 = recv.shape
    if W_ != W or rows % B or D3 % 3:
        raise ValueError("recv shape does not match W / B")
    if recv.dtype != torch.bfloat16 or k_other.dtype != torch.bfloat16 or v_other.dtype != torch.bfloat16:
        raise TypeError("attention takes bfloat16")
    Sl, D = rows // B, D3 // 3
    S = W * Sl
    if k_other.dim() != 4 or k_other.shape[0] != B or k_other.shape[2] != Hl or k_other.shape[3] != D:
        raise ValueError("k_other must be [B, S_other, H_l, D]")
    if tuple(v_other.shape) != tuple(k_other.shape):
        raise ValueError("v_other must have k_other's shape")
    So = k_other.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)

    def mask_arg(m, n, name):
        if m is None:
            return None
        if m.dtype not in (torch.uint8, torch.bool) or tuple(m.shape) != (B, n):
            raise ValueError(f"{name} must be uint8/bool [B, {n}]")
        return _dev(m, name)

    om, xm = mask_arg(own_mask, S, "own_mask"), mask_arg(other_mask, So, "other_mask")
    shape = (W, B, Sl, Hl, D)
    if out is None:
        out = torch.empty(shape, dtype=recv.dtype, device=recv.device)
    if tuple(out.shape) != shape or out.dtype != recv.dtype:
        raise ValueError(f"out must be {shape} {recv.dtype}")
    ws_ptr, ws_bytes = None, 0
    if split:
        need = int(lib.cp_attn_workspace_bytes(B, S, S + So, Hl, D))
        if workspace is None:
            workspace = staging_buffer("attn_workspace", (max(need, 16),), torch.uint8, recv.device)
        elif workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel()
    _lib.check("cp_attn_recv_to_send_2d", lib.cp_attn_recv_to_send_2d(
        _dev(recv, "recv"), _dev(k_other, "k_other"), _dev(v_other, "v_other"), So, int(bool(other_first)),
        om, xm, _dev(out, "send"), B, Sl, Hl, D, W, float(scale), ws_ptr, ws_bytes,
        _stream(stream)))
    return out


def cp_varlen_remap_cu_seqlens_q(cu_q_global, rank: int, S_local: int, out=None, stream=None) -> torch.Tensor:
    """Local packed query boundaries of AllGather-KV rank ``rank`` (span
    ``[rank*S_local, (rank+1)*S_local)``): int32 [n_docs + 1] on the device, one
    (possibly empty) entry per global document; computed on the device."""
    lib = _lib.load()
    if cu_q_global.dtype != torch.int32 or cu_q_global.dim() != 1 or cu_q_global.numel() < 2:
        raise ValueError("cu_q_global must be int32 [n_docs + 1], n_docs >= 1")
    if out is None:
        out = torch.empty_like(cu_q_global)
    if out.dtype != torch.int32 or tuple(out.shape) != tuple(cu_q_global.shape):
        raise ValueError("out must match cu_q_global")
    _lib.check("cp_varlen_remap_cu_seqlens_q", lib.cp_varlen_remap_cu_seqlens_q(
        _dev(cu_q_global, "cu_q_global"), _dev(out, "cu_q_local"), cu_q_global.numel() - 1, int(rank),
        int(S_local), _stream(stream)))
    return out


def cp_attn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale=None, out=None,
                   stream=None) -> torch.Tensor:
    """Packed variable-length attention: q [Sq, H, D], k / v [Skv, H, D] bf16; query
    document i (rows cu_seqlens_q[i]..cu_seqlens_q[i+1]) attends to key document i
    only.  The boundary arrays are int32 device tensors of n_docs + 1 entries.
    Rows of ``out`` outside every document are not written (a new ``out`` starts
    at zero)."""
    lib = _lib.load()
    if q.dim() != 3 or k.dim() != 3 or tuple(k.shape) != tuple(v.shape) or q.shape[1:] != k.shape[1:]:
        raise ValueError("expected q [Sq, H, D] and k, v [Skv, H, D]")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("attention takes bfloat16")
    for name, c in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if c.dtype != torch.int32 or c.dim() != 1 or c.numel() < 2:
            raise ValueError(f"{name} must be int32 [n_docs + 1], n_docs >= 1")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must describe the same documents")
    Sq, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.zeros_like(q)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    _lib.check("cp_attn_varlen", lib.cp_attn_varlen(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(cu_seqlens_q, "cu_seqlens_q"),
        _dev(cu_seqlens_k, "cu_seqlens_k"), cu_seqlens_q.numel() - 1, _dev(out, "o"),
        Sq, k.shape[0], H, D, float(scale), _stream(stream)))
    return out


def cp_attn_workspace_bytes(B: int, Sq: int, Skv: int, H: int, D: int) -> int:
    """Workspace bytes cp_attn_localq_globalkv may use with split=True (upper bound, current device)."""
    return int(_lib.load().cp_attn_workspace_bytes(B, Sq, Skv, H, D))


def cp_output_reverse(phase: int, src, W: int, B: int, out=None, stream=None) -> torch.Tensor:
    """phase 0: [B, W*S_l, H_l, D] -> [W, B, S_l, H_l, D]; phase 1: [W,B,S_l,H_l,D] -> [B,S_l,W*H_l,D]."""
    lib = _lib.load()
    if phase == 0:
        B_, S, Hl, D = src.shape
        if B_ != B or S % W:
            raise ValueError("src must be [B, W*S_l, H_l, D]")
        Sl = S // W
        shape = (W, B, Sl, Hl, D)
    elif phase == 1:
        W_, B_, Sl, Hl, D = src.shape
        if W_ != W or B_ != B:
            raise ValueError("src must be [W, B, S_l, H_l, D]")
        shape = (B, Sl, W * Hl, D)
    else:
        raise ValueError("phase must be 0 (send) or 1 (merge)")
    if out is None:
        out = torch.empty(shape, dtype=src.dtype, device=src.device)
    if tuple(out.shape) != shape or out.dtype != src.dtype:
        raise ValueError(f"out must be {shape} {src.dtype}")
    _lib.check("cp_output_reverse", lib.cp_output_reverse(
        phase, _dev(src, "src"), _dev(out, "dst"), B, Sl, Hl, D, W, _dtype_code(src),
        _stream(stream)))
    return out
