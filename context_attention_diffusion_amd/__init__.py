"""MI355X-native hot path of context-parallel diffusion attention (one GPU's share).

The compute lives in ``libcpattn.so`` (HIP, gfx950), whose C ABI is declared in
``include/cp_attn.h``; this package is its thin Python binding.  Importing the
package does not load the library; the first call does, and raises if it is not
built.
"""

from ._lib import CpError, load  # noqa: F401
from .ops import (  # noqa: F401
    clear_staging,
    cp_attn_joint,
    cp_attn_localq_globalkv,
    cp_attn_localq_globalkv_noalloc,
    cp_attn_merge,
    cp_attn_partial,
    cp_attn_partial_accum,
    cp_attn_recv_to_send,
    cp_attn_recv_to_send_2d,
    cp_attn_varlen,
    cp_varlen_remap_cu_seqlens_q,
    cp_attn_workspace_bytes,
    cp_output_merge_cropped,
    cp_output_reverse,
    cp_pack_qkv_dst_major,
    cp_pack_qkv_dst_major_padded,
    cp_sim_exchange,
    cp_unpack_head_sharded,
    staging_buffer,
)

__all__ = [
    "CpError", "load", "staging_buffer", "clear_staging",
    "cp_pack_qkv_dst_major", "cp_pack_qkv_dst_major_padded", "cp_output_merge_cropped", "cp_sim_exchange", "cp_unpack_head_sharded",
    "cp_attn_localq_globalkv", "cp_attn_localq_globalkv_noalloc", "cp_attn_joint", "cp_attn_partial", "cp_attn_partial_accum", "cp_attn_merge", "cp_attn_recv_to_send", "cp_attn_recv_to_send_2d", "cp_attn_varlen", "cp_varlen_remap_cu_seqlens_q", "cp_attn_workspace_bytes", "cp_output_reverse",
]
