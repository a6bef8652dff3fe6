"""ctypes loader for libcpattn.so (the HIP C-ABI library built in this directory).

There is no fallback: if the library is missing or a symbol is absent, loading
raises.  Build it with ``python -c "import __graft_entry__ as g; g.build()"`` or
``python -m context_attention_diffusion_amd.build``.
"""

from __future__ import annotations

import ctypes
import os

LIB_NAME = "libcpattn.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

# Every symbol declared in include/cp_attn.h, with its ctypes signature.
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
SIGNATURES = {
    "cp_abi_version": (ctypes.c_int, []),
    "cp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "cp_pack_qkv_dst_major": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                             ctypes.c_int, _vp]),
    "cp_sim_exchange": (ctypes.c_int, [ctypes.POINTER(_vp), _vp, _i64, _i64, _i64, _vp]),
    "cp_unpack_head_sharded": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                              ctypes.c_int, _vp]),
    "cp_attn_localq_globalkv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                               _i64, ctypes.c_float, _vp]),
    "cp_output_reverse": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                         ctypes.c_int, _vp]),
    "cp_attn_localq_globalkv_ws": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                                  _i64, ctypes.c_float, _vp,
                                                  ctypes.c_size_t, _vp]),
    "cp_attn_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, _i64, _i64]),
    "cp_attn_localq_globalkv_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                                       _i64, ctypes.c_float, _vp]),
    "cp_pack_qkv_dst_major_padded": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                                    _i64, ctypes.c_int, _vp]),
    "cp_output_merge_cropped": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                               ctypes.c_int, _vp]),
    "cp_attn_joint": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _i64, _i64,
                                     _i64, _i64, _i64, _i64, ctypes.c_float, _vp,
                                     ctypes.c_size_t, _vp]),
    "cp_attn_partial": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                       ctypes.c_float, _vp]),
    "cp_attn_partial_accum": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                             _i64, ctypes.c_float, _vp]),
    "cp_attn_merge": (ctypes.c_int, [_vp, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp]),
    "cp_attn_recv_to_send": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                            ctypes.c_float, _vp, ctypes.c_size_t, _vp]),
    "cp_varlen_remap_cu_seqlens_q": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _vp]),
    "cp_attn_varlen": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _i64,
                                      ctypes.c_float, _vp]),
    "cp_attn_recv_to_send_2d": (ctypes.c_int, [_vp, _vp, _vp, _i64, ctypes.c_int, _vp, _vp, _vp, _i64, _i64,
                                               _i64, _i64, _i64, ctypes.c_float, _vp,
                                               ctypes.c_size_t, _vp]),
}

# Status codes (enum cp_status).
CP_OK = 0
CP_ERR_NULL = 1
CP_ERR_DTYPE = 2
CP_ERR_SHAPE = 3
CP_ERR_DIVISIBILITY = 4
CP_ERR_HEAD_DIM = 5
CP_ERR_ALIGNMENT = 6
CP_ERR_ALIAS = 7
CP_ERR_SCALE = 8
CP_ERR_UNSUPPORTED = 9
CP_ERR_HIP = 10
CP_ERR_WORKSPACE = 11
CP_ERR_SCRATCH = 12

CP_DTYPE_BF16 = 0
CP_DTYPE_FP16 = 1
ABI_VERSION = 11

_lib = None


class CpError(RuntimeError):
    """A libcpattn entry point returned a nonzero status."""

    def __init__(self, fn: str, code: int, message: str):
        super().__init__(f"{fn}: {message} (status {code})")
        self.code = code


def load() -> ctypes.CDLL:
    """Load libcpattn.so once and bind every declared symbol; raises if anything is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; the HIP library is required (no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (restype, argtypes) in SIGNATURES.items():
        fn = getattr(lib, name)  # AttributeError if the export is missing
        fn.restype = restype
        fn.argtypes = argtypes
    if lib.cp_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH}: ABI version {lib.cp_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def check(fn: str, code: int) -> None:
    if code != CP_OK:
        msg = load().cp_status_string(code).decode()
        raise CpError(fn, code, msg)
