"""The C-ABI library loads, exports every symbol include/cp_attn.h declares, and
rejects invalid arguments on the host before enqueuing anything (CPU only).

The error-path calls pass fake, never-dereferenced addresses; every one of them
must be rejected by host validation.  They are skipped on a machine with a GPU
so that a validation bug can never turn them into a real launch.
"""

import ctypes
import math
import os
import re

import pytest

from context_attention_diffusion_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cp_attn.h")


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = _declared_symbols()
    for name in ("cp_pack_qkv_dst_major", "cp_unpack_head_sharded", "cp_attn_localq_globalkv",
                 "cp_output_reverse", "cp_sim_exchange", "cp_status_string", "cp_abi_version"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    syms = _declared_symbols()
    assert set(syms) == set(_lib.SIGNATURES)
    for name in syms:
        assert hasattr(lib, name), name
    assert lib.cp_abi_version() == _lib.ABI_VERSION


def test_status_strings():
    lib = _lib.load()
    seen = set()
    for code in range(0, 13):
        s = lib.cp_status_string(code).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.cp_status_string(99).decode() == "unknown status code"


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


cpu_only = pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation tests run only without a GPU")

A = 0x10000          # fake 16-byte aligned addresses, never dereferenced
BIG = 1 << 40        # far apart so that nothing overlaps unless intended
BF16 = _lib.CP_DTYPE_BF16


def _pack(**kw):
    a = dict(q=A, k=A + BIG, v=A + 2 * BIG, st=A + 3 * BIG, B=1, Sl=4, H=4, D=128, W=2,
             dtype=BF16)
    a.update(kw)
    return _lib.load().cp_pack_qkv_dst_major(a["q"], a["k"], a["v"], a["st"], a["B"], a["Sl"],
                                             a["H"], a["D"], a["W"], a["dtype"], None)


def _pack_pad(**kw):
    a = dict(q=A, k=A + BIG, v=A + 2 * BIG, st=A + 3 * BIG, B=1, Sl=4, H=14, Hp=16, D=128, W=4,
             dtype=BF16)
    a.update(kw)
    return _lib.load().cp_pack_qkv_dst_major_padded(a["q"], a["k"], a["v"], a["st"], a["B"], a["Sl"],
                                                    a["H"], a["Hp"], a["D"], a["W"], a["dtype"], None)


def _merge_crop(**kw):
    a = dict(s=A, d=A + BIG, B=1, Sl=4, Hl=4, H=14, D=128, W=4, dtype=BF16)
    a.update(kw)
    return _lib.load().cp_output_merge_cropped(a["s"], a["d"], a["B"], a["Sl"], a["Hl"], a["H"], a["D"],
                                               a["W"], a["dtype"], None)


def _unpack(**kw):
    a = dict(r=A, q=A + BIG, k=A + 2 * BIG, v=A + 3 * BIG, B=1, Sl=4, Hl=2, D=128, W=2,
             dtype=BF16)
    a.update(kw)
    return _lib.load().cp_unpack_head_sharded(a["r"], a["q"], a["k"], a["v"], a["B"], a["Sl"],
                                              a["Hl"], a["D"], a["W"], a["dtype"], None)


def _attn(**kw):
    a = dict(q=A, k=A + BIG, v=A + 2 * BIG, m=None, o=A + 3 * BIG, B=1, Sq=8, Skv=16, H=2,
             D=128, scale=0.125)
    a.update(kw)
    return _lib.load().cp_attn_localq_globalkv(a["q"], a["k"], a["v"], a["m"], a["o"], a["B"],
                                               a["Sq"], a["Skv"], a["H"], a["D"], a["scale"], None)


def _attn_ws(**kw):
    a = dict(q=A, k=A + BIG, v=A + 2 * BIG, m=None, o=A + 3 * BIG, B=1, Sq=8, Skv=16, H=2,
             D=128, scale=0.125, ws=A + 5 * BIG, nbytes=16)
    a.update(kw)
    return _lib.load().cp_attn_localq_globalkv_ws(a["q"], a["k"], a["v"], a["m"], a["o"], a["B"],
                                                  a["Sq"], a["Skv"], a["H"], a["D"], a["scale"],
                                                  a["ws"], a["nbytes"], None)


def _attn_noalloc(**kw):
    a = dict(q=A, k=A + BIG, v=A + 2 * BIG, m=None, o=A + 3 * BIG, B=1, Sq=8, Skv=16, H=2,
             D=128, scale=0.125)
    a.update(kw)
    return _lib.load().cp_attn_localq_globalkv_noalloc(a["q"], a["k"], a["v"], a["m"], a["o"], a["B"],
                                                       a["Sq"], a["Skv"], a["H"], a["D"], a["scale"], None)


def _fused(**kw):
    a = dict(r=A, m=None, s=A + BIG, B=1, Sl=128, Hl=2, D=128, W=2, scale=0.125,
             ws=None, nbytes=0)
    a.update(kw)
    return _lib.load().cp_attn_recv_to_send(a["r"], a["m"], a["s"], a["B"], a["Sl"], a["Hl"], a["D"],
                                            a["W"], a["scale"], a["ws"], a["nbytes"], None)


def _fused2d(**kw):
    a = dict(r=A, ko=A + 2 * BIG, vo=A + 3 * BIG, So=256, first=0, om=None, xm=None, s=A + BIG, B=1, Sl=128,
             Hl=2, D=128, W=2, scale=0.125, ws=None, nbytes=0)
    a.update(kw)
    return _lib.load().cp_attn_recv_to_send_2d(a["r"], a["ko"], a["vo"], a["So"], a["first"], a["om"], a["xm"],
                                               a["s"], a["B"], a["Sl"], a["Hl"], a["D"], a["W"], a["scale"],
                                               a["ws"], a["nbytes"], None)


def _varlen(**kw):
    a = dict(q=A, k=A + BIG, v=A + 2 * BIG, cq=A + 3 * BIG, ck=A + 4 * BIG, n=2, o=A + 5 * BIG, Sq=100,
             Skv=200, H=2, D=128, scale=0.125)
    a.update(kw)
    return _lib.load().cp_attn_varlen(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["n"], a["o"], a["Sq"],
                                      a["Skv"], a["H"], a["D"], a["scale"], None)


def _remap(**kw):
    a = dict(g=A, l=A + BIG, n=3, r=1, Sl=16)
    a.update(kw)
    return _lib.load().cp_varlen_remap_cu_seqlens_q(a["g"], a["l"], a["n"], a["r"], a["Sl"], None)


def _partial(**kw):
    a = dict(q=A, k=A + BIG, v=A + 2 * BIG, m=None, o=A + 3 * BIG, lse=A + 4 * BIG, B=1, Sq=8, Skv=16,
             H=2, D=128, scale=0.125)
    a.update(kw)
    return _lib.load().cp_attn_partial(a["q"], a["k"], a["v"], a["m"], a["o"], a["lse"], a["B"], a["Sq"],
                                       a["Skv"], a["H"], a["D"], a["scale"], None)


def _accum(**kw):
    a = dict(q=A, k=A + BIG, v=A + 2 * BIG, m=None, so=A + 3 * BIG, sl=A + 4 * BIG, of=None, B=1, Sq=8,
             Skv=16, H=2, D=128, scale=0.125)
    a.update(kw)
    return _lib.load().cp_attn_partial_accum(a["q"], a["k"], a["v"], a["m"], a["so"], a["sl"], a["of"], a["B"],
                                             a["Sq"], a["Skv"], a["H"], a["D"], a["scale"], None)


def _merge(**kw):
    a = dict(p=A, l=A + BIG, N=2, o=A + 2 * BIG, B=1, Sq=8, H=2, D=128)
    a.update(kw)
    return _lib.load().cp_attn_merge(a["p"], a["l"], a["N"], a["o"], a["B"], a["Sq"], a["H"], a["D"], None)


def _joint(**kw):
    a = dict(q=A, ki=A + BIG, vi=A + 2 * BIG, im=None, kj=A + 3 * BIG, vj=A + 4 * BIG, jm=None, front=0,
             o=A + 5 * BIG, B=1, Sq=8, Si=64, T=16, H=2, D=128, scale=0.125, ws=None, nbytes=0)
    a.update(kw)
    return _lib.load().cp_attn_joint(a["q"], a["ki"], a["vi"], a["im"], a["kj"], a["vj"], a["jm"], a["front"],
                                     a["o"], a["B"], a["Sq"], a["Si"], a["T"], a["H"], a["D"], a["scale"],
                                     a["ws"], a["nbytes"], None)


def _rev(**kw):
    a = dict(phase=0, s=A, d=A + BIG, B=1, Sl=4, Hl=2, D=128, W=2, dtype=BF16)
    a.update(kw)
    return _lib.load().cp_output_reverse(a["phase"], a["s"], a["d"], a["B"], a["Sl"], a["Hl"],
                                         a["D"], a["W"], a["dtype"], None)


def _xchg(W=2, rank=0, nbytes=4096, sends=None, recv=A + 8 * BIG):
    if sends is None:
        sends = [A + i * BIG for i in range(W)]
    arr = (ctypes.c_void_p * len(sends))(*sends)
    return _lib.load().cp_sim_exchange(arr, recv, W, rank, nbytes, None)


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.CP_ERR_NULL),
    (dict(st=None), _lib.CP_ERR_NULL),
    (dict(dtype=7), _lib.CP_ERR_DTYPE),
    (dict(B=0), _lib.CP_ERR_SHAPE),
    (dict(Sl=-1), _lib.CP_ERR_SHAPE),
    (dict(W=0), _lib.CP_ERR_SHAPE),
    (dict(H=6, W=4), _lib.CP_ERR_DIVISIBILITY),
    (dict(D=12), _lib.CP_ERR_HEAD_DIM),
    (dict(D=0), _lib.CP_ERR_HEAD_DIM),
    (dict(q=A + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(st=A + 3 * BIG + 2), _lib.CP_ERR_ALIGNMENT),
    (dict(st=A + 64), _lib.CP_ERR_ALIAS),
    (dict(B=1 << 20, Sl=1 << 20, H=64), _lib.CP_ERR_SHAPE),
])
def test_pack_rejects(kw, code):
    assert _pack(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(v=None), _lib.CP_ERR_NULL),
    (dict(dtype=-1), _lib.CP_ERR_DTYPE),
    (dict(Hl=0), _lib.CP_ERR_SHAPE),
    (dict(D=20), _lib.CP_ERR_HEAD_DIM),
    (dict(k=A + 2 * BIG + 4), _lib.CP_ERR_ALIGNMENT),
    (dict(k=A + BIG + 16), _lib.CP_ERR_ALIAS),       # k_out overlaps q_out
    (dict(q=A + 32), _lib.CP_ERR_ALIAS),             # q_out overlaps recv
    (dict(B=1 << 16, Sl=1 << 16, W=8), _lib.CP_ERR_SHAPE),
])
def test_unpack_rejects(kw, code):
    assert _unpack(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(o=None), _lib.CP_ERR_NULL),
    (dict(Sq=0), _lib.CP_ERR_SHAPE),
    (dict(Skv=0), _lib.CP_ERR_SHAPE),
    (dict(H=0), _lib.CP_ERR_SHAPE),
    (dict(D=96), _lib.CP_ERR_HEAD_DIM),
    (dict(D=256), _lib.CP_ERR_HEAD_DIM),
    (dict(scale=0.0), _lib.CP_ERR_SCALE),
    (dict(scale=-1.0), _lib.CP_ERR_SCALE),
    (dict(scale=math.nan), _lib.CP_ERR_SCALE),
    (dict(scale=math.inf), _lib.CP_ERR_SCALE),
    (dict(v=A + 2 * BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(o=A + 16), _lib.CP_ERR_ALIAS),             # o overlaps q
    (dict(o=A + BIG + 16), _lib.CP_ERR_ALIAS),       # o overlaps k
    (dict(m=A + 3 * BIG + 16), _lib.CP_ERR_ALIAS),   # mask inside o
    (dict(B=1 << 31), _lib.CP_ERR_SHAPE),
])
def test_attention_rejects(kw, code):
    assert _attn(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(Skv=4096), _lib.CP_ERR_WORKSPACE),          # 2 query blocks x 32 iterations split; 16 bytes is too small
    (dict(ws=A + 5 * BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(Skv=4096, ws=A + 3 * BIG, nbytes=1 << 30), _lib.CP_ERR_ALIAS),   # workspace overlaps o
    (dict(o=None), _lib.CP_ERR_NULL),
    (dict(D=96), _lib.CP_ERR_HEAD_DIM),
])
def test_attention_ws_rejects(kw, code):
    assert _attn_ws(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.CP_ERR_NULL),
    (dict(Sq=0), _lib.CP_ERR_SHAPE),
    (dict(D=96), _lib.CP_ERR_HEAD_DIM),
    (dict(scale=-1.0), _lib.CP_ERR_SCALE),
    (dict(k=A + BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(o=A + 2 * BIG + 16), _lib.CP_ERR_ALIAS),   # o overlaps v
    (dict(B=1 << 31), _lib.CP_ERR_SHAPE),
])
def test_attention_noalloc_rejects(kw, code):
    """Host validation runs before the library looks up its scratch array."""
    assert _attn_noalloc(**kw) == code


def test_noalloc_scratch_limit_matches_the_workspace_bound():
    """The static scratch holds the largest split any 256-CU device plans for D = 128:
    one 128 x (D + 2) fp32 slot per compute unit."""
    text = open(HEADER).read()
    m = re.search(r"#define CP_ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u \* (\d+)u\)", text)
    assert m
    cus, rows, cols, word = (int(x) for x in m.groups())
    assert (cus, rows, cols, word) == (256, 128, 128 + 2, 4)


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(r=None), _lib.CP_ERR_NULL),
    (dict(s=None), _lib.CP_ERR_NULL),
    (dict(W=0), _lib.CP_ERR_SHAPE),
    (dict(Sl=0), _lib.CP_ERR_SHAPE),
    (dict(B=0), _lib.CP_ERR_SHAPE),
    (dict(D=96), _lib.CP_ERR_HEAD_DIM),
    (dict(scale=0.0), _lib.CP_ERR_SCALE),
    (dict(r=A + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(ws=A + 5 * BIG + 8, nbytes=1 << 20), _lib.CP_ERR_ALIGNMENT),
    (dict(s=A + 4096), _lib.CP_ERR_ALIAS),                      # send overlaps recv
    (dict(m=A + BIG + 64), _lib.CP_ERR_ALIAS),                  # mask inside send
    (dict(B=2, Sl=70, Hl=10000), _lib.CP_ERR_SHAPE),           # tiles span chunks, recv over 2 GB
    (dict(ws=A + 5 * BIG, nbytes=16, Sl=2048), _lib.CP_ERR_WORKSPACE),  # 2 heads x 32 blocks split
    (dict(ws=A, nbytes=1 << 30, Sl=2048), _lib.CP_ERR_ALIAS),   # workspace overlaps recv
    (dict(Sl=1 << 30, W=4), _lib.CP_ERR_SHAPE),
])
def test_recv_to_send_rejects(kw, code):
    assert _fused(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(r=None), _lib.CP_ERR_NULL),
    (dict(ko=None), _lib.CP_ERR_NULL),
    (dict(vo=None), _lib.CP_ERR_NULL),
    (dict(s=None), _lib.CP_ERR_NULL),
    (dict(So=0), _lib.CP_ERR_SHAPE),
    (dict(W=0), _lib.CP_ERR_SHAPE),
    (dict(Sl=0), _lib.CP_ERR_SHAPE),
    (dict(first=2), _lib.CP_ERR_UNSUPPORTED),
    (dict(D=96), _lib.CP_ERR_HEAD_DIM),
    (dict(scale=0.0), _lib.CP_ERR_SCALE),
    (dict(ko=A + 2 * BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(s=A + 4096), _lib.CP_ERR_ALIAS),                      # send overlaps recv
    (dict(s=A + 2 * BIG + 64), _lib.CP_ERR_ALIAS),              # send overlaps k_other
    (dict(xm=A + BIG + 64), _lib.CP_ERR_ALIAS),                 # other mask inside send
    (dict(ws=A + 3 * BIG, nbytes=1 << 20), _lib.CP_ERR_ALIAS),  # workspace overlaps v_other
    (dict(B=2, Sl=70, Hl=10000), _lib.CP_ERR_SHAPE),           # tiles span chunks, recv over 2 GB
    (dict(Sl=1 << 30, W=4), _lib.CP_ERR_SHAPE),
])
def test_recv_to_send_2d_rejects(kw, code):
    assert _fused2d(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.CP_ERR_NULL),
    (dict(cq=None), _lib.CP_ERR_NULL),
    (dict(ck=None), _lib.CP_ERR_NULL),
    (dict(n=0), _lib.CP_ERR_SHAPE),
    (dict(Sq=0), _lib.CP_ERR_SHAPE),
    (dict(Skv=0), _lib.CP_ERR_SHAPE),
    (dict(H=1 << 24), _lib.CP_ERR_SHAPE),             # a K/V tile's rows beyond 32-bit offsets
    (dict(D=96), _lib.CP_ERR_HEAD_DIM),
    (dict(scale=0.0), _lib.CP_ERR_SCALE),
    (dict(o=A + 5 * BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(cq=A + 3 * BIG + 2), _lib.CP_ERR_ALIGNMENT),
    (dict(o=A + 64), _lib.CP_ERR_ALIAS),              # o over q
    (dict(o=A + 2 * BIG + 16), _lib.CP_ERR_ALIAS),    # o over v
    (dict(ck=A + 5 * BIG + 4), _lib.CP_ERR_ALIAS),    # key boundaries inside o
])
def test_varlen_rejects(kw, code):
    assert _varlen(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(g=None), _lib.CP_ERR_NULL),
    (dict(l=None), _lib.CP_ERR_NULL),
    (dict(n=0), _lib.CP_ERR_SHAPE),
    (dict(r=-1), _lib.CP_ERR_SHAPE),
    (dict(Sl=0), _lib.CP_ERR_SHAPE),
    (dict(r=1 << 20, Sl=1 << 12), _lib.CP_ERR_SHAPE),  # span start beyond int32
    (dict(l=A + BIG + 2), _lib.CP_ERR_ALIGNMENT),
    (dict(l=A + 8), _lib.CP_ERR_ALIAS),
])
def test_remap_rejects(kw, code):
    assert _remap(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(o=None), _lib.CP_ERR_NULL),
    (dict(lse=None), _lib.CP_ERR_NULL),
    (dict(Skv=0), _lib.CP_ERR_SHAPE),
    (dict(D=96), _lib.CP_ERR_HEAD_DIM),
    (dict(scale=-1.0), _lib.CP_ERR_SCALE),
    (dict(o=A + 3 * BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(lse=A + 4 * BIG + 2), _lib.CP_ERR_ALIGNMENT),
    (dict(o=A + 16), _lib.CP_ERR_ALIAS),              # o_part overlaps q
    (dict(lse=A + BIG + 64), _lib.CP_ERR_ALIAS),      # lse inside k
    (dict(lse=A + 3 * BIG + 64), _lib.CP_ERR_ALIAS),  # lse inside o_part
    (dict(m=A + 4 * BIG + 4), _lib.CP_ERR_ALIAS),     # mask inside lse
])
def test_partial_rejects(kw, code):
    assert _partial(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(so=None), _lib.CP_ERR_NULL),
    (dict(sl=None), _lib.CP_ERR_NULL),
    (dict(D=96), _lib.CP_ERR_HEAD_DIM),
    (dict(so=A + 3 * BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(of=A + 5 * BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(so=A + BIG + 64), _lib.CP_ERR_ALIAS),          # state inside k
    (dict(sl=A + 3 * BIG + 64), _lib.CP_ERR_ALIAS),      # lse inside state_o
    (dict(of=A + 3 * BIG), _lib.CP_ERR_ALIAS),           # final output over the state
    (dict(of=A + 32), _lib.CP_ERR_ALIAS),                # final output over q
])
def test_partial_accum_rejects(kw, code):
    assert _accum(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(p=None), _lib.CP_ERR_NULL),
    (dict(o=None), _lib.CP_ERR_NULL),
    (dict(N=0), _lib.CP_ERR_SHAPE),
    (dict(Sq=0), _lib.CP_ERR_SHAPE),
    (dict(D=32), _lib.CP_ERR_HEAD_DIM),
    (dict(p=A + 4), _lib.CP_ERR_ALIGNMENT),
    (dict(l=A + BIG + 1), _lib.CP_ERR_ALIGNMENT),
    (dict(o=A + 64), _lib.CP_ERR_ALIAS),              # o inside o_parts
    (dict(o=A + BIG), _lib.CP_ERR_ALIAS),             # o over lses
])
def test_merge_rejects(kw, code):
    assert _merge(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.CP_ERR_NULL),
    (dict(dtype=5), _lib.CP_ERR_DTYPE),
    (dict(Hp=13), _lib.CP_ERR_SHAPE),               # H_pad < H
    (dict(Hp=18), _lib.CP_ERR_DIVISIBILITY),        # 18 % 4
    (dict(D=12), _lib.CP_ERR_HEAD_DIM),
    (dict(st=A + 3 * BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(st=A + 16), _lib.CP_ERR_ALIAS),           # staging overlaps q
    (dict(B=1 << 20, Sl=1 << 20), _lib.CP_ERR_SHAPE),
])
def test_pack_padded_rejects(kw, code):
    assert _pack_pad(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(d=None), _lib.CP_ERR_NULL),
    (dict(H=17), _lib.CP_ERR_SHAPE),                # more heads than W * H_local
    (dict(H=0), _lib.CP_ERR_SHAPE),
    (dict(D=4), _lib.CP_ERR_HEAD_DIM),
    (dict(s=A + 4), _lib.CP_ERR_ALIGNMENT),
    (dict(d=A + 1024), _lib.CP_ERR_ALIAS),
])
def test_merge_cropped_rejects(kw, code):
    assert _merge_crop(**kw) == code


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.CP_ERR_NULL),
    (dict(kj=None), _lib.CP_ERR_NULL),               # joint tokens without joint keys
    (dict(T=-1), _lib.CP_ERR_SHAPE),
    (dict(Si=0), _lib.CP_ERR_SHAPE),
    (dict(front=2), _lib.CP_ERR_UNSUPPORTED),
    (dict(D=96), _lib.CP_ERR_HEAD_DIM),
    (dict(vj=A + 4 * BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(o=A + 3 * BIG + 32), _lib.CP_ERR_ALIAS),  # o overlaps k_joint
    (dict(jm=A + 5 * BIG + 8), _lib.CP_ERR_ALIAS),  # joint mask inside o
    (dict(ws=A + 6 * BIG, nbytes=16, Si=4096), _lib.CP_ERR_WORKSPACE),
])
def test_joint_rejects(kw, code):
    assert _joint(**kw) == code


def test_workspace_bytes():
    lib = _lib.load()
    n = lib.cp_attn_workspace_bytes(1, 1088, 4352, 24, 128)
    # one partial slot of 128 rows x (128 + 2) floats per compute unit
    assert n > 0 and n % (128 * 130 * 4) == 0
    assert lib.cp_attn_workspace_bytes(1, 1088, 4352, 24, 96) == 0
    assert lib.cp_attn_workspace_bytes(0, 1088, 4352, 24, 128) == 0


@cpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(s=None), _lib.CP_ERR_NULL),
    (dict(phase=2), _lib.CP_ERR_UNSUPPORTED),
    (dict(phase=-1), _lib.CP_ERR_UNSUPPORTED),
    (dict(dtype=3), _lib.CP_ERR_DTYPE),
    (dict(W=0), _lib.CP_ERR_SHAPE),
    (dict(D=4), _lib.CP_ERR_HEAD_DIM),
    (dict(d=A + BIG + 8), _lib.CP_ERR_ALIGNMENT),
    (dict(d=A + 128), _lib.CP_ERR_ALIAS),
])
def test_reverse_rejects(kw, code):
    assert _rev(**kw) == code


@cpu_only
def test_exchange_rejects():
    assert _xchg(W=0) == _lib.CP_ERR_SHAPE
    assert _xchg(W=65, sends=[A + i * BIG for i in range(65)]) == _lib.CP_ERR_UNSUPPORTED
    assert _xchg(rank=2) == _lib.CP_ERR_SHAPE
    assert _xchg(rank=-1) == _lib.CP_ERR_SHAPE
    assert _xchg(nbytes=48) == _lib.CP_ERR_DIVISIBILITY      # 48 % (16*2) != 0
    assert _xchg(nbytes=0) == _lib.CP_ERR_SHAPE
    assert _xchg(recv=A + 8 * BIG + 4) == _lib.CP_ERR_ALIGNMENT
    assert _xchg(sends=[A, None]) == _lib.CP_ERR_NULL
    assert _xchg(sends=[A, A + BIG + 8]) == _lib.CP_ERR_ALIGNMENT
    assert _xchg(recv=A + 1024) == _lib.CP_ERR_ALIAS
    assert _lib.load().cp_sim_exchange(None, A, 2, 0, 4096, None) == _lib.CP_ERR_NULL
