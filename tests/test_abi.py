"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (CPU only: no compute is launched)."""
import ctypes
import os
import re

import pytest

from linear_attention_sequence_modality_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdaconv.h")

FAKE = 0x7f0000000000          # 16-byte aligned, never dereferenced: every call below fails validation


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:kda|mla)_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return kda.load_library()


def test_library_exports_every_declared_function(lib):
    names = _declared_functions()
    assert set(names) == set(kda.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert kda.kda_status_string(code) not in ("", "unknown status")
    assert kda.kda_status_string(-99) == "unknown status"


def _desc(n_text=32, grid=(4, 10, 12), **kw):
    return kda.make_desc(n_text, grid, **kw)


def _ptrs(n, base=FAKE):
    return [ctypes.c_void_p(base + i * (1 << 32)) for i in range(n)]


def _conv(lib, desc, B=1, H=2, dk=64, dv=64, dtype=kda.KDA_BF16, ptrs=None, wt=None, wv=None):
    p = ptrs if ptrs is not None else _ptrs(6)
    wt = wt if wt is not None else (ctypes.c_void_p * 3)(*[FAKE + (20 + i) * (1 << 32) for i in range(3)])
    wv = wv if wv is not None else (ctypes.c_void_p * 3)(*[FAKE + (30 + i) * (1 << 32) for i in range(3)])
    return lib.kda_conv_forward(ctypes.byref(desc) if desc is not None else None, B, H, dk, dv, dtype,
                                p[0], p[1], p[2], wt, wv, p[3], p[4], p[5], None)


def test_conv_rejects_bad_arguments(lib):
    d = _desc()
    assert _conv(lib, None) == kda.KDA_ERR_INVALID_ARG
    assert _conv(lib, d, dtype=7) == kda.KDA_ERR_UNSUPPORTED
    assert _conv(lib, d, dk=96) == kda.KDA_ERR_UNSUPPORTED
    assert _conv(lib, d, dv=32) == kda.KDA_ERR_UNSUPPORTED
    assert _conv(lib, d, H=0) == kda.KDA_ERR_INVALID_ARG
    assert _conv(lib, d, B=-1) == kda.KDA_ERR_INVALID_ARG
    assert _conv(lib, _desc(k_text=3)) == kda.KDA_ERR_UNSUPPORTED
    assert _conv(lib, _desc(k_vis=5)) == kda.KDA_ERR_UNSUPPORTED
    assert _conv(lib, _desc(causal_t=2)) == kda.KDA_ERR_INVALID_ARG
    assert _conv(lib, _desc(n_text=0, grid=(0, 0, 0))) == kda.KDA_ERR_INVALID_ARG   # T = 0
    assert _conv(lib, _desc(n_text=-1)) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    p[1] = None
    assert _conv(lib, d, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    p[2] = ctypes.c_void_p(FAKE + 2 * (1 << 32) + 8)                   # misaligned
    assert _conv(lib, d, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    p[3] = ctypes.c_void_p(FAKE + 64)                                  # q_out overlaps q
    assert _conv(lib, d, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    p[5] = p[4]                                                        # two outputs alias
    assert _conv(lib, d, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    wt = (ctypes.c_void_p * 3)(FAKE + 20 * (1 << 32), None, FAKE + 22 * (1 << 32))
    assert _conv(lib, d, wt=wt) == kda.KDA_ERR_INVALID_ARG
    # huge index spaces are refused instead of overflowing 32-bit kernel indices
    assert _conv(lib, _desc(n_text=1 << 30, grid=(1, 1 << 15, 1 << 16))) == kda.KDA_ERR_UNSUPPORTED


def _conv_stream(lib, desc, n_hist, hist="ok", B=1, H=2, dk=64, dv=64, ptrs=None):
    p = ptrs if ptrs is not None else _ptrs(6)
    wt = (ctypes.c_void_p * 3)(*[FAKE + (20 + i) * (1 << 32) for i in range(3)])
    wv = (ctypes.c_void_p * 3)(*[FAKE + (30 + i) * (1 << 32) for i in range(3)])
    if hist == "ok":
        hist = (ctypes.c_void_p * 3)(*[FAKE + (40 + i) * (1 << 32) for i in range(3)])
    return lib.kda_conv_forward_stream(ctypes.byref(desc), B, H, dk, dv, kda.KDA_BF16, p[0], p[1], p[2],
                                       hist, n_hist, wt, wv, p[3], p[4], p[5], None)


def test_conv_stream_rejects_bad_arguments(lib):
    seg = _desc(n_text=0, grid=(3, 10, 12), causal_t=1)
    assert _conv_stream(lib, seg, 3) == kda.KDA_ERR_INVALID_ARG
    assert _conv_stream(lib, seg, -1) == kda.KDA_ERR_INVALID_ARG
    assert _conv_stream(lib, _desc(n_text=0, grid=(3, 10, 12)), 2) == kda.KDA_ERR_INVALID_ARG   # symmetric in t
    assert _conv_stream(lib, _desc(n_text=5, grid=(3, 10, 12), causal_t=1), 2) == kda.KDA_ERR_INVALID_ARG
    assert _conv_stream(lib, seg, 2, hist=None) == kda.KDA_ERR_INVALID_ARG
    assert _conv_stream(lib, seg, 2, hist=(ctypes.c_void_p * 3)(FAKE + 40 * (1 << 32), None,
                                                                FAKE + 42 * (1 << 32))) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    assert _conv_stream(lib, seg, 2, hist=(ctypes.c_void_p * 3)(p[3].value, FAKE + 41 * (1 << 32),
                                                                FAKE + 42 * (1 << 32))) == kda.KDA_ERR_INVALID_ARG
    assert _conv_stream(lib, seg, 2, hist=(ctypes.c_void_p * 3)(FAKE + 40 * (1 << 32) + 8, FAKE + 41 * (1 << 32),
                                                                FAKE + 42 * (1 << 32))) == kda.KDA_ERR_INVALID_ARG
    # a valid segment with no batch launches nothing
    assert _conv_stream(lib, seg, 2, B=0) == kda.KDA_OK


def test_workspace_size_is_host_arithmetic(lib):
    d = _desc()                                     # T = 512 -> 8 chunks
    s1 = kda.kda_forward_workspace_size(d, 1, 2, 64, 64, kda.KDA_F32)
    s2 = kda.kda_forward_workspace_size(d, 2, 2, 64, 64, kda.KDA_F32)
    assert s1 > 0 and s2 == 2 * s1 and s1 % (2 * 8) == 0
    assert kda.kda_forward_workspace_size(_desc(n_text=33), 1, 2, 64, 64, kda.KDA_F32) == \
        kda.kda_forward_workspace_size(_desc(n_text=32 + 64), 1, 2, 64, 64, kda.KDA_F32)
    # both dtypes at every head size in {64, 128}; nothing else
    for dt in (kda.KDA_BF16, kda.KDA_F32):
        for dk in (64, 128):
            for dv in (64, 128):
                assert kda.kda_forward_workspace_size(d, 1, 2, dk, dv, dt) > 0, (dt, dk, dv)
        assert kda.kda_forward_workspace_size(d, 1, 2, 96, 64, dt) == 0
        assert kda.kda_forward_workspace_size(d, 1, 2, 128, 32, dt) == 0
    # fp32 records are twice the bf16 ones
    assert kda.kda_forward_workspace_size(d, 1, 2, 128, 128, kda.KDA_F32) > \
        kda.kda_forward_workspace_size(d, 1, 2, 128, 128, kda.KDA_BF16)


def _fwd(lib, desc, B=1, H=2, dk=64, dv=64, dtype=kda.KDA_BF16, ptrs=None, s0=None, sT=None,
         ws=FAKE + 40 * (1 << 32), ws_bytes=1 << 40):
    p = ptrs if ptrs is not None else _ptrs(6)
    return lib.kda_forward(ctypes.byref(desc) if desc is not None else None, B, H, dk, dv, dtype,
                           p[0], p[1], p[2], p[3], p[4], s0, sT, p[5],
                           ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


def test_forward_rejects_bad_arguments(lib):
    d = _desc()
    assert _fwd(lib, None) == kda.KDA_ERR_INVALID_ARG
    assert _fwd(lib, d, dtype=kda.KDA_F32, dk=96, dv=128) == kda.KDA_ERR_UNSUPPORTED
    assert _fwd(lib, d, dk=32) == kda.KDA_ERR_UNSUPPORTED
    p = _ptrs(6)
    p[4] = None                                                       # beta
    assert _fwd(lib, d, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    p[5] = ctypes.c_void_p(FAKE + 2 * (1 << 32))                       # o aliases v
    assert _fwd(lib, d, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    assert _fwd(lib, d, ws=0) == kda.KDA_ERR_WORKSPACE
    need = kda.kda_forward_workspace_size(d, 1, 2, 64, 64, kda.KDA_BF16)
    assert _fwd(lib, d, ws_bytes=need - 1) == kda.KDA_ERR_WORKSPACE
    assert _fwd(lib, d, ws=FAKE + 40 * (1 << 32) + 4) == kda.KDA_ERR_WORKSPACE   # misaligned
    assert _fwd(lib, d, ws=FAKE + 16) == kda.KDA_ERR_INVALID_ARG                # overlaps q
    assert _fwd(lib, d, s0=ctypes.c_void_p(FAKE + 8)) == kda.KDA_ERR_INVALID_ARG
    assert _fwd(lib, d, sT=ctypes.c_void_p(FAKE + 3 * (1 << 32))) == kda.KDA_ERR_INVALID_ARG  # sT overlaps alpha


def _fused(lib, desc, B=1, H=2, dk=64, dv=64, dtype=kda.KDA_BF16, ptrs=None, wt=None, wv=None, sT=None,
           ws=FAKE + 40 * (1 << 32), ws_bytes=1 << 40):
    p = ptrs if ptrs is not None else _ptrs(6)
    wt = wt if wt is not None else (ctypes.c_void_p * 3)(*[FAKE + (20 + i) * (1 << 32) for i in range(3)])
    wv = wv if wv is not None else (ctypes.c_void_p * 3)(*[FAKE + (30 + i) * (1 << 32) for i in range(3)])
    return lib.kda_conv_kda_forward(ctypes.byref(desc) if desc is not None else None, B, H, dk, dv, dtype,
                                    p[0], p[1], p[2], wt, wv, p[3], p[4], None, sT, p[5],
                                    ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


def test_fused_workspace_and_argument_checks(lib):
    """kda_conv_kda_forward: its workspace is kda_forward's plus the taps, and it rejects
    bad arguments (every call below fails validation before any HIP call)."""
    d = _desc()
    for dt in (kda.KDA_BF16, kda.KDA_F32):
        base = kda.kda_forward_workspace_size(d, 1, 2, 64, 128, dt)
        fused = kda.kda_conv_kda_forward_workspace_size(d, 1, 2, 64, 128, dt)
        es = 2 if dt == kda.KDA_BF16 else 4
        assert fused == (base + 255) // 256 * 256 + (31 * (2 * 2 * 64 + 2 * 128) * es + 255) // 256 * 256
    assert kda.kda_conv_kda_forward_workspace_size(d, 1, 2, 96, 64, kda.KDA_BF16) == 0
    assert _fused(lib, None) == kda.KDA_ERR_INVALID_ARG
    assert _fused(lib, d, dk=32) == kda.KDA_ERR_UNSUPPORTED
    wt = (ctypes.c_void_p * 3)(FAKE + 20 * (1 << 32), None, FAKE + 22 * (1 << 32))
    assert _fused(lib, d, wt=wt) == kda.KDA_ERR_INVALID_ARG                        # a null tap array
    wv = (ctypes.c_void_p * 3)(FAKE + 30 * (1 << 32), FAKE + 31 * (1 << 32) + 2, FAKE + 32 * (1 << 32))
    assert _fused(lib, d, wv=wv) == kda.KDA_ERR_INVALID_ARG                        # misaligned taps
    need = kda.kda_conv_kda_forward_workspace_size(d, 1, 2, 64, 64, kda.KDA_BF16)
    assert _fused(lib, d, ws_bytes=need - 1) == kda.KDA_ERR_WORKSPACE               # kda_forward's is not enough
    assert _fused(lib, d, ws=0) == kda.KDA_ERR_WORKSPACE
    p = _ptrs(6)
    p[5] = ctypes.c_void_p(FAKE + 2 * (1 << 32))                                    # o aliases v
    assert _fused(lib, d, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    p[5] = ctypes.c_void_p(FAKE + 21 * (1 << 32))                                   # o over the k taps
    assert _fused(lib, d, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    wt = (ctypes.c_void_p * 3)(FAKE + 20 * (1 << 32), FAKE + 40 * (1 << 32) + need - 64, FAKE + 22 * (1 << 32))
    assert _fused(lib, d, wt=wt) == kda.KDA_ERR_INVALID_ARG                        # taps inside the workspace
    wv = (ctypes.c_void_p * 3)(FAKE + 30 * (1 << 32), FAKE + 40 * (1 << 32) + 4096, FAKE + 32 * (1 << 32))
    assert _fused(lib, d, wv=wv) == kda.KDA_ERR_INVALID_ARG                        # taps among the chunk records


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kda.kda_forward(kda.make_desc(4, (0, 0, 0)), x, x, x, x, torch.zeros(1, 4, 1, dtype=torch.bfloat16))


def _descs(*ds):
    arr = (kda.KdaStreamDesc * max(len(ds), 1))()
    for i, d in enumerate(ds):
        arr[i] = d
    return arr


def _fwd_varlen(lib, descs, n, H=2, dk=64, dv=64, dtype=kda.KDA_BF16, ptrs=None, ws=FAKE + 40 * (1 << 32),
                ws_bytes=1 << 40):
    p = ptrs if ptrs is not None else _ptrs(6)
    return lib.kda_forward_varlen(descs, n, H, dk, dv, dtype, p[0], p[1], p[2], p[3], p[4], None, None, p[5],
                                  ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


def _conv_varlen(lib, descs, n, H=2, dk=64, dv=64, ptrs=None):
    p = ptrs if ptrs is not None else _ptrs(6)
    wt = (ctypes.c_void_p * 3)(*[FAKE + (20 + i) * (1 << 32) for i in range(3)])
    wv = (ctypes.c_void_p * 3)(*[FAKE + (30 + i) * (1 << 32) for i in range(3)])
    return lib.kda_conv_forward_varlen(descs, n, H, dk, dv, kda.KDA_BF16, p[0], p[1], p[2], wt, wv,
                                       p[3], p[4], p[5], None)


def test_varlen_workspace_is_the_sum_of_the_streams(lib):
    a, b, c = _desc(n_text=5, grid=(1, 7, 9)), _desc(n_text=0, grid=(3, 10, 12)), _desc(n_text=200, grid=(0, 0, 0))
    one = [kda.kda_forward_workspace_size(d, 1, 2, 128, 128, kda.KDA_BF16) for d in (a, b, c)]
    assert all(x > 0 for x in one)
    assert kda.kda_forward_varlen_workspace_size([a, b, c], 2, 128, 128, torch_bf16()) == sum(one)
    assert kda.kda_forward_varlen_workspace_size([b], 2, 128, 128, torch_bf16()) == one[1]
    assert lib.kda_forward_varlen_workspace_size(None, 1, 2, 64, 64, kda.KDA_BF16) == 0
    assert lib.kda_forward_varlen_workspace_size(_descs(a), 0, 2, 64, 64, kda.KDA_BF16) == 0


def torch_bf16():
    import torch
    return torch.bfloat16


def test_varlen_rejects_bad_arguments(lib):
    a, b = _desc(n_text=5, grid=(1, 7, 9)), _desc(n_text=0, grid=(3, 10, 12))
    ok = _descs(a, b)
    assert _fwd_varlen(lib, None, 2) == kda.KDA_ERR_INVALID_ARG
    assert _fwd_varlen(lib, ok, 0) == kda.KDA_ERR_INVALID_ARG
    many = _descs(*([a] * (kda.KDA_MAX_SEQS + 1)))
    assert _fwd_varlen(lib, many, kda.KDA_MAX_SEQS + 1) == kda.KDA_ERR_UNSUPPORTED
    assert _conv_varlen(lib, many, kda.KDA_MAX_SEQS + 1) == kda.KDA_ERR_UNSUPPORTED
    empty = _descs(a, _desc(n_text=0, grid=(0, 0, 0)))                 # a stream of no tokens
    assert _fwd_varlen(lib, empty, 2) == kda.KDA_ERR_INVALID_ARG
    assert _conv_varlen(lib, empty, 2) == kda.KDA_ERR_INVALID_ARG
    assert _fwd_varlen(lib, _descs(a, _desc(k_vis=5)), 2) == kda.KDA_ERR_UNSUPPORTED
    need = lib.kda_forward_varlen_workspace_size(ok, 2, 2, 64, 64, kda.KDA_BF16)
    assert need > 0
    assert _fwd_varlen(lib, ok, 2, ws_bytes=need - 1) == kda.KDA_ERR_WORKSPACE
    assert _fwd_varlen(lib, ok, 2, ws=0) == kda.KDA_ERR_WORKSPACE
    p = _ptrs(6)
    p[5] = ctypes.c_void_p(FAKE + 2 * (1 << 32) + 64)                  # o overlaps v
    assert _fwd_varlen(lib, ok, 2, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    p[3] = ctypes.c_void_p(FAKE + 32)                                  # q_out overlaps q
    assert _conv_varlen(lib, ok, 2, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    # ranges cover the packed axis: o starting right after the last token of v is fine
    T = 5 + 63 + 360
    p = _ptrs(6)
    p[5] = ctypes.c_void_p(FAKE + 2 * (1 << 32) + T * 2 * 64 * 2)
    p[3] = ctypes.c_void_p(FAKE + 50 * (1 << 32))                      # alpha elsewhere
    assert _fwd_varlen(lib, ok, 2, ptrs=p, ws=0) == kda.KDA_ERR_WORKSPACE   # got past the overlap checks
    p[5] = ctypes.c_void_p(FAKE + 2 * (1 << 32) + T * 2 * 64 * 2 - 16)
    assert _fwd_varlen(lib, ok, 2, ptrs=p, ws=0) == kda.KDA_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op(lib):
    d = _desc()
    assert _fwd(lib, d, B=0) == kda.KDA_OK
    assert _conv(lib, d, B=0) == kda.KDA_OK


def _mla(lib, B=1, T=100, H=2, dn=128, dr=64, dv=128, dtype=kda.KDA_BF16, scale=0.07, ptrs=None):
    p = ptrs if ptrs is not None else _ptrs(6)
    return lib.mla_attention_forward(B, T, H, dn, dr, dv, dtype, p[0], p[1], p[2], p[3], p[4],
                                     ctypes.c_float(scale), p[5], None)


def test_mla_rejects_bad_arguments(lib):
    assert _mla(lib, dtype=kda.KDA_F32) == kda.KDA_ERR_UNSUPPORTED
    assert _mla(lib, dtype=9) == kda.KDA_ERR_UNSUPPORTED
    assert _mla(lib, dn=64) == kda.KDA_ERR_UNSUPPORTED
    assert _mla(lib, dr=32) == kda.KDA_ERR_UNSUPPORTED
    assert _mla(lib, dv=64) == kda.KDA_ERR_UNSUPPORTED
    assert _mla(lib, T=0) == kda.KDA_ERR_INVALID_ARG
    assert _mla(lib, H=0) == kda.KDA_ERR_INVALID_ARG
    assert _mla(lib, B=-1) == kda.KDA_ERR_INVALID_ARG
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert _mla(lib, scale=bad) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    p[3] = None                                                       # k_dir
    assert _mla(lib, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    p[1] = ctypes.c_void_p(FAKE + (1 << 32) + 2)                       # misaligned q_dir
    assert _mla(lib, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    p = _ptrs(6)
    p[5] = ctypes.c_void_p(FAKE + 4 * (1 << 32) + 1024)                # o overlaps v
    assert _mla(lib, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    assert _mla(lib, B=0) == kda.KDA_OK                                # nothing to do
    assert _mla(lib, T=1 << 20, H=4096) == kda.KDA_ERR_UNSUPPORTED     # indices past 32 bits
    assert _mla(lib, T=1 << 20, H=31) == kda.KDA_ERR_UNSUPPORTED       # one batch's keys past 4 GiB


def _bwd(lib, desc, B=1, H=2, dk=64, dv=64, dtype=kda.KDA_BF16, ins=None, outs=None, ws=FAKE + 60 * (1 << 32),
         ws_bytes=1 << 40):
    i = ins if ins is not None else _ptrs(6)
    o = outs if outs is not None else [ctypes.c_void_p(FAKE + (70 + n) * (1 << 32)) for n in range(6)]
    return lib.kda_backward(ctypes.byref(desc), B, H, dk, dv, dtype, i[0], i[1], i[2], i[3], i[4], None, i[5],
                            None, o[0], o[1], o[2], o[3], o[4], o[5], ctypes.c_void_p(ws) if ws else None,
                            ws_bytes, None)


def test_backward_rejects_bad_arguments(lib):
    d = _desc()
    assert kda.kda_backward_workspace_size(d, 1, 2, 64, 64, kda.KDA_BF16) > 0
    assert kda.kda_backward_workspace_size(d, 1, 2, 96, 64, kda.KDA_BF16) == 0
    assert _bwd(lib, d, dk=96) == kda.KDA_ERR_UNSUPPORTED
    i = _ptrs(6)
    i[5] = None                                                        # d_o
    assert _bwd(lib, d, ins=i) == kda.KDA_ERR_INVALID_ARG
    o = [ctypes.c_void_p(FAKE + (70 + n) * (1 << 32)) for n in range(6)]
    o[2] = ctypes.c_void_p(FAKE + 64)                                   # d_v overlaps q
    assert _bwd(lib, d, outs=o) == kda.KDA_ERR_INVALID_ARG
    o = [ctypes.c_void_p(FAKE + (70 + n) * (1 << 32)) for n in range(6)]
    o[4] = o[3]                                                         # d_beta aliases d_alpha
    assert _bwd(lib, d, outs=o) == kda.KDA_ERR_INVALID_ARG
    o = [ctypes.c_void_p(FAKE + (70 + n) * (1 << 32)) for n in range(5)] + [None]
    assert _bwd(lib, d, outs=o, ws=0) == kda.KDA_ERR_WORKSPACE          # d_initial_state is optional
    need = kda.kda_backward_workspace_size(d, 1, 2, 64, 64, kda.KDA_BF16)
    assert _bwd(lib, d, ws_bytes=need - 1) == kda.KDA_ERR_WORKSPACE
    assert _bwd(lib, d, B=0) == kda.KDA_OK


def test_conv_backward_rejects_bad_arguments(lib):
    d = _desc()
    p = _ptrs(9)
    wt = (ctypes.c_void_p * 3)(*[FAKE + (20 + i) * (1 << 32) for i in range(3)])
    wv = (ctypes.c_void_p * 3)(*[FAKE + (30 + i) * (1 << 32) for i in range(3)])
    dwt = (ctypes.c_void_p * 3)(*[FAKE + (80 + i) * (1 << 32) for i in range(3)])
    dwv = (ctypes.c_void_p * 3)(*[FAKE + (90 + i) * (1 << 32) for i in range(3)])

    def call(ptrs=p, B=1, dwt_=dwt, dwv_=dwv, desc=d):
        return lib.kda_conv_backward(ctypes.byref(desc), B, 2, 64, 64, kda.KDA_BF16, *ptrs[:3], wt, wv, *ptrs[3:6],
                                     *ptrs[6:9], dwt_, dwv_, None)

    assert call(B=0) == kda.KDA_OK
    assert call(desc=_desc(k_vis=5)) == kda.KDA_ERR_UNSUPPORTED
    bad = list(p)
    bad[4] = None                                                      # d_k_out
    assert call(ptrs=bad) == kda.KDA_ERR_INVALID_ARG
    bad = list(p)
    bad[6] = ctypes.c_void_p(FAKE + 3 * (1 << 32))                      # d_q aliases d_q_out
    assert call(ptrs=bad) == kda.KDA_ERR_INVALID_ARG
    assert call(dwt_=(ctypes.c_void_p * 3)(FAKE + 80 * (1 << 32), None, FAKE + 82 * (1 << 32))) == \
        kda.KDA_ERR_INVALID_ARG
    assert call(dwv_=(ctypes.c_void_p * 3)(FAKE + 20 * (1 << 32), FAKE + 91 * (1 << 32), FAKE + 92 * (1 << 32))) == \
        kda.KDA_ERR_INVALID_ARG                                        # a tap gradient over the text taps
