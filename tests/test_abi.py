"""CPU tests of the C-ABI library: it loads without a GPU, exports every
symbol include/kda.h declares, and rejects bad arguments on the host before
any HIP call (these calls never reach the device)."""
import ctypes
import os
import re

import pytest

import linear_attention_sequence_chunkwise_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
DEBUG_HEADER = os.path.join(ROOT, "include", "kda_debug.h")


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.fail("libkda.so not built; run python -m linear_attention_sequence_chunkwise_amd.build")
    return kda.load_library()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == {"kda_status_string", "kda_version", "kda_chunk_fwd_workspace_bytes",
                          "kda_chunk_fwd_segments",
                          "kda_chunk_fwd", "kda_chunk_fwd_ex", "kda_chunk_fwd_chain",
                          "kda_chunk_fwd_noalloc",
                          "kda_decode_step",
                          "kda_decode_step_ex", "kda_chunk_bwd_workspace_bytes",
                          "kda_chunk_bwd", "kda_dplr_chunk_fwd_workspace_bytes",
                          "kda_dplr_chunk_fwd"}
    for n in names:
        assert hasattr(lib, n), n
        assert n in kda.SIGNATURES, n


def test_exports_debug_symbols(lib):
    names = header_functions(DEBUG_HEADER)
    assert set(names) == {"kda_debug_chunk_intra_floats", "kda_debug_chunk_intra_workspace_bytes",
                          "kda_debug_chunk_intra"}
    for n in names:
        assert hasattr(lib, n), n
        assert n in kda.SIGNATURES, n
    assert lib.kda_debug_chunk_intra_floats(128, 64) == 3 * 64 * 128 + 4 * 64 * 64 + 128
    assert lib.kda_debug_chunk_intra_floats(48, 64) == 0
    E = {v: k for k, v in kda.STATUS_NAMES.items()}
    p = ctypes.c_void_p(4096)
    assert lib.kda_debug_chunk_intra(1, 64, 2, 64, 128, kda.KDA_BF16, p, p, p, p, p, p, 1 << 30,
                                     None) == E["KDA_ERR_UNSUPPORTED"]
    assert lib.kda_debug_chunk_intra(1, 64, 2, 64, 64, kda.KDA_BF16, p, p, p, p, p, p, 16,
                                     None) == E["KDA_ERR_WORKSPACE"]


def test_status_strings(lib):
    for code, name in kda.STATUS_NAMES.items():
        assert kda.kda_status_string(code).startswith(name)
    assert lib.kda_version() == 100


def test_workspace_size(lib):
    ws = lib.kda_chunk_fwd_workspace_bytes
    # B=1 T=32768 H=32 d=128 C=64 bf16: 512 chunks x 32 heads x record; a bf16
    # record holds three C x d and one C x C fp16 tiles (the products with T diag
    # beta folded in) plus d fp32 decays, in whole KiB
    rec = (3 * 64 * 128 + 64 * 64) * 2 + 4 * 128
    rec = (rec + 1023) // 1024 * 1024
    # plus, with 32 (sequence, head) chains cut into 8 segments, 3 * 8 - 3 fp32
    # d x d state planes per chain (end states, transition products, entering
    # states)
    assert ws(1, 32768, 32, 128, 128, 64, 0, kda.KDA_BF16) == 512 * 32 * rec + 21 * 32 * 128 * 128 * 4
    assert ws(1, 100, 2, 64, 64, 16, 0, kda.KDA_F32) > ws(1, 100, 2, 64, 64, 16, 0, kda.KDA_BF16)
    # packed sequences add a chunk table and room for one partial chunk per sequence
    assert ws(1, 1000, 2, 64, 64, 64, 5, kda.KDA_BF16) > ws(1, 1000, 2, 64, 64, 64, 1, kda.KDA_BF16)
    assert ws(1, 100, 2, 64, 32, 64, 0, kda.KDA_BF16) == 0      # dk != dv
    assert ws(1, 100, 2, 96, 96, 64, 0, kda.KDA_BF16) == 0      # unsupported d
    assert ws(1, 100, 2, 64, 64, 48, 0, kda.KDA_BF16) == 0      # unsupported chunk
    assert ws(2, 100, 2, 64, 64, 64, 3, kda.KDA_BF16) == 0      # packed needs B == 1
    assert ws(1, 100, 2, 64, 64, 64, 0, 7) == 0                 # bad dtype
    # at most 2^24 - 1 (chunk, head) pairs: one workgroup each in a 1-D grid
    assert ws(1, 64 * ((1 << 22) - 1), 4, 64, 64, 64, 0, kda.KDA_BF16) > 0
    assert ws(1, 64 * (1 << 22), 4, 64, 64, 64, 0, kda.KDA_BF16) == 0
    # K1 reads a chunk's rows through 32-bit byte offsets: chunk * H * dk * 4 < 2^31
    assert ws(1, 64, (1 << 16) - 1, 128, 128, 64, 0, kda.KDA_BF16) > 0
    assert ws(1, 64, 1 << 16, 128, 128, 64, 0, kda.KDA_BF16) == 0


def test_chain_segments(lib):
    seg = lib.kda_chunk_fwd_segments
    # 32 chains, 512 chunks: 8 segments of 64 chunks cover 256 CUs
    assert seg(1, 32768, 32, 128, 128, 64, 0, kda.KDA_BF16) == 8
    # at least 4 chunks per segment: 40 chunks allow 10, the CUs ask for 64
    assert seg(1, 40 * 64, 4, 64, 64, 64, 0, kda.KDA_BF16) == 10
    assert seg(2, 32768, 32, 128, 128, 64, 0, kda.KDA_BF16) == 4
    # 256 chains already: one workgroup per whole chain; also from 128 chains on
    assert seg(8, 32768, 32, 128, 128, 64, 0, kda.KDA_BF16) == -1
    assert seg(4, 32768, 32, 128, 128, 64, 0, kda.KDA_BF16) == 2
    assert seg(5, 32768, 32, 128, 128, 64, 0, kda.KDA_BF16) == -1
    assert seg(1, 32768, 127, 128, 128, 64, 0, kda.KDA_BF16) == 2
    # packed sequences: the per-slice chain below 128 chains, whole chains from there
    assert seg(1, 32768, 32, 128, 128, 64, 3, kda.KDA_BF16) == 1
    assert seg(1, 32768, 32, 128, 128, 64, 4, kda.KDA_BF16) == -1
    assert seg(1, 7 * 64, 32, 128, 128, 64, 0, kda.KDA_BF16) == 1    # too short to split
    assert seg(1, 32768, 32, 128, 128, 64, 0, kda.KDA_F32) == 1      # fp32 d=128 C=64: LDS
    assert seg(1, 32768, 32, 64, 64, 64, 0, kda.KDA_F32) == 1        # fp32 d=64 C=64: LDS
    assert seg(1, 32768, 32, 64, 64, 32, 0, kda.KDA_F32) == 8
    assert seg(1, 32768, 32, 96, 96, 64, 0, kda.KDA_BF16) == 0       # unsupported
    # one chain: the CUs would take 256 segments, the combine's depth caps it at 32
    assert seg(1, 32768, 1, 128, 128, 64, 0, kda.KDA_BF16) == 32


def test_workspace_monotone_in_T(lib):
    ws = lib.kda_chunk_fwd_workspace_bytes
    for B, H, d, c in ((1, 32, 128, 64), (1, 4, 64, 16), (3, 2, 32, 32)):
        sizes = [ws(B, T, H, d, d, c, 0, kda.KDA_BF16) for T in range(0, 4000, 37)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:])), (B, H, d, c)


def _fwd(lib, B=1, T=64, H=2, dk=64, dv=64, chunk=64, dtype=kda.KDA_BF16, ptr=4096, cu=None,
         nseq=0, ws=None, wsb=1 << 30, o=None):
    p = ctypes.c_void_p(ptr)
    return lib.kda_chunk_fwd(B, T, H, dk, dv, chunk, 1.0, dtype, p, p, p, p, p, None, cu, nseq,
                             p if o is None else o, None, p if ws is None else ws, wsb, None)


def test_prefill_validation(lib):
    E = {v: k for k, v in kda.STATUS_NAMES.items()}
    assert _fwd(lib, B=0) == E["KDA_ERR_BAD_SHAPE"]
    assert _fwd(lib, T=-1) == E["KDA_ERR_BAD_SHAPE"]
    assert _fwd(lib, H=0) == E["KDA_ERR_BAD_SHAPE"]
    assert _fwd(lib, dtype=9) == E["KDA_ERR_BAD_DTYPE"]
    assert _fwd(lib, dk=64, dv=32) == E["KDA_ERR_UNSUPPORTED"]
    assert _fwd(lib, dk=48, dv=48) == E["KDA_ERR_UNSUPPORTED"]
    assert _fwd(lib, chunk=128) == E["KDA_ERR_UNSUPPORTED"]
    assert _fwd(lib, ptr=0) == E["KDA_ERR_NULL_ARG"]
    assert _fwd(lib, ptr=4098) == E["KDA_ERR_NULL_ARG"]          # misaligned
    assert _fwd(lib, B=2, cu=ctypes.c_void_p(4096), nseq=2) == E["KDA_ERR_BAD_SHAPE"]
    assert _fwd(lib, cu=ctypes.c_void_p(4096), nseq=0) == E["KDA_ERR_BAD_SHAPE"]
    assert _fwd(lib, wsb=16) == E["KDA_ERR_WORKSPACE"]
    assert _fwd(lib, ws=ctypes.c_void_p(4096 + 16)) == E["KDA_ERR_WORKSPACE"]  # not 256-aligned


def _fwd_chain(lib, form, dtype=kda.KDA_BF16, dk=64, chunk=64):
    p = ctypes.c_void_p(4096)
    return lib.kda_chunk_fwd_chain(1, 0, 2, dk, dk, chunk, 1.0, dtype, p, p, p, p, p, None, None,
                                   0, p, None, p, 1 << 30, None, None, form, None)


def test_chain_form_validation(lib):
    """Forms outside kda_chain_form, or not built for the sizes, are rejected
    on the host (T = 0 keeps valid calls from reaching the device)."""
    E = {v: k for k, v in kda.STATUS_NAMES.items()}
    assert _fwd_chain(lib, -1) == E["KDA_ERR_UNSUPPORTED"]
    assert _fwd_chain(lib, 6) == E["KDA_ERR_UNSUPPORTED"]
    assert _fwd_chain(lib, kda.CHAIN_FORMS["reg32"], dtype=kda.KDA_F32) == E["KDA_ERR_UNSUPPORTED"]
    assert _fwd_chain(lib, kda.CHAIN_FORMS["reg64"], dk=32, chunk=16) == E["KDA_ERR_UNSUPPORTED"]
    assert _fwd_chain(lib, kda.CHAIN_FORMS["dma16"], dtype=kda.KDA_F32) == E["KDA_ERR_UNSUPPORTED"]


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


def test_no_device_reports_hip_error(lib):
    """Valid arguments with no usable GPU: every entry point returns
    KDA_ERR_HIP from its device query instead of crashing (the pointers are
    never touched)."""
    if _gpu_visible():
        pytest.skip("a GPU is visible: valid calls would launch kernels")
    E = {v: k for k, v in kda.STATUS_NAMES.items()}
    p = ctypes.c_void_p(4096)
    assert _fwd(lib) == E["KDA_ERR_HIP"]
    assert lib.kda_decode_step(2, 2, 64, 64, 1.0, kda.KDA_BF16, p, p, p, p, p, p, 2, None, p,
                               None) == E["KDA_ERR_HIP"]
    assert lib.kda_chunk_bwd(1, 64, 2, 64, 64, 64, 1.0, kda.KDA_BF16, p, p, p, p, p, None, None,
                             0, p, None, p, p, p, p, p, None, p, 1 << 34, None) == E["KDA_ERR_HIP"]
    assert lib.kda_dplr_chunk_fwd(1, 64, 2, 64, 64, 64, 1.0, kda.KDA_BF16, p, p, p, p, p, p, None,
                                  None, 0, p, None, p, 1 << 30, None) == E["KDA_ERR_HIP"]
    assert lib.kda_chunk_fwd_noalloc(1, 64, 2, 64, 64, 64, 1.0, kda.KDA_BF16, p, p, p, p, p, None,
                                     None, 0, p, None, None) == E["KDA_ERR_HIP"]


def test_noalloc_validation(lib):
    """The no-allocation entry point refuses calls whose workspace would not
    fit its fixed scratch, on the host, with KDA_ERR_SCRATCH."""
    E = {v: k for k, v in kda.STATUS_NAMES.items()}
    p = ctypes.c_void_p(4096)
    big = lib.kda_chunk_fwd_noalloc(1, 8192, 32, 128, 128, 64, 1.0, kda.KDA_BF16, p, p, p, p, p,
                                    None, None, 0, p, None, None)
    assert big == E["KDA_ERR_SCRATCH"]
    assert lib.kda_chunk_fwd_workspace_bytes(1, 8192, 32, 128, 128, 64, 0, kda.KDA_BF16) > \
        kda.NOALLOC_SCRATCH_BYTES
    assert lib.kda_chunk_fwd_noalloc(1, 64, 2, 48, 48, 64, 1.0, kda.KDA_BF16, p, p, p, p, p,
                                     None, None, 0, p, None, None) == E["KDA_ERR_UNSUPPORTED"]


def test_decode_validation(lib):
    E = {v: k for k, v in kda.STATUS_NAMES.items()}
    p = ctypes.c_void_p(4096)

    def dec(N=2, H=2, dk=64, dv=64, dtype=kda.KDA_BF16, ptr=p, slots=4, idx=None):
        return lib.kda_decode_step(N, H, dk, dv, 1.0, dtype, ptr, ptr, ptr, ptr, ptr, ptr, slots,
                                   idx, ptr, None)
    assert dec(N=-1) == E["KDA_ERR_BAD_SHAPE"]
    assert dec(N=5, slots=4) == E["KDA_ERR_BAD_SHAPE"]          # identity slots need N <= slots
    assert dec(dtype=3) == E["KDA_ERR_BAD_DTYPE"]
    assert dec(dk=64, dv=128) == E["KDA_ERR_UNSUPPORTED"]
    assert dec(dk=256, dv=256) == E["KDA_ERR_UNSUPPORTED"]
    assert dec(ptr=None) == E["KDA_ERR_NULL_ARG"]
    assert dec(ptr=ctypes.c_void_p(4100)) == E["KDA_ERR_NULL_ARG"]
    assert dec(N=0) == E["KDA_OK"]                              # nothing to do, nothing launched


def test_prep_and_epilogue_validation(lib):
    """A malformed kda_prep or kda_epilogue is rejected on the host, before any
    HIP call."""
    E = {v: k for k, v in kda.STATUS_NAMES.items()}
    p = ctypes.c_void_p(4096)

    def fwd(prep=None, epi=None):
        return lib.kda_chunk_fwd_ex(1, 64, 2, 64, 64, 64, 1.0, kda.KDA_BF16, p, p, p, p, p,
                                    None, None, 0, p, None, p, 1 << 30,
                                    None if prep is None else ctypes.byref(prep),
                                    None if epi is None else ctypes.byref(epi), None)

    def dec(prep=None, epi=None):
        return lib.kda_decode_step_ex(2, 2, 64, 64, 1.0, kda.KDA_BF16, p, p, p, p, p, p, 2,
                                      None, p, None if prep is None else ctypes.byref(prep),
                                      None if epi is None else ctypes.byref(epi), None)

    bias_only = kda.KdaPrep(0, 1e-6, 0, None, 4096)
    bad_eps = kda.KdaPrep(1, -1.0, 0, None, None)
    nan_eps = kda.KdaPrep(1, float("nan"), 0, None, None)
    odd_ptr = kda.KdaPrep(0, 0.0, 0, 4098, None)
    epi_bad_eps = kda.KdaEpilogue(-1e-3, None, None)
    epi_inf_eps = kda.KdaEpilogue(float("inf"), None, None)
    epi_odd_w = kda.KdaEpilogue(1e-6, 4098, None)
    epi_odd_gate = kda.KdaEpilogue(1e-6, None, 4100)
    for call in (fwd, dec):
        assert call(prep=bias_only) == E["KDA_ERR_NULL_ARG"]
        assert call(prep=bad_eps) == E["KDA_ERR_BAD_SHAPE"]
        assert call(prep=nan_eps) == E["KDA_ERR_BAD_SHAPE"]
        assert call(prep=odd_ptr) == E["KDA_ERR_NULL_ARG"]
        assert call(epi=epi_bad_eps) == E["KDA_ERR_BAD_SHAPE"]
        assert call(epi=epi_inf_eps) == E["KDA_ERR_BAD_SHAPE"]
        assert call(epi=epi_odd_w) == E["KDA_ERR_NULL_ARG"]
        assert call(epi=epi_odd_gate) == E["KDA_ERR_NULL_ARG"]


def test_backward_workspace_and_validation(lib):
    """The backward's workspace holds fp32 chunk records plus, per (chunk,
    head), T and the k Gram (C x C each), two fp32 states, four C x d tiles
    (X, U, dU, dX) and a gradient record; bad arguments are rejected on the
    host."""
    E = {v: k for k, v in kda.STATUS_NAMES.items()}
    wf = lib.kda_chunk_fwd_workspace_bytes
    wb = lib.kda_chunk_bwd_workspace_bytes
    nch, H, d, C = 512, 32, 128, 64
    grec = (3 * C * d + 2 * C * C + d + 63) // 64 * 64
    # fp32 chunk records for either input type
    assert wb(1, 32768, H, d, d, C, 0, kda.KDA_BF16) == (
        wf(1, 32768, H, d, d, C, 0, kda.KDA_F32) + nch * H * 2 * C * C * 4 +
        2 * nch * H * d * d * 4 + 4 * nch * H * C * d * 4 + nch * H * grec * 4)
    assert wb(1, 32768, H, d, d, C, 0, kda.KDA_BF16) == wb(1, 32768, H, d, d, C, 0, kda.KDA_F32)
    assert wb(1, 100, 2, 64, 32, 64, 0, kda.KDA_BF16) == 0
    assert wb(1, 100, 2, 64, 64, 48, 0, kda.KDA_BF16) == 0
    assert wb(2, 100, 2, 64, 64, 64, 3, kda.KDA_BF16) == 0
    # at most 2^23 - 1 (chunk, head) pairs (512-thread workgroups in a 1-D grid)
    assert wb(1, 64 * ((1 << 21) - 1), 4, 64, 64, 64, 0, kda.KDA_BF16) > 0
    assert wb(1, 64 * (1 << 21), 4, 64, 64, 64, 0, kda.KDA_BF16) == 0
    p = ctypes.c_void_p(4096)

    def bwd(B=1, T=64, H=2, dk=64, dv=64, chunk=64, dtype=kda.KDA_BF16, ptr=p, gb=p, dS0=None,
            cu=None, nseq=0, ws=p, wsb=1 << 34):
        return lib.kda_chunk_bwd(B, T, H, dk, dv, chunk, 1.0, dtype, ptr, ptr, ptr, ptr, ptr,
                                 None, cu, nseq, ptr, None, ptr, ptr, ptr, ptr, gb, dS0, ws, wsb,
                                 None)
    assert bwd(B=0) == E["KDA_ERR_BAD_SHAPE"]
    assert bwd(dtype=5) == E["KDA_ERR_BAD_DTYPE"]
    assert bwd(dk=64, dv=128) == E["KDA_ERR_UNSUPPORTED"]
    assert bwd(chunk=8) == E["KDA_ERR_UNSUPPORTED"]
    assert bwd(ptr=None) == E["KDA_ERR_NULL_ARG"]
    assert bwd(ptr=ctypes.c_void_p(4104)) == E["KDA_ERR_NULL_ARG"]
    assert bwd(gb=ctypes.c_void_p(4098)) == E["KDA_ERR_NULL_ARG"]     # grad_beta: 4-byte
    assert bwd(dS0=ctypes.c_void_p(4100)) == E["KDA_ERR_NULL_ARG"]
    assert bwd(B=2, cu=p, nseq=2) == E["KDA_ERR_BAD_SHAPE"]
    assert bwd(wsb=1024) == E["KDA_ERR_WORKSPACE"]
    assert bwd(ws=ctypes.c_void_p(4096 + 64)) == E["KDA_ERR_WORKSPACE"]


def test_dplr_workspace_and_validation(lib):
    """The DPLR record holds two C x d and two d x C tiles, three C x C tiles and
    d fp32 decays; the fp32 chunk-64 tiles at d = 128 do not fit LDS."""
    E = {v: k for k, v in kda.STATUS_NAMES.items()}
    ws = lib.kda_dplr_chunk_fwd_workspace_bytes
    rec = (2 * 64 * 128 + 2 * 128 * 64 + 3 * 64 * 64) * 2 + 4 * 128
    rec = (rec + 1023) // 1024 * 1024
    assert ws(1, 32768, 32, 128, 128, 64, 0, kda.KDA_BF16) == 512 * 32 * rec
    assert ws(1, 100, 2, 128, 128, 64, 0, kda.KDA_F32) == 0
    assert ws(1, 100, 2, 128, 128, 32, 0, kda.KDA_F32) > 0
    assert ws(1, 100, 2, 64, 32, 64, 0, kda.KDA_BF16) == 0
    p = ctypes.c_void_p(4096)

    def fwd(B=1, T=64, H=2, dk=64, dv=64, chunk=64, dtype=kda.KDA_BF16, ptr=p, ab=p, wsb=1 << 30):
        return lib.kda_dplr_chunk_fwd(B, T, H, dk, dv, chunk, 1.0, dtype, ptr, ptr, ptr, ab, ab,
                                      ptr, None, None, 0, ptr, None, p, wsb, None)
    assert fwd(B=0) == E["KDA_ERR_BAD_SHAPE"]
    assert fwd(dtype=3) == E["KDA_ERR_BAD_DTYPE"]
    assert fwd(chunk=48) == E["KDA_ERR_UNSUPPORTED"]
    assert fwd(dk=128, dv=128, dtype=kda.KDA_F32) == E["KDA_ERR_UNSUPPORTED"]
    assert fwd(ab=None) == E["KDA_ERR_NULL_ARG"]
    assert fwd(ab=ctypes.c_void_p(4104)) == E["KDA_ERR_NULL_ARG"]
    assert fwd(wsb=64) == E["KDA_ERR_WORKSPACE"]
