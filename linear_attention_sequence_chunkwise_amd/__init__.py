"""Python binding of libkda.so -- the KDA operator on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/kda.h``.  PyTorch provides
device memory and streams.  If the library is not built, importing works but
every call raises ``RuntimeError`` -- there is no fallback of any kind.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_F32 = 0
KDA_BF16 = 1
KDA_OK = 0
# kda_chain_form codes (kda_chunk_fwd_chain)
CHAIN_FORMS = {"auto": 0, "reg16": 1, "reg32": 2, "reg64": 3, "dma16": 4, "dma32": 5}
STATUS_NAMES = {0: "KDA_OK", 1: "KDA_ERR_NULL_ARG", 2: "KDA_ERR_BAD_SHAPE",
                3: "KDA_ERR_UNSUPPORTED", 4: "KDA_ERR_BAD_DTYPE", 5: "KDA_ERR_WORKSPACE",
                6: "KDA_ERR_HIP", 7: "KDA_ERR_SCRATCH"}

# name -> (restype, argtypes), mirroring include/kda.h
_P, _I, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


class KdaPrep(ctypes.Structure):
    """kda_prep of include/kda.h."""
    _fields_ = [("normalize_qk", ctypes.c_int), ("qk_eps", ctypes.c_float),
                ("beta_is_logit", ctypes.c_int), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p)]


class KdaEpilogue(ctypes.Structure):
    """kda_epilogue of include/kda.h."""
    _fields_ = [("eps", ctypes.c_float), ("weight", ctypes.c_void_p), ("gate", ctypes.c_void_p)]


_PREP = ctypes.POINTER(KdaPrep)
_EPI = ctypes.POINTER(KdaEpilogue)
SIGNATURES = {
    "kda_status_string": (ctypes.c_char_p, [_I]),
    "kda_version": (_I, []),
    "kda_chunk_fwd_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "kda_chunk_fwd_segments": (_I, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "kda_chunk_fwd": (_I, [_I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P, _P, _I,
                           _P, _P, _P, _SZ, _P]),
    "kda_chunk_fwd_ex": (_I, [_I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P, _P, _I,
                              _P, _P, _P, _SZ, _PREP, _EPI, _P]),
    "kda_chunk_fwd_chain": (_I, [_I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P, _P, _I,
                                 _P, _P, _P, _SZ, _PREP, _EPI, _I, _P]),
    "kda_chunk_fwd_noalloc": (_I, [_I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P, _P,
                                   _I, _P, _P, _P]),
    "kda_debug_chunk_intra_floats": (_SZ, [_I, _I]),
    "kda_debug_chunk_intra_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "kda_debug_chunk_intra": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "kda_chunk_bwd_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "kda_chunk_bwd": (_I, [_I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P, _P, _I,
                           _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "kda_dplr_chunk_fwd_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "kda_dplr_chunk_fwd": (_I, [_I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                _I, _P, _P, _P, _SZ, _P]),
    "kda_decode_step": (_I, [_I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P]),
    "kda_decode_step_ex": (_I, [_I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                _PREP, _EPI, _P]),
}

_lib = None


class KDAError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__("%s failed: %s" % (fn, kda_status_string(code)))


def load_library(path: str = LIB_PATH):
    """Load libkda.so (raises if it is missing: the HIP path is the only path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError("libkda.so is not built (%s); run "
                               "`python -m linear_attention_sequence_chunkwise_amd.build`" % path)
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def kda_status_string(code: int) -> str:
    try:
        return load_library().kda_status_string(int(code)).decode()
    except RuntimeError:
        return STATUS_NAMES.get(int(code), "KDA_ERR_UNKNOWN")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc_stream(stream):
    """Context under which the binding allocates: the launch stream, so that
    the caching allocator orders any reuse of a block after the kernels that
    use it (a block freed while other streams still run work on it could
    otherwise be handed out again too early)."""
    if stream is None:
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


def _check(t, name, dtype=None, device=None, shape=None):
    """Contiguity, dtype, device and exact shape of a tensor argument.  The C
    ABI sees only pointers, so this is the only place a mis-shaped buffer
    (one the kernels would read or write past) can be caught."""
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s" % (name, device))
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _on_gpu(t, name):
    """Host tensors would hand host pointers to the kernels."""
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor, got device %s" % (name, t.device))


def _dims(t, name, n):
    if t.dim() != n:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, n, tuple(t.shape)))
    return t.shape


def make_prep(prep, H, dk, device):
    """kda_prep from a dict: normalize_qk (bool), eps (float, default 1e-6),
    beta_logit (bool), A_log ([H] fp32 tensor or None), dt_bias ([H, dk] fp32
    tensor or None).  Returns (struct or None, tensors to keep alive)."""
    if prep is None:
        return None, ()
    a = prep.get("A_log")
    b = prep.get("dt_bias")
    _check(a, "A_log", torch.float32, device, (H,))
    _check(b, "dt_bias", torch.float32, device, (H, dk))
    st = KdaPrep(1 if prep.get("normalize_qk") else 0, float(prep.get("eps", 1e-6)),
                 1 if prep.get("beta_logit") else 0,
                 None if a is None else a.data_ptr(), None if b is None else b.data_ptr())
    return st, (a, b)


def make_epilogue(epilogue, dv, o_shape, qkv_dtype, device):
    """kda_epilogue from a dict: eps (float, default 1e-6), weight ([dv] fp32
    tensor or None), gate (tensor shaped like o in the q/k/v dtype, or None).
    Returns (struct or None, tensors to keep alive)."""
    if epilogue is None:
        return None, ()
    w = epilogue.get("weight")
    z = epilogue.get("gate")
    _check(w, "weight", torch.float32, device, (dv,))
    _check(z, "gate", qkv_dtype, device, o_shape)
    st = KdaEpilogue(float(epilogue.get("eps", 1e-6)), None if w is None else w.data_ptr(),
                     None if z is None else z.data_ptr())
    return st, (w, z)


def _prefill_shapes(q, k, v, g, beta, initial_state, cu_seqlens):
    """Sizes of a prefill-shaped call, every token tensor checked against q:
    q, k, g [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H]; initial_state
    [N, H, dk, dv]; cu_seqlens [N + 1] int32 with B = 1.  (beta None: not
    part of the call, or missing -- the C ABI reports the latter.)"""
    B, T, H, dk = _dims(q, "q", 4)
    dv = _dims(v, "v", 4)[-1]
    dev = q.device
    _check(q, "q", None, dev)
    for t, n in ((k, "k"), (v, "v")):
        _check(t, n, q.dtype, dev, (B, T, H, dk if n == "k" else dv))
    _check(g, "g", torch.float32, dev, (B, T, H, dk))
    _check(beta, "beta", torch.float32, dev, (B, T, H))
    N = B
    if cu_seqlens is not None:
        _dims(cu_seqlens, "cu_seqlens", 1)
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
        if B != 1:
            raise ValueError("cu_seqlens needs B == 1, got B = %d" % B)
        N = cu_seqlens.numel() - 1
    _check(initial_state, "initial_state", torch.float32, dev, (N, H, dk, dv))
    return B, T, H, dk, dv, N, dev


def kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, num_seqs=0, dtype=torch.bfloat16):
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load_library().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, num_seqs,
                                                             code))


def kda_chunk_fwd_segments(B, T, H, dk, dv, chunk, num_seqs=0, dtype=torch.bfloat16):
    """How the prefill's chain runs for these sizes: n > 1 segments per
    sequence, 1 the per-slice chain, -1 one workgroup per whole (sequence,
    head) chain, 0 unsupported sizes."""
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load_library().kda_chunk_fwd_segments(B, T, H, dk, dv, chunk, num_seqs, code))


def kda_chunk_fwd(q, k, v, g, beta, scale=None, chunk=64, initial_state=None, cu_seqlens=None,
                  output_final_state=True, o=None, final_state=None, workspace=None,
                  stream=None, prep=None, epilogue=None, chain_form=None):
    """Chunkwise KDA prefill.

    q, k: [B, T, H, dk]; v: [B, T, H, dv] (bf16 or fp32); g: [B, T, H, dk] fp32
    (log gate); beta: [B, T, H] fp32; initial_state: [N, H, dk, dv] fp32 or
    None; cu_seqlens: int32 [N + 1] (B must be 1) or None; prep: optional
    in-kernel input preparation (see make_prep); epilogue: optional output
    RMSNorm + gate (see make_epilogue).  With either, kda_chunk_fwd_ex is
    called.  chain_form: None, or a key of CHAIN_FORMS to force how the chain
    runs (kda_chunk_fwd_chain; for comparing forms).  Returns (o [B, T, H, dv]
    fp32, final_state [N, H, dk, dv] fp32 or None).
    """
    lib = load_library()
    B, T, H, dk, dv, N, dev = _prefill_shapes(q, k, v, g, beta, initial_state, cu_seqlens)
    if scale is None:
        scale = dk ** -0.5
    _check(o, "o", torch.float32, dev, (B, T, H, dv))
    _check(final_state, "final_state", torch.float32, dev, (N, H, dk, dv))
    code = _dtype_code(q)
    need = lib.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk,
                                             N if cu_seqlens is not None else 0, code)
    _check(workspace, "workspace", torch.uint8, dev)
    _on_gpu(q, "q")
    with _alloc_stream(stream):
        if o is None:
            o = torch.empty(B, T, H, dv, dtype=torch.float32, device=dev)
        if output_final_state and final_state is None:
            final_state = torch.empty(N, H, dk, dv, dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=dev)
    args = (B, T, H, dk, dv, chunk, float(scale), code, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
            _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
            N if cu_seqlens is not None else 0, _ptr(o), _ptr(final_state), _ptr(workspace),
            workspace.numel())
    if prep is None and epilogue is None and chain_form is None:
        rc = lib.kda_chunk_fwd(*args, _stream(stream))
        fn = "kda_chunk_fwd"
    else:
        st, _keep = make_prep(prep, H, dk, dev)
        et, _keep2 = make_epilogue(epilogue, dv, (B, T, H, dv), q.dtype, dev)
        pst = None if st is None else ctypes.byref(st)
        pet = None if et is None else ctypes.byref(et)
        if chain_form is None:
            rc = lib.kda_chunk_fwd_ex(*args, pst, pet, _stream(stream))
            fn = "kda_chunk_fwd_ex"
        else:
            rc = lib.kda_chunk_fwd_chain(*args, pst, pet, CHAIN_FORMS[chain_form],
                                         _stream(stream))
            fn = "kda_chunk_fwd_chain"
    if rc != KDA_OK:
        raise KDAError(fn, rc)
    return o, final_state


NOALLOC_SCRATCH_BYTES = 128 << 20   # KDA_NOALLOC_SCRATCH_BYTES


def kda_chunk_fwd_noalloc(q, k, v, g, beta, o, final_state=None, scale=None, chunk=64,
                          initial_state=None, cu_seqlens=None, stream=None):
    """kda_chunk_fwd through the entry point that allocates nothing: the
    library's fixed per-GPU scratch replaces the workspace, and the caller
    passes the outputs (o [B, T, H, dv] fp32, final_state [N, H, dk, dv] fp32
    or None).  Calls that overlap on one GPU race on that scratch.  Returns
    (o, final_state)."""
    lib = load_library()
    B, T, H, dk, dv, N, dev = _prefill_shapes(q, k, v, g, beta, initial_state, cu_seqlens)
    if o is None:
        raise ValueError("o must be given (this entry point allocates nothing)")
    _check(o, "o", torch.float32, dev, (B, T, H, dv))
    _check(final_state, "final_state", torch.float32, dev, (N, H, dk, dv))
    _on_gpu(q, "q")
    if scale is None:
        scale = dk ** -0.5
    rc = lib.kda_chunk_fwd_noalloc(B, T, H, dk, dv, chunk, float(scale), _dtype_code(q), _ptr(q),
                                   _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                   _ptr(cu_seqlens), N if cu_seqlens is not None else 0, _ptr(o),
                                   _ptr(final_state), _stream(stream))
    if rc != KDA_OK:
        raise KDAError("kda_chunk_fwd_noalloc", rc)
    return o, final_state


def kda_debug_chunk_intra(q, k, g, beta, chunk=64, stream=None):
    """Diagnostics (include/kda_debug.h): the intra-chunk kernel alone, its
    per-(chunk, head) results unpacked to fp32.  q, k, g [B, T, H, dk]; beta
    [B, T, H].  Returns a dict of tensors shaped [B, nchunk, H, ...]: KG, QG
    [C, dk]; KP [dk, C]; TB, MM, T, P [C, C]; GN [dk]."""
    lib = load_library()
    B, T, H, dk = _dims(q, "q", 4)
    dev = q.device
    _check(q, "q", None, dev)
    _check(k, "k", q.dtype, dev, (B, T, H, dk))
    _check(g, "g", torch.float32, dev, (B, T, H, dk))
    _check(beta, "beta", torch.float32, dev, (B, T, H))
    _on_gpu(q, "q")
    C = chunk
    code = _dtype_code(q)
    per = int(lib.kda_debug_chunk_intra_floats(dk, C))
    need = int(lib.kda_debug_chunk_intra_workspace_bytes(B, T, H, dk, C, code))
    if per == 0 or (need == 0 and T > 0):
        raise KDAError("kda_debug_chunk_intra", 3)
    nch = (T + C - 1) // C
    with _alloc_stream(stream):
        out = torch.zeros(B * nch * H * per, dtype=torch.float32, device=dev)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    rc = lib.kda_debug_chunk_intra(B, T, H, dk, C, code, _ptr(q), _ptr(k), _ptr(g), _ptr(beta),
                                   _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    if rc != KDA_OK:
        raise KDAError("kda_debug_chunk_intra", rc)
    out = out.view(B, nch, H, per)
    res, off = {}, 0
    for name, shape in (("KG", (C, dk)), ("QG", (C, dk)), ("KP", (dk, C)), ("TB", (C, C)),
                        ("MM", (C, C)), ("GN", (dk,)), ("T", (C, C)), ("P", (C, C))):
        n = 1
        for x in shape:
            n *= x
        res[name] = out[..., off:off + n].reshape(B, nch, H, *shape)
        off += n
    return res


def kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, chunk, num_seqs=0, dtype=torch.bfloat16):
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load_library().kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, chunk, num_seqs,
                                                             code))


def kda_chunk_bwd(q, k, v, g, beta, grad_o, scale=None, chunk=64, initial_state=None,
                  cu_seqlens=None, grad_final_state=None, want_grad_initial_state=True,
                  workspace=None, stream=None):
    """Gradients of kda_chunk_fwd (no preparation, no epilogue) for the loss
    <o, grad_o> + <final_state, grad_final_state>.

    Forward arguments as in kda_chunk_fwd; grad_o: [B, T, H, dv] fp32;
    grad_final_state: [N, H, dk, dv] fp32 or None (zero).  Returns (dq, dk, dv,
    dg, dbeta, d_initial_state), all fp32, the last None when not wanted.
    """
    lib = load_library()
    B, T, H, dk, dv, N, dev = _prefill_shapes(q, k, v, g, beta, initial_state, cu_seqlens)
    _check(grad_o, "grad_o", torch.float32, dev, (B, T, H, dv))
    _check(grad_final_state, "grad_final_state", torch.float32, dev, (N, H, dk, dv))
    _check(workspace, "workspace", torch.uint8, dev)
    _on_gpu(q, "q")
    if scale is None:
        scale = dk ** -0.5
    code = _dtype_code(q)
    nseq = N if cu_seqlens is not None else 0
    need = lib.kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, chunk, nseq, code)
    f = dict(dtype=torch.float32, device=dev)
    with _alloc_stream(stream):
        dq = torch.empty(B, T, H, dk, **f)
        dk_ = torch.empty(B, T, H, dk, **f)
        dv_ = torch.empty(B, T, H, dv, **f)
        dg = torch.empty(B, T, H, dk, **f)
        db = torch.empty(B, T, H, **f)
        dS0 = torch.empty(N, H, dk, dv, **f) if want_grad_initial_state else None
        if workspace is None:
            workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=dev)
    rc = lib.kda_chunk_bwd(B, T, H, dk, dv, chunk, float(scale), code, _ptr(q), _ptr(k),
                           _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
                           nseq, _ptr(grad_o), _ptr(grad_final_state), _ptr(dq), _ptr(dk_),
                           _ptr(dv_), _ptr(dg), _ptr(db), _ptr(dS0), _ptr(workspace),
                           workspace.numel(), _stream(stream))
    if rc != KDA_OK:
        raise KDAError("kda_chunk_bwd", rc)
    return dq, dk_, dv_, dg, db, dS0


def kda_dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, num_seqs=0,
                                       dtype=torch.bfloat16):
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load_library().kda_dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk,
                                                                  num_seqs, code))


def kda_dplr_chunk_fwd(q, k, v, a, b, g, scale=None, chunk=64, initial_state=None,
                       cu_seqlens=None, output_final_state=True, o=None, final_state=None,
                       workspace=None, stream=None):
    """Chunkwise forward of the general diagonal-plus-low-rank recurrence
    S_t = (Diag(exp(g_t)) - a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = scale S_t^T q_t.
    q, k, a, b: [B, T, H, dk]; v: [B, T, H, dv] (all bf16 or all fp32); g:
    [B, T, H, dk] fp32; the rest as in kda_chunk_fwd.  Returns (o, final_state)."""
    lib = load_library()
    B, T, H, dk, dv, N, dev = _prefill_shapes(q, k, v, g, None, initial_state, cu_seqlens)
    for t, n in ((a, "a"), (b, "b")):
        _check(t, n, q.dtype, dev, (B, T, H, dk))
    _check(o, "o", torch.float32, dev, (B, T, H, dv))
    _check(final_state, "final_state", torch.float32, dev, (N, H, dk, dv))
    _check(workspace, "workspace", torch.uint8, dev)
    _on_gpu(q, "q")
    if scale is None:
        scale = dk ** -0.5
    code = _dtype_code(q)
    nseq = N if cu_seqlens is not None else 0
    need = lib.kda_dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, nseq, code)
    with _alloc_stream(stream):
        if o is None:
            o = torch.empty(B, T, H, dv, dtype=torch.float32, device=dev)
        if output_final_state and final_state is None:
            final_state = torch.empty(N, H, dk, dv, dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=dev)
    rc = lib.kda_dplr_chunk_fwd(B, T, H, dk, dv, chunk, float(scale), code, _ptr(q), _ptr(k),
                                _ptr(v), _ptr(a), _ptr(b), _ptr(g), _ptr(initial_state),
                                _ptr(cu_seqlens), nseq, _ptr(o), _ptr(final_state),
                                _ptr(workspace), workspace.numel(), _stream(stream))
    if rc != KDA_OK:
        raise KDAError("kda_dplr_chunk_fwd", rc)
    return o, final_state


def kda_decode_step(q, k, v, g, beta, state_cache, scale=None, slot_idx=None, o=None,
                    stream=None, prep=None, epilogue=None):
    """One decode step.  q, k, g: [N, H, dk]; v: [N, H, dv]; beta: [N, H];
    state_cache: [num_slots, H, dk, dv] fp32, updated in place; slot_idx:
    int32 [N] or None; prep and epilogue as in kda_chunk_fwd.  Returns
    o [N, H, dv] fp32."""
    lib = load_library()
    N, H, dk = _dims(q, "q", 3)
    dv = _dims(v, "v", 3)[-1]
    dev = q.device
    _check(q, "q", None, dev)
    _check(k, "k", q.dtype, dev, (N, H, dk))
    _check(v, "v", q.dtype, dev, (N, H, dv))
    _check(g, "g", torch.float32, dev, (N, H, dk))
    _check(beta, "beta", torch.float32, dev, (N, H))
    slots = _dims(state_cache, "state_cache", 4)[0]
    _check(state_cache, "state_cache", torch.float32, dev, (slots, H, dk, dv))
    _check(slot_idx, "slot_idx", torch.int32, dev, (N,))
    _check(o, "o", torch.float32, dev, (N, H, dv))
    _on_gpu(q, "q")
    if scale is None:
        scale = dk ** -0.5
    if o is None:
        with _alloc_stream(stream):
            o = torch.empty(N, H, dv, dtype=torch.float32, device=dev)
    args = (N, H, dk, dv, float(scale), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
            _ptr(beta), _ptr(state_cache), state_cache.shape[0], _ptr(slot_idx), _ptr(o))
    if prep is None and epilogue is None:
        rc = lib.kda_decode_step(*args, _stream(stream))
        fn = "kda_decode_step"
    else:
        st, _keep = make_prep(prep, H, dk, dev)
        et, _keep2 = make_epilogue(epilogue, dv, (N, H, dv), q.dtype, dev)
        rc = lib.kda_decode_step_ex(*args, None if st is None else ctypes.byref(st),
                                    None if et is None else ctypes.byref(et), _stream(stream))
        fn = "kda_decode_step_ex"
    if rc != KDA_OK:
        raise KDAError(fn, rc)
    return o
