"""fp64 CPU oracle for the Kimi Delta Attention (KDA) operator.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  It
shares no code with the HIP path and never imports it; the two meet only in
the seeded input generators of ``kda_inputs``.

Contents
--------
* ``kda_fwd`` / ``kda_decode_step``: the token-by-token fp64 recurrence in C
  (``kda_oracle.c``, OpenMP over independent (sequence, head) chains) -- the
  reference every GPU result is compared with.
* ``kda_bwd``: exact gradients by reverse mode through the same token loop.
* ``dplr_fwd``: the general diagonal-plus-low-rank recurrence
  S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T, of which KDA is the
  case a = beta k, b = alpha * k with write key beta k.
* NumPy fp64 forms for one (sequence, head) chain, used only to pin the C
  oracle to something other than itself (see ``tests/test_oracle_pins.py``):

  - ``recurrence_np``    the delta-rule token loop, written out again in NumPy;
  - ``bruteforce_np``    the literal matrix product (I - b k k^T) Diag(a) S + b k v^T;
  - ``chunked_np``       the chunkwise WY/UT form, derived from the recurrence
    (its per-chunk quantities from ``chunk_terms_np``);
  - ``linear_attention_closed_form``, ``scalar_gated_deltanet_np``: the textbook
    special cases the method reduces to.

Source of the method: the GeekNews summary of Kimi Linear (es.news.hada.io,
topic 31936) and its Indonesian twin (id.news.hada.io, topic 31936) --
sections "De la atencion lineal a Gated DeltaNet" (fast-weight state, delta
rule as online gradient descent, rank-1 generalised Householder update,
scalar forget gate), "Control fino de memoria en Kimi Delta Attention"
(per-channel diagonal gate, DPLR transition tied to the key) and "Algoritmo
paralelo por chunks" (chunks that hand their final state to the next, WY
packing, UT transform, forward substitution, intra/inter split).  The pages
print no formula; the recurrence used is

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = scale * S_t^T q_t,      alpha_t = exp(g_t).

Parity status: every function here is pinned (closed forms, invariants,
brute force on tiny inputs, hand-computed scalar fixture).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_kda.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (OpenMP) into ``liboracle_kda.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_kda_fwd.argtypes = [I, I, I, I, I, D, P, P, P, P, P, P, P, I, I, P, P]
        lib.oracle_kda_fwd.restype = I
        lib.oracle_kda_decode_step.argtypes = [I, I, I, I, D, P, P, P, P, P, P, I, P, P]
        lib.oracle_kda_decode_step.restype = I
        lib.oracle_kda_fwd_ex.argtypes = [I, I, I, I, I, D, P, P, P, P, P, P, P, I, I, D, P, P,
                                          I, D, P, P, P, P]
        lib.oracle_kda_fwd_ex.restype = I
        lib.oracle_kda_decode_step_ex.argtypes = [I, I, I, I, D, P, P, P, P, P, P, I, P, I, D,
                                                  P, P, I, D, P, P, P]
        lib.oracle_kda_decode_step_ex.restype = I
        lib.oracle_kda_bwd.argtypes = [I, I, I, I, I, D, P, P, P, P, P, P, P, I, P, P, P, P, P, P,
                                       P, P]
        lib.oracle_kda_bwd.restype = I
        lib.oracle_dplr_fwd.argtypes = [I, I, I, I, I, D, P, P, P, P, P, P, P, P, I, P, P]
        lib.oracle_dplr_fwd.restype = I
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = I
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the C oracle uses (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_num_threads())


def _f32(a):
    a = np.asarray(a)
    if a.dtype != np.float32:
        # bf16 arrive upcast to float32 by the caller; float64 test inputs are
        # rounded to float32 here and the tests build their expectations from
        # these same float32 values.
        a = a.astype(np.float32)
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep_args(prep, H, dk):
    """(flags, eps, A_log, dt_bias) for the C oracle from a prep dict:
    normalize_qk (bool), eps (float), beta_logit (bool), A_log ([H] or None),
    dt_bias ([H, dk] or None).  See prepare_token in kda_oracle.c."""
    flags = (1 if prep.get("normalize_qk") else 0) | (2 if prep.get("beta_logit") else 0)
    a = prep.get("A_log")
    b = prep.get("dt_bias")
    a = None if a is None else _f32(a).reshape(H)
    b = None if b is None else _f32(b).reshape(H, dk)
    return flags, float(prep.get("eps", 1e-6)), a, b


def _epi_args(epi, shape_o, dv):
    """(on, eps, w, z) for the C oracle from an epilogue dict: eps (float),
    weight ([dv] or None), gate ([..., dv] shaped like o, or None).  See
    epilogue_row in kda_oracle.c."""
    if epi is None:
        return 0, 0.0, None, None
    w = epi.get("weight")
    z = epi.get("gate")
    w = None if w is None else _f32(w).reshape(dv)
    z = None if z is None else _f32(z).reshape(shape_o)
    return 1, float(epi.get("eps", 1e-6)), w, z


def kda_fwd(q, k, v, g, beta, scale, S0=None, cu_seqlens=None, drop_erase=False, prep=None,
            epilogue=None):
    """Exact KDA forward in fp64.

    q, k, g: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H] (float32 values,
    upcast to fp64 inside).  S0: [N, H, dk, dv] or None.  cu_seqlens: int32
    [N + 1] or None (then N = B).  prep: optional input preparation (see
    _prep_args): L2 normalisation of q and k, beta given as logits, g given as
    the gate pre-activation of the Mamba/GDN-style decay.  epilogue: optional
    per-head RMSNorm + sigmoid output gate applied to every output row (see
    _epi_args).  Returns (o [B, T, H, dv], S [N, H, dk, dv]), both float64.
    """
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape and v.shape[:3] == (B, T, H)
    assert beta.shape == (B, T, H)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        cu = None
        N = B
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
        assert s0.shape == (N, H, dk, dv)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S = np.zeros((N, H, dk, dv), dtype=np.float64)
    if prep is not None or epilogue is not None:
        assert not drop_erase
        flags, eps, a, b = _prep_args(prep or {}, H, dk)
        on, e_eps, w, z = _epi_args(epilogue, (B, T, H, dv), dv)
        rc = _load().oracle_kda_fwd_ex(B, T, H, dk, dv, float(scale), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(cu), N,
                                       flags, eps, _ptr(a), _ptr(b), on, e_eps, _ptr(w), _ptr(z),
                                       _ptr(o), _ptr(S))
    else:
        rc = _load().oracle_kda_fwd(B, T, H, dk, dv, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(g), _ptr(beta), _ptr(s0), _ptr(cu), N,
                                    1 if drop_erase else 0, _ptr(o), _ptr(S))
    if rc != 0:
        raise ValueError("oracle_kda_fwd rejected its arguments (code %d)" % rc)
    return o, S


def kda_bwd(q, k, v, g, beta, scale, d_o, S0=None, cu_seqlens=None, d_S_final=None):
    """Exact gradients of L = sum(o * d_o) + sum(S_final * d_S_final) in fp64
    (reverse mode through the token recurrence).  Shapes as in kda_fwd; d_o
    like o, d_S_final like the final state (None = 0).  Returns
    (dq, dk, dv, dg, dbeta, dS0), float64; dS0 has the initial state's shape."""
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        cu = None
        N = B
    s0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
    do = np.ascontiguousarray(np.asarray(d_o, dtype=np.float64))
    assert do.shape == (B, T, H, dv)
    dsf = None if d_S_final is None else np.ascontiguousarray(np.asarray(d_S_final, np.float64))
    dq = np.zeros((B, T, H, dk))
    dkk = np.zeros((B, T, H, dk))
    dvv = np.zeros((B, T, H, dv))
    dg = np.zeros((B, T, H, dk))
    db = np.zeros((B, T, H))
    dS0 = np.zeros((N, H, dk, dv))
    rc = _load().oracle_kda_bwd(B, T, H, dk, dv, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(s0), _ptr(cu), N, _ptr(do), _ptr(dsf), _ptr(dq),
                                _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(db), _ptr(dS0))
    if rc != 0:
        raise ValueError("oracle_kda_bwd rejected its arguments (code %d)" % rc)
    return dq, dkk, dvv, dg, db, dS0


def kda_decode_step(q, k, v, g, beta, scale, state, slot_idx=None, prep=None, epilogue=None):
    """One exact decode step.  q, k, g [N, H, dk]; v [N, H, dv]; beta [N, H];
    state: float64 [num_slots, H, dk, dv], updated IN PLACE; prep and epilogue
    as in kda_fwd.  Returns o [N, H, dv]."""
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert state.dtype == np.float64 and state.flags.c_contiguous
    num_slots = state.shape[0]
    si = None if slot_idx is None else np.ascontiguousarray(np.asarray(slot_idx, dtype=np.int32))
    o = np.zeros((N, H, dv), dtype=np.float64)
    if prep is not None or epilogue is not None:
        flags, eps, a, b = _prep_args(prep or {}, H, dk)
        on, e_eps, w, z = _epi_args(epilogue, (N, H, dv), dv)
        rc = _load().oracle_kda_decode_step_ex(N, H, dk, dv, float(scale), _ptr(q), _ptr(k),
                                               _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                               num_slots, _ptr(si), flags, eps, _ptr(a),
                                               _ptr(b), on, e_eps, _ptr(w), _ptr(z), _ptr(o))
    else:
        rc = _load().oracle_kda_decode_step(N, H, dk, dv, float(scale), _ptr(q), _ptr(k),
                                            _ptr(v), _ptr(g), _ptr(beta), _ptr(state), num_slots,
                                            _ptr(si), _ptr(o))
    if rc != 0:
        raise ValueError("oracle_kda_decode_step rejected its arguments (code %d)" % rc)
    return o


# ---------------------------------------------------------------------------
# NumPy fp64 forms for one (sequence, head) chain.  Arrays: q, k, g [T, dk];
# v [T, dv]; beta [T]; S0 [dk, dv] or None.
# ---------------------------------------------------------------------------

def _chain(q, k, v, g, beta, S0):
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64)
    dk, dv = q.shape[1], v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    return q, k, v, g, beta, S


def recurrence_np(q, k, v, g, beta, scale, S0=None):
    """Delta-rule form of one KDA step per token (summary page, "De la atencion
    lineal a Gated DeltaNet": online gradient step on the reconstruction loss;
    "Control fino de memoria": per-channel gate applied to the state first)."""
    q, k, v, g, beta, S = _chain(q, k, v, g, beta, S0)
    o = np.zeros((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        S = np.exp(g[t])[:, None] * S
        err = v[t] - S.T @ k[t]
        S = S + beta[t] * np.outer(k[t], err)
        o[t] = scale * (S.T @ q[t])
    return o, S


def bruteforce_np(q, k, v, g, beta, scale, S0=None):
    """The transition written as the literal dk x dk matrix product
    (I - beta k k^T) Diag(alpha) -- a generalised Householder factor times the
    channel-wise diagonal gate (summary page, "Control fino de memoria": DPLR
    transition whose low-rank part is tied to the key)."""
    q, k, v, g, beta, S = _chain(q, k, v, g, beta, S0)
    dk = q.shape[1]
    I = np.eye(dk)
    o = np.zeros((q.shape[0], v.shape[1]))
    for t in range(q.shape[0]):
        A = (I - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t]))
        S = A @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = scale * (S.T @ q[t])
    return o, S


def chunk_terms_np(Q, K, Gl, b):
    """The intra-chunk quantities of the chunkwise form for one chunk of n
    tokens (summary page, "Algoritmo paralelo por chunks": the two decayed
    Gram blocks, the UT transform by forward substitution), with G_r =
    sum_{j<=r} g_j per channel and Gamma = exp(G):
        KG = K*Gamma,  QG = Q*Gamma,  KE = K*exp(G_n - G)          (n x dk)
        A  = strict_lower(diag(beta) (K*Gamma) (K/Gamma)^T)        (n x n)
        M  = lower_incl_diag((Q*Gamma) (K/Gamma)^T)                 (n x n)
        T  = (I + A)^-1,   Gn = exp(G_n)                            (dk)
    Returned as a dict.  The division by Gamma is done in fp64 with the chunk
    start as reference; for cross-checks on gates whose chunk sums stay above
    about -700."""
    G = np.cumsum(Gl, axis=0)
    Gam = np.exp(G)
    Kp, Km, Qp = K * Gam, K * np.exp(-G), Q * Gam
    A = np.tril(b[:, None] * (Kp @ Km.T), -1)
    M = np.tril(Qp @ Km.T, 0)
    Tm = forward_substitution_inverse(np.eye(Q.shape[0]) + A)
    return dict(KG=Kp, QG=Qp, KE=K * np.exp(G[-1] - G), A=A, M=M, T=Tm, Gn=np.exp(G[-1]))


def chunked_np(q, k, v, g, beta, scale, S0=None, chunk=64):
    """Chunkwise form (summary page, "Algoritmo paralelo por chunks"): fixed
    chunks, each starting from the previous chunk's final state; inside a chunk
    the rank-1 updates are packed into a WY pair by the UT transform
    T = (I + A)^-1, obtained by forward substitution, and the output joins the
    inter-chunk (state) and intra-chunk (masked Gram) parts.

    Within a chunk of n tokens starting from state S, with the quantities of
    chunk_terms_np:
        W = T diag(beta) KG,   Ut = T diag(beta) V
        U = Ut - W S
        O = scale (QG S + M U)
        S <- Diag(Gn) S + KE^T U
    """
    q, k, v, g, beta, S = _chain(q, k, v, g, beta, S0)
    T_len = q.shape[0]
    o = np.zeros((T_len, v.shape[1]))
    for c0 in range(0, T_len, chunk):
        c1 = min(c0 + chunk, T_len)
        b, V = beta[c0:c1], v[c0:c1]
        t = chunk_terms_np(q[c0:c1], k[c0:c1], g[c0:c1], b)
        W = t["T"] @ (b[:, None] * t["KG"])
        Ut = t["T"] @ (b[:, None] * V)
        U = Ut - W @ S
        o[c0:c1] = scale * (t["QG"] @ S + t["M"] @ U)
        S = t["Gn"][:, None] * S + t["KE"].T @ U
    return o, S


def forward_substitution_inverse(L):
    """Inverse of a unit lower-triangular matrix, row by row by forward
    substitution (summary page, "Algoritmo paralelo por chunks")."""
    n = L.shape[0]
    X = np.zeros((n, n))
    for r in range(n):
        X[r, r] = 1.0
        for c in range(r):
            X[r, c] = -L[r, c:r] @ X[c:r, c]
    return X


def linear_attention_closed_form(q, k, v, beta, scale, S0=None):
    """Causal linear attention with write strength beta and no forgetting:
    O = scale (tril(Q K^T) diag(beta) V + Q S0), S_T = S0 + K^T diag(beta) V.
    (Summary page, "De la atencion lineal a Gated DeltaNet": key-value
    associations accumulated into a matrix-valued state.)"""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    beta = np.asarray(beta, dtype=np.float64)
    S0 = np.zeros((q.shape[1], v.shape[1])) if S0 is None else np.asarray(S0, np.float64)
    O = scale * (np.tril(q @ k.T) @ (beta[:, None] * v) + q @ S0)
    S = S0 + k.T @ (beta[:, None] * v)
    return O, S


def scalar_gated_deltanet_np(q, k, v, a, beta, scale, S0=None):
    """Gated DeltaNet with one scalar gate a_t per token (summary page, "De la
    atencion lineal a Gated DeltaNet"): S_t = a_t (I - b k k^T) S + b k v^T."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    a = np.asarray(a, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    dk, dv = q.shape[1], v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((q.shape[0], dv))
    for t in range(q.shape[0]):
        kS = k[t] @ S
        S = a[t] * (S - beta[t] * np.outer(k[t], kS)) + beta[t] * np.outer(k[t], v[t])
        o[t] = scale * (q[t] @ S)
    return o, S


def dplr_fwd(q, k, v, a, b, g, scale, S0=None, cu_seqlens=None):
    """Exact forward of the general diagonal-plus-low-rank recurrence in fp64:
    S_t = (Diag(exp(g_t)) - a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = scale S_t^T q_t.
    q, k, a, b, g: [B, T, H, dk]; v: [B, T, H, dv] (float32 values).  S0 and
    cu_seqlens as in kda_fwd.  Returns (o [B, T, H, dv], S [N, H, dk, dv]),
    float64."""
    q, k, v, a, b, g = (_f32(x) for x in (q, k, v, a, b, g))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for x in (k, a, b, g):
        assert x.shape == q.shape
    assert v.shape[:3] == (B, T, H)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        cu = None
        N = B
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
        assert s0.shape == (N, H, dk, dv)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().oracle_dplr_fwd(B, T, H, dk, dv, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(a), _ptr(b), _ptr(g), _ptr(s0), _ptr(cu), N, _ptr(o),
                                 _ptr(S))
    if rc != 0:
        raise ValueError("oracle_dplr_fwd rejected its arguments (code %d)" % rc)
    return o, S
