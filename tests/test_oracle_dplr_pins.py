"""Pins for the oracle's general diagonal-plus-low-rank recurrence (CPU only).

    S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = scale S_t^T q_t

(summary page, "Menor cantidad de operaciones que DPLR general": KDA is the
member of this family whose two low-rank vectors are tied to the key; the page
gives no formula, this is the plainest form consistent with KDA's).

Pins, each against something other than the oracle itself:
  P1  KDA reduction, exact: a = beta k, b = k, write key beta k with alpha = 1
      and dyadic beta equals the (separately pinned) KDA oracle to 1e-12;
  P2  KDA reduction, general gates: a = beta k, b = alpha * k (fp32-rounded
      products) equals the KDA oracle within the fp32 rounding of the inputs;
  P3  a = 0: gated linear attention, written as the direct double sum
      o_t = scale sum_{i<=t} (q_t * exp(G_t - G_i))^T k_i v_i^T + decayed S0;
  P4  erasure: alpha = 1, a = b = e_c: row c of the state is k_t[c] v_t after
      every step, the other rows accumulate k v^T;
  P5  reflections: alpha = 1, k = 0, a = 2 u_t, b = u_t (unit u_t): the state
      is the explicit product of Householder matrices applied to S0;
  P6  packed sequences give each sequence's own result.
Planted mistakes in a NumPy copy of the recurrence must each fail a pin.
A further test checks the chunkwise form the GPU kernels evaluate (four
decayed Gram matrices, one triangular solve) against the oracle.
"""
import numpy as np
import pytest

import oracle


def _rand(seed, T=24, d=8, dv=6, H=1, B=1):
    rng = np.random.default_rng(seed)
    sh = (B, T, H, d)
    q = rng.standard_normal(sh)
    k = rng.standard_normal(sh)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    a = 0.5 * rng.standard_normal(sh)
    b = 0.5 * rng.standard_normal(sh)
    g = -rng.uniform(0.01, 0.3, sh)
    S0 = 0.3 * rng.standard_normal((B, H, d, dv))
    return [x.astype(np.float32) for x in (q, k, v, a, b, g)] + [S0]


def _np_fwd(kind):
    """The recurrence in NumPy (one batch row, every head), optionally with
    one planted mistake."""
    def fwd(q, k, v, a, b, g, scale, S0):
        q, k, v, a, b, g = (x.astype(np.float64) for x in (q, k, v, a, b, g))
        B, T, H, d = q.shape
        o = np.zeros(v.shape)
        S = S0.copy()
        for h in range(H):
            St = S[0, h]
            for t in range(T):
                al = np.exp(g[0, t, h])
                u = b[0, t, h] @ St
                if kind == "read_after_decay":
                    u = b[0, t, h] @ (al[:, None] * St)
                sign = 1.0 if kind == "plus_sign" else -1.0
                aa, bb = (b, a) if kind == "swap_ab" else (a, b)
                if kind == "swap_ab":
                    u = bb[0, t, h] @ St
                St_new = al[:, None] * St + sign * np.outer(aa[0, t, h], u)
                if kind != "no_write":
                    St_new = St_new + np.outer(k[0, t, h], v[0, t, h])
                ot = St if kind == "output_before_update" else St_new
                o[0, t, h] = scale * (q[0, t, h] @ ot)
                St = St_new
            S[0, h] = St
        return o, S
    return fwd


def _oracle(q, k, v, a, b, g, scale, S0):
    return oracle.dplr_fwd(q, k, v, a, b, g, scale, S0=S0)


def pin_p1(fwd):
    q, k, v, a, b, g, S0 = _rand(1)
    rng = np.random.default_rng(11)
    beta = rng.choice([0.25, 0.5, 1.0], size=q.shape[:3]).astype(np.float32)
    g = np.zeros_like(g)
    bk = (beta[..., None] * k).astype(np.float32)        # exact: dyadic beta
    o1, S1 = fwd(q, bk, v, bk, k, g, 0.5, S0)
    o2, S2 = oracle.kda_fwd(q, k, v, g, beta, 0.5, S0=S0)
    return np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(S1 - S2)) < 1e-12


def pin_p2(fwd):
    q, k, v, a, b, g, S0 = _rand(2)
    beta = np.random.default_rng(12).uniform(0.1, 0.9, q.shape[:3]).astype(np.float32)
    bk = (beta[..., None].astype(np.float64) * k).astype(np.float32)
    ak = (np.exp(g.astype(np.float64)) * k).astype(np.float32)
    o1, S1 = fwd(q, bk, v, bk, ak, g, 0.5, S0)
    o2, S2 = oracle.kda_fwd(q, k, v, g, beta, 0.5, S0=S0)
    rms = np.sqrt(np.mean(o2 ** 2))
    return np.max(np.abs(o1 - o2)) < 1e-5 * rms and np.max(np.abs(S1 - S2)) < 1e-5


def gla_closed_form(q, k, v, g, scale, S0):
    q, k, v, g = (x.astype(np.float64)[0, :, 0] for x in (q, k, v, g))
    T = q.shape[0]
    G = np.cumsum(g, axis=0)
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        o[t] = scale * ((q[t] * np.exp(G[t])) @ S0[0, 0])
        for i in range(t + 1):
            o[t] += scale * np.dot(q[t] * np.exp(G[t] - G[i]), k[i]) * v[i]
    S = np.exp(G[-1])[:, None] * S0[0, 0]
    for i in range(T):
        S += np.outer(k[i] * np.exp(G[-1] - G[i]), v[i])
    return o, S


def pin_p3(fwd):
    q, k, v, a, b, g, S0 = _rand(3)
    o1, S1 = fwd(q, k, v, np.zeros_like(a), b, g, 0.7, S0)
    o2, S2 = gla_closed_form(q, k, v, g, 0.7, S0)
    return np.max(np.abs(o1[0, :, 0] - o2)) < 1e-12 and np.max(np.abs(S1[0, 0] - S2)) < 1e-12


def pin_p4(fwd):
    q, k, v, a, b, g, S0 = _rand(4)
    c = 3
    e = np.zeros_like(a)
    e[..., c] = 1.0
    o1, S1 = fwd(q, k, v, e, e, np.zeros_like(g), 0.5, S0)
    kk, vv = k[0, :, 0].astype(np.float64), v[0, :, 0].astype(np.float64)
    ref = S0[0, 0] + kk.T @ vv
    ref[c] = kk[-1, c] * vv[-1]
    return np.max(np.abs(S1[0, 0] - ref)) < 1e-12


def pin_p5(fwd):
    q, k, v, a, b, g, S0 = _rand(5)
    rng = np.random.default_rng(15)
    u = rng.standard_normal(a.shape)
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    u = u.astype(np.float32)
    u64 = u.astype(np.float64)
    a2 = (2.0 * u64).astype(np.float32)                  # exact
    o1, S1 = fwd(q, np.zeros_like(k), v, a2, u, np.zeros_like(g), 0.5, S0)
    S = S0[0, 0].copy()
    ok = True
    for t in range(q.shape[1]):
        Hm = np.eye(S.shape[0]) - 2.0 * np.outer(u64[0, t, 0], u64[0, t, 0])
        S = Hm @ S
        ok &= np.max(np.abs(o1[0, t, 0] - 0.5 * q[0, t, 0].astype(np.float64) @ S)) < 1e-12
    return ok and np.max(np.abs(S1[0, 0] - S)) < 1e-12


PINS = [pin_p1, pin_p2, pin_p3, pin_p4, pin_p5]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_dplr_pin(pin):
    assert pin(_oracle)


def test_numpy_copy_passes_every_pin():
    for pin in PINS:
        assert pin(_np_fwd("none")), pin.__name__


@pytest.mark.parametrize("kind", ["read_after_decay", "plus_sign", "no_write",
                                  "output_before_update", "swap_ab"])
def test_dplr_pins_detect_planted_mistakes(kind):
    assert not all(pin(_np_fwd(kind)) for pin in PINS)


def test_dplr_varlen_splits_by_sequence():
    rng = np.random.default_rng(16)
    lens = [5, 0, 9, 1]
    T, H, d = sum(lens), 2, 8
    x = [rng.standard_normal((1, T, H, d)).astype(np.float32) for _ in range(5)]
    g = (-rng.uniform(0.01, 0.3, (1, T, H, d))).astype(np.float32)
    S0 = rng.standard_normal((len(lens), H, d, d))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, S = oracle.dplr_fwd(x[0], x[1], x[2], x[3], x[4], g, 0.5, S0=S0, cu_seqlens=cu)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        o1, S1 = oracle.dplr_fwd(*(t[:, sl] for t in x), g[:, sl], 0.5, S0=S0[n:n + 1])
        assert np.allclose(o[:, sl], o1, atol=1e-12) and np.allclose(S[n], S1[0], atol=1e-12)


def dplr_chunked_np(q, k, v, a, b, g, scale, S0, C):
    """The chunkwise form the GPU kernels evaluate, for one (sequence, head):
    with G the chunk-local inclusive cumulative log gate, Gx = G - g (exclusive),
        Pba[i, j] = sum_c b_ic e^{Gx_ic - G_jc} a_jc   (j < i)
        Pbk[i, j] = sum_c b_ic e^{Gx_ic - G_jc} k_jc   (j < i)
        Pqa[r, i] = sum_c q_rc e^{G_rc - G_ic} a_ic     (i <= r)
        Pqk[r, i] = sum_c q_rc e^{G_rc - G_ic} k_ic     (i <= r)
        U = T (Bd S + Pbk V), T = (I + Pba)^-1, Bd = b * e^{Gx}   (U_i = b_i^T S_{i-1})
        O = scale (QG S + Pqk V - Pqa U),  QG = q * e^{G}
        S <- e^{G_n} * S + KE^T V - AE^T U,  KE = k * e^{G_n - G}, AE = a * e^{G_n - G}."""
    q, k, v, a, b, g = (x.astype(np.float64) for x in (q, k, v, a, b, g))
    T = q.shape[0]
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        Q, K, V, A, Bv, gg = q[sl], k[sl], v[sl], a[sl], b[sl], g[sl]
        L = Q.shape[0]
        G = np.cumsum(gg, axis=0)
        Gx = G - gg
        Gn = G[-1]
        Bd = Bv * np.exp(Gx)
        AI, KI = A * np.exp(-G), K * np.exp(-G)
        QG = Q * np.exp(G)
        strict = np.tril(np.ones((L, L)), -1)
        incl = np.tril(np.ones((L, L)))
        Pba, Pbk = (Bd @ AI.T) * strict, (Bd @ KI.T) * strict
        Pqa, Pqk = (QG @ AI.T) * incl, (QG @ KI.T) * incl
        Tm = np.linalg.inv(np.eye(L) + Pba)
        U = Tm @ (Bd @ S + Pbk @ V)
        o[sl] = scale * (QG @ S + Pqk @ V - Pqa @ U)
        E = np.exp(Gn - G)
        S = np.exp(Gn)[:, None] * S + (K * E).T @ V - (A * E).T @ U
    return o, S


@pytest.mark.parametrize("C", [1, 4, 16])
def test_dplr_chunk_form_matches_oracle(C):
    q, k, v, a, b, g, S0 = _rand(7, T=37)
    o, S = oracle.dplr_fwd(q, k, v, a, b, g, 0.5, S0=S0)
    oc, Sc = dplr_chunked_np(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0], b[0, :, 0],
                             g[0, :, 0], 0.5, S0[0, 0], C)
    assert np.max(np.abs(oc - o[0, :, 0])) < 1e-10 and np.max(np.abs(Sc - S[0, 0])) < 1e-10
