"""Pins for the oracle's gradients (CPU only).

The oracle's backward (reverse mode through the token recurrence) is checked
against central finite differences of the loss
    L = sum(o * d_o) + sum(S_final * d_S_final)
evaluated with the fp64 NumPy recurrence (recurrence_np, itself pinned to the
C oracle): for random directions d in every input, (L(x + h d) - L(x - h d)) / 2h
must equal <grad L, d> to ~1e-7 relative.  A copy of the backward with planted
mistakes must fail the same check.
"""
import numpy as np
import pytest

import oracle


def _inputs(seed, T=9, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    g = -rng.uniform(0.05, 0.5, (T, dk))
    beta = rng.uniform(0.2, 0.9, T)
    S0 = rng.standard_normal((dk, dv))
    do = rng.standard_normal((T, dv))
    dS = rng.standard_normal((dk, dv))
    # exactly representable in float32 (the C oracle reads float32 inputs)
    q, k, v, g, beta = (x.astype(np.float32).astype(np.float64) for x in (q, k, v, g, beta))
    return q, k, v, g, beta, S0, do, dS


def _loss(q, k, v, g, beta, S0, do, dS, scale):
    o, S = oracle.recurrence_np(q, k, v, g, beta, scale, S0)
    return float((o * do).sum() + (S * dS).sum())


def _oracle_grads(q, k, v, g, beta, S0, do, dS, scale):
    T, dk = q.shape
    dv = v.shape[1]
    r = lambda x: x.reshape((1, T, 1) + x.shape[1:])
    dq, dk_, dv_, dg, db, dS0 = oracle.kda_bwd(r(q), r(k), r(v), r(g), beta.reshape(1, T, 1),
                                                scale, r(do), S0=S0.reshape(1, 1, dk, dv),
                                                d_S_final=dS.reshape(1, 1, dk, dv))
    return dict(q=dq[0, :, 0], k=dk_[0, :, 0], v=dv_[0, :, 0], g=dg[0, :, 0], beta=db[0, :, 0],
                S0=dS0[0, 0])


def _mutant_grads(kind):
    """The same reverse mode in NumPy with one planted mistake."""
    def grads(q, k, v, g, beta, S0, do, dS, scale):
        T = q.shape[0]
        hist = [S0.copy()]
        S = S0.copy()
        for t in range(T):
            S = np.exp(g[t])[:, None] * S
            S = S + beta[t] * np.outer(k[t], v[t] - S.T @ k[t])
            hist.append(S.copy())
        out = {n: np.zeros_like(x) for n, x in (("q", q), ("k", k), ("v", v), ("g", g),
                                                 ("beta", beta))}
        dSt = dS.copy()
        for t in range(T - 1, -1, -1):
            a = np.exp(g[t])
            S1 = a[:, None] * hist[t]
            u = S1.T @ k[t]
            e = beta[t] * (v[t] - u)
            dSt = dSt + scale * np.outer(q[t], do[t])
            out["q"][t] = scale * hist[t + 1] @ do[t]
            de = dSt.T @ k[t]
            out["k"][t] = dSt @ e
            out["beta"][t] = de @ (v[t] - u) * (-1 if kind == "beta_sign" else 1)
            out["v"][t] = beta[t] * de
            du = -beta[t] * de
            if kind != "drop_recall_term":
                dSt = dSt + np.outer(k[t], du)
            out["k"][t] += S1 @ du
            out["g"][t] = a * ((dSt * hist[t]).sum(1) if kind != "gate_on_new_state"
                               else (dSt * hist[t + 1]).sum(1))
            if kind != "no_decay_in_adjoint":
                dSt = a[:, None] * dSt
        out["S0"] = dSt
        return out
    return grads


def _fd_check(grad_fn, seed, scale=0.7, h=1e-5, tol=1e-6):
    x = _inputs(seed)
    names = ["q", "k", "v", "g", "beta", "S0"]
    grads = grad_fn(*x, scale)
    rng = np.random.default_rng(seed + 100)
    worst = 0.0
    for i, n in enumerate(names):
        for _ in range(3):
            d = rng.standard_normal(x[i].shape)
            xp = list(x)
            xm = list(x)
            xp[i] = x[i] + h * d
            xm[i] = x[i] - h * d
            fd = (_loss(*xp, scale) - _loss(*xm, scale)) / (2 * h)
            an = float((grads[n] * d).sum())
            worst = max(worst, abs(fd - an) / max(1.0, abs(fd)))
    return worst < tol, worst


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_oracle_gradients_match_finite_differences(seed):
    ok, worst = _fd_check(_oracle_grads, seed)
    assert ok, worst


def test_correct_copy_matches_finite_differences():
    ok, worst = _fd_check(_mutant_grads("none"), 4)
    assert ok, worst


@pytest.mark.parametrize("kind", ["beta_sign", "drop_recall_term", "gate_on_new_state",
                                  "no_decay_in_adjoint"])
def test_finite_differences_detect_planted_mistakes(kind):
    ok, worst = _fd_check(_mutant_grads(kind), 5)
    assert not ok, worst


def test_varlen_and_batch_gradients_split_by_sequence():
    """Packed sequences give each sequence's own gradients (the same as one call
    per sequence), and the initial-state gradient per sequence."""
    rng = np.random.default_rng(8)
    lens = [5, 1, 7]
    T, H, dk, dv = sum(lens), 2, 4, 3
    q = rng.standard_normal((1, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((1, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((1, T, H, dv)).astype(np.float32)
    g = (-rng.uniform(0.05, 0.5, (1, T, H, dk))).astype(np.float32)
    b = rng.uniform(0.2, 0.9, (1, T, H)).astype(np.float32)
    S0 = rng.standard_normal((3, H, dk, dv))
    do = rng.standard_normal((1, T, H, dv))
    dSf = rng.standard_normal((3, H, dk, dv))
    cu = np.array([0, 5, 6, 13], np.int32)
    packed = oracle.kda_bwd(q, k, v, g, b, 0.5, do, S0=S0, cu_seqlens=cu, d_S_final=dSf)
    for n in range(3):
        sl = slice(cu[n], cu[n + 1])
        one = oracle.kda_bwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], b[:, sl], 0.5, do[:, sl],
                             S0=S0[n:n + 1], d_S_final=dSf[n:n + 1])
        for a, c in zip(packed[:5], one[:5]):
            assert np.allclose(a[:, sl], c, atol=1e-12)
        assert np.allclose(packed[5][n], one[5][0], atol=1e-12)
