"""Pins for the oracle's optional input preparation (CPU only).

The preparation is what a model layer applies before the operator (summary
page, "Configuracion del modelo Kimi Linear"): L2 normalisation of queries and
keys, beta from logits, and the per-channel decay gate computed from a
pre-activation with a Mamba/GDN-style decay function, read here as
    log alpha = -exp(A_log[h]) * softplus(g + dt_bias[h, c]).

Every pin is a property or a special value, not the formula typed again:
  N1  with normalisation, rescaling q or k per token by positive factors
      changes nothing (and without it, it does);
  N2  normalised orthonormal keys of arbitrary length, beta -> 1 and no decay
      store values that are read back exactly (the delta rule's exactness);
  B1  a zero logit means beta = 1/2 (one token from a zero state:
      o = scale * beta * (q.k) * v);
  B2  a very negative logit means no write at all;
  G1  A_log = 0 with a zero pre-activation and zero bias gives alpha = 1/2;
  G2  a huge negative A_log, or a huge negative bias, means no decay;
  G3  a large pre-activation passes through softplus unchanged (log alpha = -x).
Each planted mistake in a copy of the preparation must fail at least one pin.
"""
import numpy as np
import pytest

import oracle


def _rand(rng, B, T, H, dk, dv):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = -rng.uniform(0.01, 0.2, (B, T, H, dk))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    return [x.astype(np.float32) for x in (q, k, v, g, beta)]


def _unit_rows(n, d, rng):
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return Q[:n]


# ---- a copy of the preparation with planted mistakes, run through the plain
# oracle (prep done in fp64 here, the recurrence in the oracle) ----
def _mutant_fwd(kind):
    def fwd(q, k, v, g, beta, scale, prep, S0=None):
        q, k, g, beta = (np.asarray(x, np.float64) for x in (q, k, g, beta))
        H, dk = q.shape[2], q.shape[3]
        if prep.get("normalize_qk"):
            eps = prep.get("eps", 1e-6)
            if kind == "no_sqrt":
                nq = 1.0 / ((q * q).sum(-1, keepdims=True) + eps)
                nk = 1.0 / ((k * k).sum(-1, keepdims=True) + eps)
            else:
                nq = 1.0 / np.sqrt((q * q).sum(-1, keepdims=True) + eps)
                nk = 1.0 / np.sqrt((k * k).sum(-1, keepdims=True) + eps)
            q = q * nq
            if kind != "k_not_normalised":
                k = k * nk
        if prep.get("beta_logit"):
            beta = 1.0 / (1.0 + np.exp(beta)) if kind == "sigmoid_sign" else 1.0 / (1.0 + np.exp(-beta))
        if prep.get("A_log") is not None:
            a = np.asarray(prep["A_log"], np.float64).reshape(1, 1, H, 1)
            b = prep.get("dt_bias")
            b = 0.0 if b is None else np.asarray(b, np.float64).reshape(1, 1, H, dk)
            if kind == "exp_for_softplus":
                g = -np.exp(a) * np.exp(g + b)
            elif kind == "rate_without_exp":
                g = -a * np.log1p(np.exp(g + b))
            elif kind == "bias_after_softplus":
                g = -np.exp(a) * (np.log1p(np.exp(g)) + b)
            else:
                g = -np.exp(a) * np.logaddexp(0.0, g + b)
        # the oracle takes float32 arrays; keep the prepared values as exact as
        # float32 allows (the pins' tolerances cover that rounding)
        return oracle.kda_fwd(q, k, v, g, beta, scale, S0=S0)
    return fwd


def _oracle_fwd(q, k, v, g, beta, scale, prep, S0=None):
    return oracle.kda_fwd(q, k, v, g, beta, scale, S0=S0, prep=prep)


# ---- pins: each returns True when the property holds ----
def pin_n1(fwd):
    rng = np.random.default_rng(1)
    q, k, v, g, beta = _rand(rng, 1, 24, 2, 8, 5)
    prep = dict(normalize_qk=True, eps=0.0)
    o1, S1 = fwd(q, k, v, g, beta, 0.4, prep)
    cq = rng.uniform(0.2, 5.0, (1, 24, 2, 1)).astype(np.float32)
    ck = rng.uniform(0.2, 5.0, (1, 24, 2, 1)).astype(np.float32)
    o2, S2 = fwd(q * cq, k * ck, v, g, beta, 0.4, prep)
    same = np.max(np.abs(o1 - o2)) < 1e-5 and np.max(np.abs(S1 - S2)) < 1e-5
    o3, _ = oracle.kda_fwd(q * cq, k * ck, v, g, beta, 0.4)
    return same and np.max(np.abs(o3 - o1)) > 1e-2


def pin_n2(fwd):
    rng = np.random.default_rng(2)
    n, dk, dv = 5, 8, 3
    keys = _unit_rows(n, dk, rng) * rng.uniform(0.3, 4.0, (n, 1))
    vals = rng.standard_normal((n, dv))
    q = rng.standard_normal((1, n, 1, dk)).astype(np.float32)
    k = keys.reshape(1, n, 1, dk).astype(np.float32)
    v = vals.reshape(1, n, 1, dv).astype(np.float32)
    g = np.zeros((1, n, 1, dk), np.float32)
    b = np.full((1, n, 1), 40.0, np.float32)        # sigmoid(40) = 1 - 4e-18
    _, S = fwd(q, k, v, g, b, 1.0, dict(normalize_qk=True, eps=0.0, beta_logit=True))
    kh = k[0, :, 0].astype(np.float64)
    kh = kh / np.linalg.norm(kh, axis=1, keepdims=True)
    return np.max(np.abs(kh @ S[0, 0] - vals)) < 1e-5


def pin_b1(fwd):
    rng = np.random.default_rng(3)
    q, k, v, g, _ = _rand(rng, 1, 1, 1, 6, 4)
    b = np.zeros((1, 1, 1), np.float32)
    o, _ = fwd(q, k, v, g, b, 0.7, dict(beta_logit=True))
    want = 0.7 * 0.5 * float(q[0, 0, 0].astype(np.float64) @ k[0, 0, 0]) * v[0, 0, 0].astype(np.float64)
    return np.max(np.abs(o[0, 0, 0] - want)) < 1e-12


def pin_b2(fwd):
    rng = np.random.default_rng(4)
    q, k, v, _, _ = _rand(rng, 1, 10, 2, 6, 4)
    g = np.zeros_like(q)
    b = np.full((1, 10, 2), -80.0, np.float32)       # sigmoid(-80) = 1.8e-35
    S0 = rng.standard_normal((1, 2, 6, 4))
    _, S = fwd(q, k, v, g, b, 1.0, dict(beta_logit=True), S0=S0)
    return np.max(np.abs(S - S0)) < 1e-12


def pin_g1(fwd):
    rng = np.random.default_rng(5)
    q, k, v, _, beta = _rand(rng, 1, 12, 2, 6, 4)
    zero = np.zeros_like(q)
    prep = dict(A_log=np.zeros(2, np.float32), dt_bias=np.zeros((2, 6), np.float32))
    o1, S1 = fwd(q, k, v, zero, beta, 0.5, prep)
    half = np.full_like(q, np.log(0.5))               # alpha = 1/2 given directly
    o2, S2 = oracle.kda_fwd(q, k, v, half, beta, 0.5)
    return np.max(np.abs(o1 - o2)) < 1e-6 and np.max(np.abs(S1 - S2)) < 1e-6


def pin_g2(fwd):
    rng = np.random.default_rng(6)
    q, k, v, graw, beta = _rand(rng, 1, 12, 2, 6, 4)
    graw = rng.standard_normal(graw.shape).astype(np.float32)
    zero = np.zeros_like(q)
    o0, S0 = oracle.kda_fwd(q, k, v, zero, beta, 0.5)
    a = dict(A_log=np.full(2, -60.0, np.float32), dt_bias=np.zeros((2, 6), np.float32))
    b = dict(A_log=np.zeros(2, np.float32), dt_bias=np.full((2, 6), -90.0, np.float32))
    ok = True
    for prep in (a, b):
        o1, S1 = fwd(q, k, v, graw, beta, 0.5, prep)
        ok = ok and np.max(np.abs(o1 - o0)) < 1e-9 and np.max(np.abs(S1 - S0)) < 1e-9
    return ok


def pin_g3(fwd):
    rng = np.random.default_rng(7)
    q, k, v, _, beta = _rand(rng, 1, 12, 2, 6, 4)
    x = rng.uniform(25.0, 35.0, q.shape).astype(np.float32)
    prep = dict(A_log=np.zeros(2, np.float32))
    o1, S1 = fwd(q, k, v, x, beta, 0.5, prep)
    o2, S2 = oracle.kda_fwd(q, k, v, -x, beta, 0.5)   # softplus(x) = x + log1p(e^-x)
    return np.max(np.abs(o1 - o2)) < 1e-9 and np.max(np.abs(S1 - S2)) < 1e-9


PINS = [pin_n1, pin_n2, pin_b1, pin_b2, pin_g1, pin_g2, pin_g3]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_prep_pin(pin):
    assert pin(_oracle_fwd)


def test_correct_copy_passes_every_pin():
    """The unmutated copy agrees with the oracle's own preparation."""
    for pin in PINS:
        assert pin(_mutant_fwd("none")), pin.__name__


@pytest.mark.parametrize("kind", ["no_sqrt", "k_not_normalised", "sigmoid_sign",
                                  "exp_for_softplus", "rate_without_exp",
                                  "bias_after_softplus"])
def test_prep_pins_detect_planted_mistakes(kind):
    fwd = _mutant_fwd(kind)
    assert not all(pin(fwd) for pin in PINS)
