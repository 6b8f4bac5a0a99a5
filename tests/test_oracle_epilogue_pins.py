"""Pins for the oracle's optional output epilogue (CPU only).

The epilogue is what a Kimi Linear layer applies to the operator's output
before the output projection (summary page, "Configuracion del modelo Kimi
Linear": per-head RMSNorm and a data-dependent output gate), read as
    y = o / sqrt(mean(o^2) + eps) * w * sigmoid(z)     per (token, head) row.

Pins (properties and special values of the definition, checked against the
plain oracle's own output o):
  E1  with w = 1, no gate and eps = 0 every row of y has unit RMS and points
      the same way as the row of o;
  E2  with eps = 0, scaling v and S0 by c > 0 (which scales o by c) leaves y
      unchanged;
  E3  gate logits 0 halve y; logits of -80 zero it; +80 leave it;
  E4  y is linear in w, channel by channel;
  E5  the state is untouched by the epilogue.
Each planted mistake in a copy of the epilogue must fail at least one pin.
"""
import numpy as np
import pytest

import oracle


def _rand(seed, B=1, T=20, H=2, d=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, H, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, d))
    g = -rng.uniform(0.01, 0.2, (B, T, H, d))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    S0 = 0.3 * rng.standard_normal((B, H, d, d))
    return [x.astype(np.float32) for x in (q, k, v, g, beta)] + [S0]


def _oracle(q, k, v, g, beta, S0, epi):
    return oracle.kda_fwd(q, k, v, g, beta, 0.5, S0=S0, epilogue=epi)


def _mutant(kind):
    def fwd(q, k, v, g, beta, S0, epi):
        o, S = oracle.kda_fwd(q, k, v, g, beta, 0.5, S0=S0)
        eps = epi.get("eps", 1e-6)
        if kind == "sum_not_mean":
            ms = (o * o).sum(-1, keepdims=True)
        elif kind == "norm_over_heads":
            ms = (o * o).mean(axis=(-2, -1), keepdims=True)
        else:
            ms = (o * o).mean(-1, keepdims=True)
        y = o / ms if kind == "no_sqrt" else o / np.sqrt(ms + eps)
        w = epi.get("weight")
        if w is not None:
            w = np.asarray(w, np.float64)
            y = y * (w * w if kind == "weight_twice" else w)
        z = epi.get("gate")
        if z is not None:
            z = np.asarray(z, np.float64)
            y = y / (1.0 + np.exp(z)) if kind == "sigmoid_sign" else y / (1.0 + np.exp(-z))
        return y, S
    return fwd


def pin_e1(fwd):
    q, k, v, g, beta, S0 = _rand(1)
    y, _ = fwd(q, k, v, g, beta, S0, dict(eps=0.0))
    o, _ = oracle.kda_fwd(q, k, v, g, beta, 0.5, S0=S0)
    rms = np.sqrt((y * y).mean(-1))
    cos = (y * o).sum(-1) / (np.linalg.norm(y, axis=-1) * np.linalg.norm(o, axis=-1))
    return np.max(np.abs(rms - 1.0)) < 1e-12 and np.min(cos) > 1 - 1e-12


def pin_e2(fwd):
    q, k, v, g, beta, S0 = _rand(2)
    y1, _ = fwd(q, k, v, g, beta, S0, dict(eps=0.0))
    y2, _ = fwd(q, k, v * np.float32(4.0), g, beta, S0 * 4.0, dict(eps=0.0))
    return np.max(np.abs(y1 - y2)) < 1e-9


def pin_e3(fwd):
    q, k, v, g, beta, S0 = _rand(3)
    y0, _ = fwd(q, k, v, g, beta, S0, dict(eps=1e-6))
    z = np.zeros(q.shape[:3] + (v.shape[-1],), np.float32)
    yh, _ = fwd(q, k, v, g, beta, S0, dict(eps=1e-6, gate=z))
    yn, _ = fwd(q, k, v, g, beta, S0, dict(eps=1e-6, gate=z - 80.0))
    yp, _ = fwd(q, k, v, g, beta, S0, dict(eps=1e-6, gate=z + 80.0))
    return (np.max(np.abs(yh - 0.5 * y0)) < 1e-12 and np.max(np.abs(yn)) < 1e-30 and
            np.max(np.abs(yp - y0)) < 1e-12)


def pin_e4(fwd):
    q, k, v, g, beta, S0 = _rand(4)
    w = np.random.default_rng(9).uniform(-2, 2, v.shape[-1]).astype(np.float32)
    y1, _ = fwd(q, k, v, g, beta, S0, dict(eps=1e-6))
    yw, _ = fwd(q, k, v, g, beta, S0, dict(eps=1e-6, weight=w))
    return np.max(np.abs(yw - y1 * w.astype(np.float64))) < 1e-12


def pin_e5(fwd):
    q, k, v, g, beta, S0 = _rand(5)
    _, S1 = fwd(q, k, v, g, beta, S0, dict(eps=1e-6, gate=np.ones(q.shape[:3] + (8,), np.float32)))
    _, S0r = oracle.kda_fwd(q, k, v, g, beta, 0.5, S0=S0)
    return np.array_equal(S1, S0r)


PINS = [pin_e1, pin_e2, pin_e3, pin_e4, pin_e5]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_epilogue_pin(pin):
    assert pin(_oracle)


def test_correct_copy_passes_every_pin():
    for pin in PINS:
        assert pin(_mutant("none")), pin.__name__


@pytest.mark.parametrize("kind", ["sum_not_mean", "norm_over_heads", "no_sqrt", "weight_twice",
                                  "sigmoid_sign"])
def test_epilogue_pins_detect_planted_mistakes(kind):
    assert not all(pin(_mutant(kind)) for pin in PINS)


def test_decode_epilogue_matches_prefill():
    """The decode step's epilogue is the same row operation."""
    q, k, v, g, beta, S0 = _rand(6, T=5)
    z = np.random.default_rng(1).standard_normal(q.shape[:3] + (8,)).astype(np.float32)
    w = np.random.default_rng(2).uniform(0.5, 1.5, 8).astype(np.float32)
    y, _ = oracle.kda_fwd(q, k, v, g, beta, 0.5, S0=S0, epilogue=dict(eps=1e-5, weight=w, gate=z))
    st = np.ascontiguousarray(S0.copy())
    for t in range(q.shape[1]):
        yt = oracle.kda_decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], 0.5, st,
                                    epilogue=dict(eps=1e-5, weight=w, gate=z[:, t]))
        assert np.max(np.abs(yt - y[:, t])) < 1e-12
