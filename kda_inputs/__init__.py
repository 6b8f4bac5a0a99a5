"""Seeded synthetic inputs for the KDA operator.

This module is shared by the HIP path's tests/benchmark and by the oracle's
tests.  It draws random tensors and nothing else: it holds none of the
operator's arithmetic.

Recipe (the Kimi-Linear-shaped workloads; head dimension 128 is the one the
GeekNews summary of Kimi Linear gives in "Configuracion del modelo Kimi
Linear", where q and k are also L2-normalised):

* draw order per call: q, k, v, beta-logit, g, S0;
* q, k ~ N(0, 1), then L2-normalised over the key dimension in float32,
  then cast to the input dtype (so bf16 keys are only nearly unit-norm);
* v ~ N(0, 1), cast to the input dtype;
* beta = sigmoid(N(0, 1)), float32 (passed to the operator as is);
* g = log(alpha) = -U(0.001, 0.1), float32 (passed as is);
* S0 ~ N(0, std) float32 when an initial state is asked for, else none.

All draws come from a ``torch.Generator`` seeded with ``seed`` on the device
the tensors are made on, so a given (seed, device) always yields the same
bytes.  The tests hand the oracle an exact float32 copy of whatever the GPU
receives; the two never need to regenerate each other's data.
"""
from __future__ import annotations

import torch

CFG_SEED = {0: 1000, 1: 1001, 2: 1002, 3: 1003, 4: 1004}

# name -> shape description (mirrors the five benchmark/parity configurations)
CONFIGS = {
    0: dict(name="B1 H1 T128 d32 C16 fp32", B=1, H=1, T=128, dk=32, dv=32, chunk=16,
            dtype=torch.float32, s0_std=None),
    1: dict(name="B2 H4 T2048 d64 C64 bf16 S0~N(0,0.02)", B=2, H=4, T=2048, dk=64, dv=64,
            chunk=64, dtype=torch.bfloat16, s0_std=0.02),
    2: dict(name="B1 H32 T32768 d128 C64 bf16", B=1, H=32, T=32768, dk=128, dv=128,
            chunk=64, dtype=torch.bfloat16, s0_std=None),
    3: dict(name="varlen 16 x U[256,8192] H32 d128 C64 bf16", N=16, H=32, dk=128, dv=128,
            chunk=64, dtype=torch.bfloat16, s0_std=None, len_lo=256, len_hi=8192),
    4: dict(name="decode N256 H32 d128, 4096-token prefill init, 512 steps", N=256, H=32,
            dk=128, dv=128, chunk=64, dtype=torch.bfloat16, init_T=4096, steps=512),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


def prefill_inputs(seed, B, T, H, dk, dv, dtype=torch.bfloat16, device="cpu",
                   s0_std=None, n_states=None, g_range=(0.001, 0.1), normalize=True):
    """Token tensors [B, T, H, d] (q, k, v in ``dtype``), beta [B, T, H] and
    g [B, T, H, dk] in float32, optional S0 [n_states or B, H, dk, dv] float32."""
    gen = _gen(seed, device)
    f = dict(device=device, dtype=torch.float32, generator=gen)
    q = torch.randn(B, T, H, dk, **f)
    k = torch.randn(B, T, H, dk, **f)
    v = torch.randn(B, T, H, dv, **f)
    bl = torch.randn(B, T, H, **f)
    u = torch.rand(B, T, H, dk, **f)
    if normalize:
        q, k = _unit(q), _unit(k)
    lo, hi = g_range
    g = -(lo + (hi - lo) * u)
    out = dict(q=q.to(dtype).contiguous(), k=k.to(dtype).contiguous(), v=v.to(dtype).contiguous(),
               beta=torch.sigmoid(bl).contiguous(), g=g.contiguous(), S0=None)
    if s0_std is not None:
        ns = B if n_states is None else n_states
        out["S0"] = (s0_std * torch.randn(ns, H, dk, dv, **f)).contiguous()
    return out


def raw_layer_inputs(seed, B, T, H, dk, dv, dtype=torch.bfloat16, device="cpu"):
    """Inputs as a model layer hands them over before its preparation step:
    q, k un-normalised (each row N(0, 1) times a length in [0.3, 3.3]), beta
    as a N(0, 1) logit, g as a 0.5 N(0, 1) gate pre-activation, plus per-head
    A_log ~ U(-1, 0.5) and per-channel dt_bias ~ U(-5, -2) (so the prepared
    log-gate stays in [-0.5, 0) like the configs' gates)."""
    gen = _gen(seed, device)
    f = dict(device=device, dtype=torch.float32, generator=gen)
    q = torch.randn(B, T, H, dk, **f) * (0.3 + 3 * torch.rand(B, T, H, 1, **f))
    k = torch.randn(B, T, H, dk, **f) * (0.3 + 3 * torch.rand(B, T, H, 1, **f))
    v = torch.randn(B, T, H, dv, **f)
    b = torch.randn(B, T, H, **f)
    g = 0.5 * torch.randn(B, T, H, dk, **f)
    A_log = -1.0 + 1.5 * torch.rand(H, **f)
    dt_bias = -5.0 + 3.0 * torch.rand(H, dk, **f)
    return dict(q=q.to(dtype).contiguous(), k=k.to(dtype).contiguous(),
                v=v.to(dtype).contiguous(), beta=b.contiguous(), g=g.contiguous(),
                A_log=A_log.contiguous(), dt_bias=dt_bias.contiguous())


def varlen_lengths(seed, n, lo, hi):
    """n integer lengths, uniform on [lo, hi] inclusive (CPU generator, so the
    same on every machine)."""
    gen = _gen(seed, "cpu")
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen)]


def cu_seqlens_of(lengths):
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32)


def decode_inputs(seed, step, N, H, dk, dv, dtype=torch.bfloat16, device="cpu"):
    """One decode step's q, k, v [N, H, d], g [N, H, dk], beta [N, H] with the
    prefill recipe; each step has its own seed."""
    d = prefill_inputs(seed * 100003 + 7919 * (step + 1), 1, N, H, dk, dv, dtype, device)
    return dict(q=d["q"][0], k=d["k"][0], v=d["v"][0], g=d["g"][0], beta=d["beta"][0])


def config_inputs(cfg: int, device="cpu"):
    """Full inputs of configuration ``cfg`` in {0, 1, 2, 3} (prefill).  For 3
    the tokens are packed along T with B = 1 and ``cu_seqlens`` is returned."""
    c = CONFIGS[cfg]
    seed = CFG_SEED[cfg]
    if cfg == 3:
        lens = varlen_lengths(seed, c["N"], c["len_lo"], c["len_hi"])
        T = sum(lens)
        d = prefill_inputs(seed, 1, T, c["H"], c["dk"], c["dv"], c["dtype"], device)
        d["cu_seqlens"] = cu_seqlens_of(lens).to(device)
        d["lengths"] = lens
        return d
    d = prefill_inputs(seed, c["B"], c["T"], c["H"], c["dk"], c["dv"], c["dtype"], device,
                       s0_std=c["s0_std"])
    d["cu_seqlens"] = None
    return d


def dplr_inputs(seed, B, T, H, dk, dv, dtype=torch.bfloat16, device="cpu", s0_std=None,
                n_states=None, g_range=(0.001, 0.1)):
    """Inputs of the general diagonal-plus-low-rank recurrence: q, k unit rows,
    v ~ N(0, 1), g as in prefill_inputs, and untied low-rank vectors drawn as
    independent perturbations of the key direction,
        a = beta * unit(k + 0.5 n1),   b = unit(k + 0.5 n2),   beta ~ sigmoid(N(0, 1)),
    so the transitions stay near the contractive KDA ones over long sequences.
    q, k, v, a, b in ``dtype``; g [B, T, H, dk] and S0 float32."""
    gen = _gen(seed, device)
    f = dict(device=device, dtype=torch.float32, generator=gen)
    q = _unit(torch.randn(B, T, H, dk, **f))
    k = _unit(torch.randn(B, T, H, dk, **f))
    v = torch.randn(B, T, H, dv, **f)
    a = _unit(k + 0.5 * torch.randn(B, T, H, dk, **f))
    b = _unit(k + 0.5 * torch.randn(B, T, H, dk, **f))
    beta = torch.sigmoid(torch.randn(B, T, H, 1, **f))
    lo, hi = g_range
    g = -(lo + (hi - lo) * torch.rand(B, T, H, dk, **f))
    out = dict(q=q, k=k, v=v, a=beta * a, b=b)
    out = {n: t.to(dtype).contiguous() for n, t in out.items()}
    out["g"] = g.contiguous()
    out["S0"] = None
    if s0_std is not None:
        out["S0"] = (s0_std * torch.randn(n_states or B, H, dk, dv, **f)).contiguous()
    return out
