"""Shared helpers for the GPU parity tests: seeded inputs (from kda_inputs),
exact float32 host copies for the oracle, and the error metric.

Error metric: max |gpu - ref| / RMS(ref), over every compared element; the
bound is 1e-4 for float32 inputs and 2e-2 for bfloat16 inputs, for outputs
and final states alike.
"""
import numpy as np
import torch

import kda_inputs
import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def np32(t):
    """Exact float32 host copy (bf16 upcasts exactly)."""
    return t.detach().float().cpu().numpy()


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    return float(np.max(np.abs(x - ref))) / rms


def oracle_prefill(d, scale, heads=None, cu=None):
    """Run the fp64 oracle on (a subset of) heads of a prefill input dict."""
    sel = (lambda t: t) if heads is None else (lambda t: t[:, :, heads])
    q, k, v, g = (np32(sel(d[n])) for n in ("q", "k", "v", "g"))
    beta = np32(d["beta"] if heads is None else d["beta"][:, :, heads])
    S0 = None
    if d.get("S0") is not None:
        S0 = d["S0"].detach().double().cpu().numpy()
        if heads is not None:
            S0 = S0[:, heads]
    cu_np = None if cu is None else cu.cpu().numpy()
    return oracle.kda_fwd(q, k, v, g, beta, scale, S0=S0, cu_seqlens=cu_np)


def make_prefill(seed, B, T, H, D, dtype, s0_std=None, device="cuda", g_range=(0.001, 0.1),
                 n_states=None):
    return kda_inputs.prefill_inputs(seed, B, T, H, D, D, dtype, device, s0_std=s0_std,
                                     g_range=g_range, n_states=n_states)
