"""GPU parity of the in-kernel input preparation (kda_chunk_fwd_prep,
kda_decode_step_prep) against the fp64 oracle with the same preparation.

Raw inputs, as a model layer would hand them over: q and k un-normalised (rows
of random length), beta as logits, g as the gate pre-activation with per-head
A_log and per-channel dt_bias.  The default gate parameters keep log alpha
within [-0.5, 0); the wide ones (A_log up to 1.5, dt_bias up to 3) give
per-token log gates down to about -20, where the chunk form's strong-decay
path takes over.
"""
import numpy as np
import pytest
import torch

import linear_attention_sequence_chunkwise_amd as kda
import oracle
from kda_testlib import TOL, np32, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def raw_inputs(seed, B, T, H, D, dtype, s0=True, n_states=None, wide_gate=False):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    f = dict(device="cuda", dtype=torch.float32, generator=gen)
    q = torch.randn(B, T, H, D, **f) * (0.3 + 3 * torch.rand(B, T, H, 1, **f))
    k = torch.randn(B, T, H, D, **f) * (0.3 + 3 * torch.rand(B, T, H, 1, **f))
    v = torch.randn(B, T, H, D, **f)
    b = torch.randn(B, T, H, **f)
    g = 0.5 * torch.randn(B, T, H, D, **f)
    A_log = -1.0 + 1.5 * torch.rand(H, **f)
    dt_bias = -5.0 + 3.0 * torch.rand(H, D, **f)
    if wide_gate:
        A_log = 1.5 * torch.rand(H, **f)
        dt_bias = -1.0 + 4.0 * torch.rand(H, D, **f)
    S0 = None
    if s0:
        S0 = 0.1 * torch.randn(n_states or B, H, D, D, **f)
    return dict(q=q.to(dtype).contiguous(), k=k.to(dtype).contiguous(),
                v=v.to(dtype).contiguous(), beta=b.contiguous(), g=g.contiguous(),
                A_log=A_log, dt_bias=dt_bias, S0=S0)


def prep_of(d, normalize=True, beta_logit=True, gate=True, bias=True, eps=1e-6):
    return dict(normalize_qk=normalize, eps=eps, beta_logit=beta_logit,
                A_log=d["A_log"] if gate else None,
                dt_bias=d["dt_bias"] if gate and bias else None)


def oracle_prep(p):
    return {kk: (np32(vv) if torch.is_tensor(vv) else vv) for kk, vv in p.items()}


def run_prefill(d, chunk, prep, cu=None):
    o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=chunk,
                             initial_state=d["S0"], cu_seqlens=cu, prep=prep)
    torch.cuda.synchronize()
    D = d["q"].shape[-1]
    ro, rS = oracle.kda_fwd(np32(d["q"]), np32(d["k"]), np32(d["v"]), np32(d["g"]),
                            np32(d["beta"]), D ** -0.5,
                            S0=None if d["S0"] is None else d["S0"].double().cpu().numpy(),
                            cu_seqlens=None if cu is None else cu.cpu().numpy(),
                            prep=oracle_prep(prep))
    return rel_err(o.cpu().numpy(), ro), rel_err(S.cpu().numpy(), rS)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 64])
def test_prefill_prep_all_steps(dtype, D, chunk):
    d = raw_inputs(100 + D + chunk, 2, 150, 2, D, dtype)
    eo, es = run_prefill(d, chunk, prep_of(d))
    assert eo < TOL[dtype] and es < TOL[dtype], (eo, es)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_prep_wide_gate(dtype):
    """The Mamba/GDN gate with un-narrowed A_log and dt_bias, d = 128, chunk
    64: prepared log gates reach about -20 per token."""
    d = raw_inputs(150, 2, 300, 4, 128, dtype, wide_gate=True)
    eo, es = run_prefill(d, 64, prep_of(d))
    assert eo < TOL[dtype] and es < TOL[dtype], (eo, es)


@pytest.mark.parametrize("which", ["normalize", "beta_logit", "gate", "gate_no_bias"])
def test_prefill_prep_single_step(which):
    d = raw_inputs(7, 1, 200, 3, 64, torch.float32)
    p = prep_of(d, normalize=which == "normalize", beta_logit=which == "beta_logit",
                gate=which.startswith("gate"), bias=which == "gate")
    if which != "gate" and which != "gate_no_bias":
        # keep an already-activated gate when the gate step is off
        d["g"] = -0.05 * torch.rand_like(d["g"])
    if which == "gate_no_bias":
        d["g"] = d["g"] - 4.0          # softplus(x) ~ e^-4 without the bias
    if which != "beta_logit":
        d["beta"] = torch.sigmoid(d["beta"])
    if which != "normalize":
        d["q"] = torch.nn.functional.normalize(d["q"], dim=-1)
        d["k"] = torch.nn.functional.normalize(d["k"], dim=-1)
    eo, es = run_prefill(d, 64, p)
    assert eo < 1e-4 and es < 1e-4, (eo, es)


def test_prefill_prep_varlen_bf16():
    lens = [1, 63, 64, 65, 130, 7]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    d = raw_inputs(11, 1, int(sum(lens)), 4, 128, torch.bfloat16, n_states=len(lens))
    eo, es = run_prefill(d, 64, prep_of(d), cu=cu)
    assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16], (eo, es)


def test_prefill_prep_matches_host_prepared_inputs():
    """Preparation inside the kernels == the plain entry point on inputs the
    oracle prepared (fp32 path, tight bound)."""
    d = raw_inputs(12, 2, 96, 2, 64, torch.float32)
    p = prep_of(d)
    o1, S1 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64,
                               initial_state=d["S0"], prep=p)
    qn = torch.nn.functional.normalize(d["q"].double(), dim=-1, eps=0).float()
    kn = torch.nn.functional.normalize(d["k"].double(), dim=-1, eps=0).float()
    rate = torch.exp(d["A_log"].double()).view(1, 1, -1, 1)
    lg = (-rate * torch.nn.functional.softplus(d["g"].double() + d["dt_bias"].double())).float()
    bt = torch.sigmoid(d["beta"].double()).float()
    o2, S2 = kda.kda_chunk_fwd(qn.contiguous(), kn.contiguous(), d["v"], lg.contiguous(),
                               bt.contiguous(), chunk=64, initial_state=d["S0"])
    torch.cuda.synchronize()
    assert rel_err(o1.cpu().numpy(), o2.double().cpu().numpy()) < 1e-4
    assert rel_err(S1.cpu().numpy(), S2.double().cpu().numpy()) < 1e-4


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_decode_prep(dtype, D):
    N, H, slots = 6, 3, 8
    d = raw_inputs(200 + D, 1, N, H, D, dtype, s0=False)
    x = {kk: (vv[0].contiguous() if torch.is_tensor(vv) and vv.dim() >= 3 else vv)
         for kk, vv in d.items()}
    gen = torch.Generator(device="cuda").manual_seed(3)
    state = 0.2 * torch.randn(slots, H, D, D, device="cuda", generator=gen)
    idx = torch.tensor([5, 0, 7, 2, 30, 3], dtype=torch.int32, device="cuda")  # 30: no-op
    ref_state = state.double().cpu().numpy().copy()
    p = prep_of(d)
    o = torch.full((N, H, D), 7.0, device="cuda")
    kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, slot_idx=idx, o=o,
                        prep=p)
    torch.cuda.synchronize()
    ro = oracle.kda_decode_step(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["g"]),
                                np32(x["beta"]), D ** -0.5, ref_state,
                                slot_idx=idx.cpu().numpy(), prep=oracle_prep(p))
    valid = [0, 1, 2, 3, 5]
    assert rel_err(o.cpu().numpy()[valid], ro[valid]) < 1e-5
    assert np.all(o.cpu().numpy()[4] == 7.0)
    assert rel_err(state.cpu().numpy(), ref_state) < 1e-5


def test_decode_prep_equals_prefill_prep():
    """T decode steps with preparation == one prefill with preparation."""
    B, T, H, D = 2, 40, 2, 64
    d = raw_inputs(21, B, T, H, D, torch.float32)
    p = prep_of(d)
    o_p, S_p = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=16,
                                 initial_state=d["S0"], prep=p)
    st = d["S0"].clone()
    o_d = torch.empty(B, T, H, D, device="cuda")
    for t in range(T):
        o_d[:, t] = kda.kda_decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                        d["v"][:, t].contiguous(), d["g"][:, t].contiguous(),
                                        d["beta"][:, t].contiguous(), st, prep=p)
    torch.cuda.synchronize()
    assert rel_err(o_d.cpu().numpy(), o_p.double().cpu().numpy()) < 1e-4
    assert rel_err(st.cpu().numpy(), S_p.double().cpu().numpy()) < 1e-4
