"""GPU parity of the output epilogue (per-head RMSNorm, weight, sigmoid output
gate) of kda_chunk_fwd_ex and kda_decode_step_ex against the fp64 oracle with
the same epilogue, alone and together with the input preparation."""
import numpy as np
import pytest
import torch

import kda_inputs
import linear_attention_sequence_chunkwise_amd as kda
import oracle
from kda_testlib import TOL, np32, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def epi_params(seed, shape_o, dtype, weight=True, gate=True, eps=1e-6):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    dv = shape_o[-1]
    w = (0.5 + torch.rand(dv, device="cuda", generator=gen)) if weight else None
    z = torch.randn(*shape_o, device="cuda", generator=gen).to(dtype) if gate else None
    return dict(eps=eps, weight=w, gate=z)


def np_epi(e):
    return {kk: (np32(vv) if torch.is_tensor(vv) else vv) for kk, vv in e.items()}


def np_prep(p):
    return None if p is None else {kk: (np32(vv) if torch.is_tensor(vv) else vv)
                                   for kk, vv in p.items()}


def check_prefill(d, chunk, epi, prep=None, cu=None, tol=None):
    o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=chunk,
                             initial_state=d.get("S0"), cu_seqlens=cu, prep=prep, epilogue=epi)
    torch.cuda.synchronize()
    D = d["q"].shape[-1]
    S0 = d.get("S0")
    ro, rS = oracle.kda_fwd(np32(d["q"]), np32(d["k"]), np32(d["v"]), np32(d["g"]),
                            np32(d["beta"]), D ** -0.5,
                            S0=None if S0 is None else S0.double().cpu().numpy(),
                            cu_seqlens=None if cu is None else cu.cpu().numpy(),
                            prep=np_prep(prep), epilogue=np_epi(epi))
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(S.cpu().numpy(), rS)
    tol = tol or TOL[d["q"].dtype]
    assert eo < tol and es < tol, (eo, es)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 64])
def test_prefill_epilogue(dtype, D, chunk):
    d = kda_inputs.prefill_inputs(300 + D + chunk, 2, 150, 3, D, D, dtype, "cuda", s0_std=0.1)
    check_prefill(d, chunk, epi_params(1, (2, 150, 3, D), dtype))


@pytest.mark.parametrize("weight,gate", [(False, False), (True, False), (False, True)])
def test_prefill_epilogue_parts(weight, gate):
    d = kda_inputs.prefill_inputs(31, 1, 130, 2, 64, 64, torch.float32, "cuda", s0_std=0.1)
    check_prefill(d, 64, epi_params(2, (1, 130, 2, 64), torch.float32, weight, gate))


def test_prefill_epilogue_with_preparation_varlen_bf16():
    lens = [1, 63, 64, 65, 130, 7]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    T = int(sum(lens))
    raw = kda_inputs.raw_layer_inputs(41, 1, T, 4, 128, 128, torch.bfloat16, "cuda")
    raw["S0"] = 0.1 * torch.randn(len(lens), 4, 128, 128, device="cuda")
    prep = dict(normalize_qk=True, eps=1e-6, beta_logit=True, A_log=raw["A_log"],
                dt_bias=raw["dt_bias"])
    check_prefill(raw, 64, epi_params(3, (1, T, 4, 128), torch.bfloat16), prep=prep, cu=cu)


def test_prefill_config2_with_preparation_and_epilogue():
    """The 32K-token layer with both fused steps, as the benchmark runs it;
    every output and final state against the oracle with the same steps."""
    B, T, H, D = 1, 32768, 32, 128
    raw = kda_inputs.raw_layer_inputs(kda_inputs.CFG_SEED[2] + 50, B, T, H, D, D,
                                      torch.bfloat16, "cuda")
    prep = dict(normalize_qk=True, eps=1e-6, beta_logit=True, A_log=raw["A_log"],
                dt_bias=raw["dt_bias"])
    epi = epi_params(4, (B, T, H, D), torch.bfloat16)
    o, S = kda.kda_chunk_fwd(raw["q"], raw["k"], raw["v"], raw["g"], raw["beta"], chunk=64,
                             prep=prep, epilogue=epi)
    torch.cuda.synchronize()
    p1 = dict(normalize_qk=True, eps=1e-6, beta_logit=True, A_log=np32(raw["A_log"]),
              dt_bias=np32(raw["dt_bias"]))
    e1 = dict(eps=1e-6, weight=np32(epi["weight"]), gate=np32(epi["gate"]))
    ro, rS = oracle.kda_fwd(np32(raw["q"]), np32(raw["k"]), np32(raw["v"]), np32(raw["g"]),
                            np32(raw["beta"]), D ** -0.5, prep=p1, epilogue=e1)
    assert rel_err(o.cpu().numpy(), ro) < TOL[torch.bfloat16]
    assert rel_err(S.cpu().numpy(), rS) < TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("with_prep", [False, True])
def test_decode_epilogue(dtype, D, with_prep):
    N, H, slots = 6, 3, 8
    raw = kda_inputs.raw_layer_inputs(400 + D, 1, N, H, D, D, dtype, "cuda")
    x = {kk: (vv[0].contiguous() if vv.dim() >= 3 else vv) for kk, vv in raw.items()}
    if not with_prep:
        x["q"] = torch.nn.functional.normalize(x["q"].float(), dim=-1).to(dtype)
        x["k"] = torch.nn.functional.normalize(x["k"].float(), dim=-1).to(dtype)
        x["beta"] = torch.sigmoid(x["beta"])
        x["g"] = -0.05 * torch.rand_like(x["g"])
    prep = (dict(normalize_qk=True, eps=1e-6, beta_logit=True, A_log=x["A_log"],
                 dt_bias=x["dt_bias"]) if with_prep else None)
    epi = epi_params(5, (N, H, D), dtype)
    gen = torch.Generator(device="cuda").manual_seed(3)
    state = 0.2 * torch.randn(slots, H, D, D, device="cuda", generator=gen)
    idx = torch.tensor([5, 0, 7, 2, 30, 3], dtype=torch.int32, device="cuda")  # 30: no-op
    ref_state = state.double().cpu().numpy().copy()
    o = torch.full((N, H, D), 7.0, device="cuda")
    kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, slot_idx=idx, o=o,
                        prep=prep, epilogue=epi)
    torch.cuda.synchronize()
    ro = oracle.kda_decode_step(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["g"]),
                                np32(x["beta"]), D ** -0.5, ref_state,
                                slot_idx=idx.cpu().numpy(), prep=np_prep(prep),
                                epilogue=np_epi(epi))
    valid = [0, 1, 2, 3, 5]
    assert rel_err(o.cpu().numpy()[valid], ro[valid]) < 1e-5
    assert np.all(o.cpu().numpy()[4] == 7.0)
    assert rel_err(state.cpu().numpy(), ref_state) < 1e-5


@pytest.mark.parametrize("dtype,D,chunk", [(torch.bfloat16, 128, 64), (torch.float32, 64, 32),
                                           (torch.bfloat16, 32, 16)])
@pytest.mark.parametrize("weight,gate", [(True, True), (False, False), (True, False),
                                         (False, True)])
def test_prefill_epilogue_fused_in_segments(dtype, D, chunk, weight, gate):
    """Epilogue fused into the segment-parallel chain's pass with outputs
    (several segments, ragged last chunk), against the oracle."""
    B, T, H = 1, 1100, 2
    assert kda.kda_chunk_fwd_segments(B, T, H, D, D, chunk, 0, dtype) > 2
    d = kda_inputs.prefill_inputs(500 + D + chunk, B, T, H, D, D, dtype, "cuda", s0_std=0.1)
    check_prefill(d, chunk, epi_params(6, (B, T, H, D), dtype, weight, gate))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_epilogue_fused_equals_separate_pass(dtype):
    """Fused epilogue (segment chain) and the separate epilogue pass after the
    per-slice chain agree to rounding."""
    B, T, H, D, chunk = 1, 2000, 2, 64, 32
    d = kda_inputs.prefill_inputs(77, B, T, H, D, D, dtype, "cuda", s0_std=0.1)
    epi = epi_params(8, (B, T, H, D), dtype)
    run = lambda form=None: kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                              chunk=chunk, initial_state=d["S0"], epilogue=epi,
                                              chain_form=form)
    assert kda.kda_chunk_fwd_segments(B, T, H, D, D, chunk, 0, dtype) > 1
    o1, _ = run()
    o2, _ = run("reg16")
    torch.cuda.synchronize()
    assert rel_err(o1.cpu().numpy(), o2.double().cpu().numpy()) < TOL[dtype]


@pytest.mark.parametrize("varlen", [False, True])
def test_prefill_epilogue_fused_in_whole_chains(varlen):
    """Epilogue fused into the one-workgroup-per-chain form (>= 128 chains),
    fixed-length rows and packed sequences, against the oracle."""
    H, D, chunk = 40, 64, 64
    if varlen:
        lens = [150, 0, 64, 1, 300, 77]
        cu = kda_inputs.cu_seqlens_of(lens).cuda()
        B, T, nseq = 1, sum(lens), len(lens)
        d = kda_inputs.prefill_inputs(610, 1, T, H, D, D, torch.bfloat16, "cuda", s0_std=0.1,
                                      n_states=nseq)
    else:
        cu, B, T, nseq = None, 4, 150, 0
        d = kda_inputs.prefill_inputs(611, B, T, H, D, D, torch.bfloat16, "cuda", s0_std=0.1)
    assert kda.kda_chunk_fwd_segments(B, T, H, D, D, chunk, nseq) == -1
    check_prefill(d, chunk, epi_params(7, (B, T, H, D), torch.bfloat16), cu=cu)
