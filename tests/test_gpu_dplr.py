"""GPU parity of kda_dplr_chunk_fwd (general diagonal-plus-low-rank forward)
against the fp64 oracle's token recurrence, with the bounds of the KDA
forward (max |gpu - ref| / RMS(ref) below 1e-4 for float32 inputs, 2e-2 for
bfloat16, for outputs and final states)."""
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


def run(d, chunk, cu=None):
    o, S = kda.kda_dplr_chunk_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["g"], chunk=chunk,
                                  initial_state=d["S0"], cu_seqlens=cu)
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


def ref(d, cu=None, heads=None):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, :, heads])
    D = d["q"].shape[-1]
    S0 = None if d["S0"] is None else d["S0"].double().cpu().numpy()
    if S0 is not None and heads is not None:
        S0 = S0[:, heads]
    return oracle.dplr_fwd(*(np32(sel(d[n])) for n in ("q", "k", "v", "a", "b", "g")), D ** -0.5,
                           S0=S0, cu_seqlens=None if cu is None else cu.cpu().numpy())


def supported(D, chunk, dtype):
    return kda.kda_dplr_chunk_fwd_workspace_bytes(1, 64, 1, D, D, chunk, 0, dtype) > 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_dplr_forward(dtype, D, chunk):
    if not supported(D, chunk, dtype):
        pytest.skip("fp32 tiles of this size exceed LDS (KDA_ERR_UNSUPPORTED)")
    d = kda_inputs.dplr_inputs(700 + D + chunk, 2, 150, 2, D, D, dtype, "cuda", s0_std=0.1)
    o, S = run(d, chunk)
    ro, rS = ref(d)
    assert rel_err(o, ro) < TOL[dtype] and rel_err(S, rS) < TOL[dtype], (rel_err(o, ro),
                                                                         rel_err(S, rS))


@pytest.mark.parametrize("dtype,D,chunk", [(torch.bfloat16, 128, 64), (torch.float32, 64, 16)])
def test_dplr_varlen(dtype, D, chunk):
    lens = [1, 63, 64, 65, 130, 7, 0]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    d = kda_inputs.dplr_inputs(71, 1, int(sum(lens)), 3, D, D, dtype, "cuda", s0_std=0.1,
                               n_states=len(lens))
    o, S = run(d, chunk, cu)
    ro, rS = ref(d, cu)
    assert rel_err(o, ro) < TOL[dtype] and rel_err(S, rS) < TOL[dtype]
    assert np.array_equal(S[-1], d["S0"][-1].cpu().numpy())      # empty sequence


@pytest.mark.parametrize("dtype,D,chunk", [(torch.bfloat16, 128, 64), (torch.float32, 64, 64),
                                           (torch.float32, 128, 32)])
def test_dplr_any_gate(dtype, D, chunk):
    """log alpha ~ -U(0.1, 5) per token and channel: every 16-token sub-block
    takes the exact diagonal path for its four Gram tiles, and the bridges
    between sub-blocks are products of factors below one."""
    d = kda_inputs.dplr_inputs(720 + D + chunk, 2, 300, 2, D, D, dtype, "cuda", s0_std=0.1,
                               g_range=(0.1, 5.0))
    o, S = run(d, chunk)
    ro, rS = ref(d)
    assert rel_err(o, ro) < TOL[dtype] and rel_err(S, rS) < TOL[dtype], (rel_err(o, ro),
                                                                         rel_err(S, rS))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 64])
def test_dplr_mixed_decay(dtype, D, chunk):
    """Gates whose 16-token sums straddle the exact-path threshold (-8 for
    bf16 inputs, -40 for fp32): within one chunk some sub-blocks take the
    matrix-core diagonal tiles and others the exact path."""
    if not supported(D, chunk, dtype):
        pytest.skip("fp32 tiles of this size exceed LDS (KDA_ERR_UNSUPPORTED)")
    gr = (0.001, 1.0) if dtype == torch.bfloat16 else (1.5, 3.5)
    d = kda_inputs.dplr_inputs(740 + D + chunk, 2, 3 * chunk + 9, 2, D, D, dtype, "cuda",
                               s0_std=0.1, g_range=gr)
    o, S = run(d, chunk)
    ro, rS = ref(d)
    assert rel_err(o, ro) < TOL[dtype] and rel_err(S, rS) < TOL[dtype], (rel_err(o, ro),
                                                                         rel_err(S, rS))


def test_dplr_huge_gates():
    """Scattered per-channel gates of -1e6 and whole tokens at -1e30 (alpha = 0)
    among the usual ones, bf16, d = 128, chunk 64."""
    d = kda_inputs.dplr_inputs(760, 1, 400, 2, 128, 128, torch.bfloat16, "cuda", s0_std=0.1)
    gen = torch.Generator(device="cuda").manual_seed(761)
    u = torch.rand(d["g"].shape, device="cuda", generator=gen)
    g = torch.where(u < 0.03, torch.full_like(d["g"], -1e6), d["g"])
    tok = torch.rand(d["g"].shape[:3], device="cuda", generator=gen) < 0.02
    g = torch.where(tok[..., None], torch.full_like(g, -1e30), g)
    d["g"] = g.contiguous()
    o, S = run(d, 64)
    ro, rS = ref(d)
    tol = TOL[torch.bfloat16]
    assert rel_err(o, ro) < tol and rel_err(S, rS) < tol, (rel_err(o, ro), rel_err(S, rS))


def test_dplr_reduces_to_kda():
    """a = beta k, b = alpha * k, write key beta k: the DPLR kernels give the
    KDA kernels' result (fp32, within rounding)."""
    B, T, H, D = 1, 200, 2, 64
    d = kda_inputs.prefill_inputs(72, B, T, H, D, D, torch.float32, "cuda", s0_std=0.1)
    bk = (d["beta"][..., None] * d["k"]).contiguous()
    ak = (torch.exp(d["g"]) * d["k"]).contiguous()
    o1, S1 = kda.kda_dplr_chunk_fwd(d["q"], bk, d["v"], bk, ak, d["g"], chunk=32,
                                    initial_state=d["S0"])
    o2, S2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=32,
                               initial_state=d["S0"])
    torch.cuda.synchronize()
    assert rel_err(o1.cpu().numpy(), o2.double().cpu().numpy()) < 1e-4
    assert rel_err(S1.cpu().numpy(), S2.double().cpu().numpy()) < 1e-4


def test_dplr_zero_tokens_keeps_state():
    d = kda_inputs.dplr_inputs(73, 1, 0, 2, 64, 64, torch.bfloat16, "cuda", s0_std=0.1)
    o, S = run(d, 64)
    assert o.size == 0 and np.array_equal(S, d["S0"].cpu().numpy())


def test_dplr_config2_all_heads():
    """The 32K-token layer shape (B 1, H 32, d 128, bf16, chunk 64) as the
    benchmark runs it; every output and final state against the oracle."""
    d = kda_inputs.dplr_inputs(74, 1, 32768, 32, 128, 128, torch.bfloat16, "cuda")
    o, S = run(d, 64)
    ro, rS = ref(d)
    assert rel_err(o, ro) < TOL[torch.bfloat16]
    assert rel_err(S, rS) < TOL[torch.bfloat16]


def test_dplr_config2_strong_gates_all_heads():
    """The 32K-token layer shape with log alpha ~ -U(0.1, 5): every sub-block
    takes the exact diagonal path; every output and final state."""
    d = kda_inputs.dplr_inputs(75, 1, 32768, 32, 128, 128, torch.bfloat16, "cuda",
                               g_range=(0.1, 5.0))
    o, S = run(d, 64)
    ro, rS = ref(d)
    assert rel_err(o, ro) < TOL[torch.bfloat16]
    assert rel_err(S, rS) < TOL[torch.bfloat16]
