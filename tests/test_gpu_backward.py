"""GPU parity of kda_chunk_bwd (gradients of the chunkwise prefill) against
the oracle's fp64 reverse mode through the token recurrence.

The loss is L = <o, grad_o> + <final_state, grad_final_state> with random
grad_o and grad_final_state; every gradient (q, k, v, g, beta and the
initial state) is compared element by element.  The backward keeps its chunk
records in fp32 and multiplies in fp32 for either input type (bfloat16 inputs
are read exactly), so the bound is the fp32 one for both: max |gpu - ref| /
RMS(ref) below 1e-4.
"""
import numpy as np
import pytest
import torch

import linear_attention_sequence_chunkwise_amd as kda
import oracle
from kda_testlib import make_prefill, np32, rel_err

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")
TOL_BWD = 1e-4


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def cotangents(seed, B, T, H, D, n_states, final=True):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    do = torch.randn(B, T, H, D, device="cuda", generator=gen)
    dSf = torch.randn(n_states, H, D, D, device="cuda", generator=gen) if final else None
    return do, dSf


def run_gpu(d, chunk, do, dSf=None, cu=None, want_dS0=True):
    out = kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, chunk=chunk,
                            initial_state=d.get("S0"), cu_seqlens=cu, grad_final_state=dSf,
                            want_grad_initial_state=want_dS0)
    torch.cuda.synchronize()
    return [None if x is None else x.cpu().numpy() for x in out]


def run_oracle(d, do, dSf=None, cu=None, heads=None):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, :, heads])
    D = d["q"].shape[-1]
    S0 = d.get("S0")
    S0 = None if S0 is None else S0.double().cpu().numpy()
    dsf = None if dSf is None else dSf.double().cpu().numpy()
    if heads is not None:
        S0 = None if S0 is None else S0[:, heads]
        dsf = None if dsf is None else dsf[:, heads]
    return oracle.kda_bwd(np32(sel(d["q"])), np32(sel(d["k"])), np32(sel(d["v"])),
                          np32(sel(d["g"])), np32(sel(d["beta"])), D ** -0.5,
                          sel(do).double().cpu().numpy(), S0=S0,
                          cu_seqlens=None if cu is None else cu.cpu().numpy(), d_S_final=dsf)


def errors(got, ref):
    return {n: rel_err(a, b) for n, a, b in zip(NAMES, got, ref) if a is not None}


def assert_close(got, ref, tol):
    e = errors(got, ref)
    assert all(v < tol for v in e.values()), e


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_backward(dtype, D, chunk):
    """B = 2 rows of 150 tokens (several chunks and a ragged tail), initial
    state and final-state gradient given."""
    B, T, H = 2, 150, 2
    d = make_prefill(500 + D + chunk, B, T, H, D, dtype, s0_std=0.1)
    do, dSf = cotangents(1 + D, B, T, H, D, B)
    assert_close(run_gpu(d, chunk, do, dSf), run_oracle(d, do, dSf), TOL_BWD)


@pytest.mark.parametrize("dtype,chunk", [(torch.bfloat16, 64), (torch.float32, 16),
                                         (torch.float32, 64)])
def test_backward_varlen(dtype, chunk):
    lens = [1, 63, 64, 65, 130, 7]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    T, H, D = int(sum(lens)), 3, 64
    d = make_prefill(61, 1, T, H, D, dtype, s0_std=0.1, n_states=len(lens))
    do, dSf = cotangents(2, 1, T, H, D, len(lens))
    assert_close(run_gpu(d, chunk, do, dSf, cu=cu), run_oracle(d, do, dSf, cu=cu), TOL_BWD)


def test_backward_varlen_with_empty_sequences():
    """Empty sequences pass the final-state gradient straight to the initial
    state; their neighbours are unaffected."""
    lens = [0, 40, 0, 0, 17, 0]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    T, H, D = int(sum(lens)), 2, 64
    d = make_prefill(62, 1, T, H, D, torch.float32, s0_std=0.1, n_states=len(lens))
    do, dSf = cotangents(3, 1, T, H, D, len(lens))
    got = run_gpu(d, 32, do, dSf, cu=cu)
    assert_close(got, run_oracle(d, do, dSf, cu=cu), TOL_BWD)
    for n in (0, 2, 3, 5):
        assert np.array_equal(got[5][n], dSf[n].cpu().numpy())


def test_backward_without_states():
    """No initial state, no final-state gradient, initial-state gradient not
    wanted."""
    B, T, H, D = 1, 200, 2, 128
    d = make_prefill(63, B, T, H, D, torch.bfloat16)
    do, _ = cotangents(4, B, T, H, D, B, final=False)
    got = run_gpu(d, 64, do, None, want_dS0=False)
    assert got[5] is None
    assert_close(got, run_oracle(d, do, None), TOL_BWD)


def test_backward_zero_tokens():
    """T = 0: the initial-state gradient is the final-state gradient."""
    H, D = 2, 64
    d = make_prefill(64, 1, 0, H, D, torch.float32, s0_std=0.1)
    _, dSf = cotangents(5, 1, 0, H, D, 1)
    do = torch.empty(1, 0, H, D, device="cuda")
    got = run_gpu(d, 64, do, dSf)
    assert np.array_equal(got[5], dSf.cpu().numpy())


def test_backward_strong_decay():
    """Gates down to -0.5 per token (chunk decay sums up to ~32), the edge of
    the documented domain, fp32."""
    B, T, H, D = 1, 192, 2, 64
    d = make_prefill(65, B, T, H, D, torch.float32, s0_std=0.1, g_range=(0.05, 0.5))
    do, dSf = cotangents(6, B, T, H, D, B)
    assert_close(run_gpu(d, 64, do, dSf), run_oracle(d, do, dSf), TOL_BWD)


def test_backward_chunk_invariance():
    """The gradients do not depend on the chunk length beyond rounding."""
    B, T, H, D = 2, 100, 2, 64
    d = make_prefill(66, B, T, H, D, torch.float32, s0_std=0.1)
    do, dSf = cotangents(7, B, T, H, D, B)
    g16 = run_gpu(d, 16, do, dSf)
    g64 = run_gpu(d, 64, do, dSf)
    assert all(v < 1e-4 for v in errors(g16, g64).values()), errors(g16, g64)


def test_backward_repeatable():
    """Two calls give bitwise identical gradients (no atomics, fixed order)."""
    B, T, H, D = 1, 300, 4, 128
    d = make_prefill(67, B, T, H, D, torch.bfloat16, s0_std=0.1)
    do, dSf = cotangents(8, B, T, H, D, B)
    a = run_gpu(d, 64, do, dSf)
    b = run_gpu(d, 64, do, dSf)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_backward_config2_sampled():
    """The 32K-token layer (B 1, H 32, d 128, bf16, chunk 64) as the benchmark
    runs it; sampled heads checked against the oracle."""
    B, T, H, D = 1, 32768, 32, 128
    d = make_prefill(68, B, T, H, D, torch.bfloat16, s0_std=0.1)
    do, dSf = cotangents(9, B, T, H, D, B)
    got = run_gpu(d, 64, do, dSf)
    heads = [0, 19, 31]
    ref = run_oracle(d, do, dSf, heads=heads)
    for i, h in enumerate(heads):
        one = [x[:, :, h] for x in got[:5]] + [got[5][:, h]]
        e = errors(one, [x[:, :, i] for x in ref[:5]] + [ref[5][:, i]])
        assert all(v < TOL_BWD for v in e.values()), (h, e)
