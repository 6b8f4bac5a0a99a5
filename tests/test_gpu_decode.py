"""GPU parity of kda_decode_step (through the C ABI) against the fp64 oracle."""
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


def _step_inputs(seed, N, H, D, dtype):
    return kda_inputs.decode_inputs(seed, 0, N, H, D, D, dtype, "cuda")


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_small_with_slots(D, dtype):
    N, H, slots = 5, 3, 9
    torch.manual_seed(0)
    x = _step_inputs(11 + D, N, H, D, dtype)
    gen = torch.Generator(device="cuda").manual_seed(5)
    state = 0.3 * torch.randn(slots, H, D, D, device="cuda", generator=gen)
    idx = torch.tensor([7, 0, 3, 42, 5], dtype=torch.int32, device="cuda")   # 42: no-op
    ref_state = state.double().cpu().numpy().copy()
    o = torch.full((N, H, D), 123.0, device="cuda")
    kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, scale=D ** -0.5,
                        slot_idx=idx, o=o)
    torch.cuda.synchronize()
    o_ref = oracle.kda_decode_step(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["g"]),
                                   np32(x["beta"]), D ** -0.5, ref_state,
                                   slot_idx=idx.cpu().numpy())
    valid = [0, 1, 2, 4]
    tol = TOL[dtype] if dtype == torch.float32 else 1e-5   # one step: fp32 arithmetic only
    assert rel_err(o.cpu().numpy()[valid], o_ref[valid]) < max(tol, 1e-5)
    assert np.all(o.cpu().numpy()[3] == 123.0)            # skipped row untouched
    assert rel_err(state.cpu().numpy(), ref_state) < 1e-5
    untouched = [1, 2, 4, 6, 8]
    assert np.array_equal(state.cpu().numpy()[untouched], ref_state[untouched].astype(np.float32))


def test_decode_identity_slots_full_width():
    """One step at the decode benchmark's width: N=256, H=32, d=128."""
    N, H, D = 256, 32, 128
    x = _step_inputs(1004, N, H, D, torch.bfloat16)
    gen = torch.Generator(device="cuda").manual_seed(9)
    state = 0.5 * torch.randn(N, H, D, D, device="cuda", generator=gen)
    ref_state = state.double().cpu().numpy()
    o = kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state)
    torch.cuda.synchronize()
    o_ref = oracle.kda_decode_step(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["g"]),
                                   np32(x["beta"]), D ** -0.5, ref_state)
    assert rel_err(o.cpu().numpy(), o_ref) < 1e-5
    assert rel_err(state.cpu().numpy(), ref_state) < 1e-5


def test_decode_matches_prefill_and_is_deterministic():
    """T decode steps from S0 == one prefill over the same T tokens (GPU vs GPU
    and both vs the oracle); two identical runs are bitwise equal."""
    B, T, H, D = 2, 40, 4, 64
    d = kda_inputs.prefill_inputs(77, B, T, H, D, D, torch.bfloat16, "cuda", s0_std=0.1)
    o_p, S_p = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=16,
                                 initial_state=d["S0"])
    outs = []
    for rep in range(2):
        st = d["S0"].clone()
        o_d = torch.empty(B, T, H, D, device="cuda")
        for t in range(T):
            o_d[:, t] = kda.kda_decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                            d["v"][:, t].contiguous(), d["g"][:, t].contiguous(),
                                            d["beta"][:, t].contiguous(), st)
        outs.append((o_d, st))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    o_ref, S_ref = oracle.kda_fwd(np32(d["q"]), np32(d["k"]), np32(d["v"]), np32(d["g"]),
                                  np32(d["beta"]), D ** -0.5, S0=d["S0"].double().cpu().numpy())
    assert rel_err(outs[0][0].cpu().numpy(), o_ref) < 1e-5
    assert rel_err(outs[0][1].cpu().numpy(), S_ref) < 1e-5
    assert rel_err(o_p.cpu().numpy(), o_ref) < TOL[torch.bfloat16]
    assert rel_err(S_p.cpu().numpy(), S_ref) < TOL[torch.bfloat16]


def test_config4_decode_workload():
    """The decode benchmark's workload exactly as bench.py times it: a 256 x 32
    x 128 x 128 cache filled by a 4096-token prefill per sequence (32 per call),
    then 512 decode steps with fresh inputs.  Every chain (8192) is recomputed
    by the oracle -- prefill over the same 4096 tokens, then the 512 steps --
    and compared at every step's output and in the final state, jointly.  To
    separate the decode's own error from the prefill's, the oracle's steps are
    also run from the GPU's prefill states for the first 32 sequences, held to
    the fp32 bound."""
    import bench
    stream = torch.cuda.current_stream()
    n_steps = 512
    cache, steps, o = bench.decode_setup(kda, kda_inputs, n_steps, stream)
    nd = 32   # decode-only check: the oracle's steps restarted from the GPU's prefill states
    gpu_init = cache[:nd].double().cpu().numpy()
    bench.decode_run(kda, cache, steps, o, stream)
    torch.cuda.synchronize()
    N, D = cache.shape[0], cache.shape[-1]
    st = gpu_init.copy()
    o_dec = np.empty((n_steps, nd) + tuple(o.shape[2:]))
    for s in range(n_steps):
        x = {name: np32(steps[s][name][:nd]) for name in ("q", "k", "v", "g", "beta")}
        o_dec[s] = oracle.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], D ** -0.5, st)
    e_dec = rel_err(o[:, :nd].cpu().numpy(), o_dec)
    e_dst = rel_err(cache[:nd].cpu().numpy(), st)
    print("decode alone (from the GPU's prefill states): err_o %.2e err_S %.2e" % (e_dec, e_dst),
          flush=True)
    assert e_dec < 1e-5 and e_dst < 1e-5
    NB = bench.DECODE_INIT_BATCH
    ref_state = []
    for b0 in range(0, N, NB):
        d = bench.decode_init_inputs(kda_inputs, b0, "cuda")
        _, S = oracle.kda_fwd(np32(d["q"]), np32(d["k"]), np32(d["v"]), np32(d["g"]),
                              np32(d["beta"]), D ** -0.5)
        ref_state.append(S)
        del d
        print("oracle prefill of sequences %d..%d done" % (b0, b0 + NB - 1), flush=True)
    state = np.concatenate(ref_state, 0)       # [N, H, D, D] fp64
    del ref_state
    err_o = 0.0
    o_host = o.cpu().numpy()
    sq, rms = 0.0, 0
    o_ref = np.empty(o_host.shape[1:])
    for s in range(n_steps):
        x = {name: np32(steps[s][name]) for name in ("q", "k", "v", "g", "beta")}
        o_ref[...] = oracle.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], D ** -0.5,
                                            state)
        err_o = max(err_o, float(np.max(np.abs(o_host[s] - o_ref))))
        sq += float(np.sum(o_ref * o_ref))
        rms += o_ref.size
        if s % 128 == 127:
            print("oracle decode step %d done" % s, flush=True)
    err_o /= np.sqrt(sq / rms)
    print("decode err_o %.3e" % err_o, flush=True)
    assert err_o < TOL[torch.bfloat16]
    assert rel_err(cache.cpu().numpy(), state) < TOL[torch.bfloat16]
