"""GPU parity of kda_chunk_fwd (through the C ABI) against the fp64 oracle.

Every case is compared element by element in full: small shapes spanning
several chunks and a ragged tail, and the benchmark-sized configurations
(every head, every output and final state)."""
import numpy as np
import pytest
import torch

import kda_inputs
import linear_attention_sequence_chunkwise_amd as kda
import oracle
from kda_testlib import TOL, make_prefill, np32, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(d, chunk, cu=None, scale=None):
    D = d["q"].shape[-1]
    scale = D ** -0.5 if scale is None else scale
    o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=scale, chunk=chunk,
                             initial_state=d.get("S0"), cu_seqlens=cu)
    torch.cuda.synchronize()
    return o, S


def check(d, chunk, cu=None, heads=None, tol=None):
    D = d["q"].shape[-1]
    o, S = run(d, chunk, cu)
    o_ref, S_ref = oracle_prefill(d, D ** -0.5, heads=heads, cu=cu)
    if heads is not None:
        o, S = o[:, :, heads], S[:, heads]
    tol = TOL[d["q"].dtype] if tol is None else tol
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(S.cpu().numpy(), S_ref)
    print("err_o %.3e err_S %.3e (tol %.0e)" % (eo, es, tol), flush=True)
    assert eo < tol and es < tol
    return eo, es


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_small_ragged(dtype, D, chunk):
    for T, s0 in ((1, None), (chunk - 1, 0.1), (3 * chunk + 5, 0.05), (200, None)):
        d = make_prefill(T * 31 + D + chunk, 2, T, 3, D, dtype, s0_std=s0)
        check(d, chunk)


def test_config0_fp32():
    d = kda_inputs.config_inputs(0, "cuda")
    check(d, 16)


def test_config1_bf16_initial_state():
    d = kda_inputs.config_inputs(1, "cuda")
    check(d, 64)


def test_config2_all_heads():
    """The 32K-token layer (B 1, H 32, T 32768, d 128, chunk 64, bf16) in the
    launch configuration bench.py times: every output and final state."""
    d = kda_inputs.config_inputs(2, "cuda")
    check(d, 64)


def test_config2_strong_gates_all_heads():
    """The 32K-token layer of the benchmark with log alpha ~ -U(0.1, 5): every
    16-token sub-block of every head takes the exact diagonal path, in the
    launch configuration bench.py times; every output and final state."""
    d = make_prefill(13, 1, 32768, 32, 128, torch.bfloat16, s0_std=0.1, g_range=(0.1, 5.0))
    check(d, 64)


def test_config2_few_fast_channels_all_heads():
    """The 32K-token layer with the usual gates except 5 % of each head's
    channels at log alpha ~ -U(1, 2.5) (a gate with a few fast-decaying
    channels): fast and exact sub-blocks side by side in every chunk; every
    output and final state."""
    d = make_prefill(14, 1, 32768, 32, 128, torch.bfloat16, s0_std=0.1)
    gen = torch.Generator(device="cuda").manual_seed(15)
    fast = torch.rand(32, 128, device="cuda", generator=gen) < 0.05
    u = torch.rand(d["g"].shape, device="cuda", generator=gen)
    d["g"] = torch.where(fast, -(1.0 + 1.5 * u), d["g"]).contiguous()
    check(d, 64)


def test_config3_varlen_all_chains():
    """The packed 16-sequence layer: every output and every per-sequence
    final state (512 chains)."""
    d = kda_inputs.config_inputs(3, "cuda")
    check(d, 64, cu=d["cu_seqlens"])


def test_varlen_edge_lengths():
    lens = [0, 1, 63, 64, 65, 0, 130, 2]
    cu = kda_inputs.cu_seqlens_of(lens).cuda()
    d = make_prefill(5, 1, sum(lens), 4, 64, torch.bfloat16, s0_std=0.1, n_states=len(lens))
    check(d, 64, cu=cu)
    d32 = make_prefill(6, 1, sum(lens), 2, 32, torch.float32, s0_std=0.1, n_states=len(lens))
    check(d32, 16, cu=cu)


def test_varlen_equals_separate_calls():
    lens = [70, 5, 128, 33]
    cu = kda_inputs.cu_seqlens_of(lens).cuda()
    d = make_prefill(8, 1, sum(lens), 4, 128, torch.bfloat16, s0_std=0.05, n_states=len(lens))
    o, S = run(d, 64, cu)
    for n, (a, b) in enumerate(zip(cu[:-1].tolist(), cu[1:].tolist())):
        dn = {k: d[k][:, a:b].contiguous() for k in ("q", "k", "v", "g", "beta")}
        dn["S0"] = d["S0"][n:n + 1].contiguous()
        on, Sn = run(dn, 64)
        assert torch.equal(on, o[:, a:b]) and torch.equal(Sn[0], S[n])


def test_split_and_resume():
    B, T, H, D = 2, 300, 4, 128
    d = make_prefill(9, B, T, H, D, torch.bfloat16, s0_std=0.1)
    o, S = run(d, 64)
    m = 130
    d1 = {k: d[k][:, :m].contiguous() for k in ("q", "k", "v", "g", "beta")}
    d1["S0"] = d["S0"]
    o1, S1 = run(d1, 64)
    d2 = {k: d[k][:, m:].contiguous() for k in ("q", "k", "v", "g", "beta")}
    d2["S0"] = S1
    o2, S2 = run(d2, 64)
    o_ref, S_ref = oracle_prefill(d, D ** -0.5)
    assert rel_err(torch.cat([o1, o2], 1).cpu().numpy(), o_ref) < TOL[torch.bfloat16]
    assert rel_err(S2.cpu().numpy(), S_ref) < TOL[torch.bfloat16]


def test_in_place_state_and_determinism():
    B, T, H, D = 2, 257, 8, 64
    d = make_prefill(10, B, T, H, D, torch.bfloat16, s0_std=0.1)
    o1, S1 = run(d, 64)
    st = d["S0"].clone()
    o2, S2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64,
                               initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, st)


def test_strong_decay():
    """Per-token log gates down to -0.6: 16-token sub-block sums around -5.4,
    near the edge where sub-blocks start to take the exact diagonal path."""
    d = make_prefill(12, 1, 512, 4, 128, torch.bfloat16, s0_std=0.1, g_range=(0.05, 0.6))
    check(d, 64)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_strong_decay_any_gate(dtype):
    """log alpha ~ -U(0.1, 5) per token and channel (16-token sums around -41):
    every sub-block's diagonal Gram tiles take the exact path; the state of a
    chunk is forgotten within a few tokens, so the outputs are dominated by
    the most recent tokens.  d = 128, chunk 64, with an initial state."""
    d = make_prefill(40, 2, 700, 4, 128, dtype, s0_std=0.1, g_range=(0.1, 5.0))
    check(d, 64)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_mixed_decay(dtype, D, chunk):
    """Gates whose 16-token sums straddle the exact-path threshold (-8 for
    bf16 inputs, -40 for fp32): within one chunk some sub-blocks take the
    matrix-core diagonal tiles and others the exact path."""
    gr = (0.001, 1.0) if dtype == torch.bfloat16 else (1.5, 3.5)
    d = make_prefill(41 + D + chunk, 2, 3 * chunk + 9, 3, D, dtype, s0_std=0.1, g_range=gr)
    check(d, chunk)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_huge_gates(dtype):
    """Most gates in the usual range, with scattered per-channel gates of -1e6
    and whole tokens at -1e30 (alpha = 0): the decay factors between
    sub-blocks are summed directly, so a huge gate sum in one sub-block does
    not swamp the factors of its neighbours."""
    d = make_prefill(42, 1, 400, 4, 128, dtype, s0_std=0.1)
    gen = torch.Generator(device="cuda").manual_seed(43)
    u = torch.rand(d["g"].shape, device="cuda", generator=gen)
    g = torch.where(u < 0.03, torch.full_like(d["g"], -1e6), d["g"])
    tok = torch.rand(d["g"].shape[:3], device="cuda", generator=gen) < 0.02
    g = torch.where(tok[..., None], torch.full_like(g, -1e30), g)
    d["g"] = g.contiguous()
    check(d, 64)


def test_empty_input_copies_state():
    d = make_prefill(13, 2, 0, 2, 64, torch.bfloat16, s0_std=0.1)
    o, S = run(d, 64)
    assert o.numel() == 0 and torch.equal(S, d["S0"])



def test_prefill_under_graph_capture():
    """A long prefill captured into a HIP graph replays correctly, several
    times, with other work in between."""
    B, T, H, D = 1, 16384, 8, 128
    d = kda_inputs.prefill_inputs(83, B, T, H, D, D, torch.bfloat16, "cuda", s0_std=0.1)
    ref_o, ref_S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64,
                                     initial_state=d["S0"])
    torch.cuda.synchronize()
    ref_o, ref_S = ref_o.cpu().numpy(), ref_S.cpu().numpy()
    o = torch.empty(B, T, H, D, device="cuda")
    S = torch.empty(B, H, D, D, device="cuda")
    ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(B, T, H, D, D, 64), dtype=torch.uint8,
                     device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up outside the capture
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64,
                          initial_state=d["S0"], o=o, final_state=S, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64,
                          initial_state=d["S0"], o=o, final_state=S, workspace=ws, stream=s)
    for rep in range(3):
        o.fill_(0.0)
        S.fill_(0.0)
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(o.cpu().numpy(), ref_o), rep
        assert np.array_equal(S.cpu().numpy(), ref_S), rep
        del junk


def test_concurrent_streams():
    """Two prefills on two streams at once give the results of running them one
    after the other (the library keeps no state between calls)."""
    B, T, H, D = 1, 4096, 8, 128
    da = kda_inputs.prefill_inputs(84, B, T, H, D, D, torch.bfloat16, "cuda", s0_std=0.1)
    db = kda_inputs.prefill_inputs(85, B, T, H, D, D, torch.bfloat16, "cuda", s0_std=0.1)
    run = lambda d, st=None: kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                               chunk=64, initial_state=d["S0"], stream=st)
    ra, rb = run(da), run(db)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        ca = run(da, s1)
    with torch.cuda.stream(s2):
        cb = run(db, s2)
    torch.cuda.synchronize()
    for x, y in zip(ra + rb, ca + cb):
        assert torch.equal(x, y)


def test_side_stream_not_current():
    """stream= a side stream that is not made current: the binding allocates
    the outputs and the workspace on that stream, and a burst of allocations
    on the current stream meanwhile (which would reuse a block freed on the
    wrong stream) does not disturb the result."""
    B, T, H, D = 1, 8192, 8, 128
    d = kda_inputs.prefill_inputs(86, B, T, H, D, D, torch.bfloat16, "cuda", s0_std=0.1)
    ref_o, ref_S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64,
                                     initial_state=d["S0"])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        o, S = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64,
                                 initial_state=d["S0"], stream=s)
        junk = [torch.full((1 << 20,), float(i), device="cuda") for i in range(64)]
        s.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(S, ref_S), rep
        del junk, o, S


# Shapes where the chain is cut into segments (B*H small, many chunks), each
# with a ragged last chunk: (B, T, H, d, chunk, dtype).
SEG_CASES = [
    (2, 1000, 2, 64, 64, torch.bfloat16),
    (1, 1100, 3, 128, 64, torch.bfloat16),
    (1, 700, 2, 32, 16, torch.float32),
    (2, 1050, 2, 64, 32, torch.float32),
    (1, 1000, 4, 128, 16, torch.float32),
]


def _segments(B, T, H, D, chunk, dtype):
    return kda.kda_chunk_fwd_segments(B, T, H, D, D, chunk, 0, dtype)


@pytest.mark.parametrize("case", SEG_CASES, ids=lambda c: "B%dT%dH%dd%dC%d%s" % (
    c[0], c[1], c[2], c[3], c[4], "bf16" if c[5] == torch.bfloat16 else "f32"))
@pytest.mark.parametrize("s0", [None, 0.1])
def test_segmented_chain(case, s0):
    """Segment-parallel chain (local runs, transition products, combine, rerun)
    against the oracle, element by element."""
    B, T, H, D, chunk, dtype = case
    assert _segments(*case) > 2, case
    d = make_prefill(B * 7 + T + D + chunk, B, T, H, D, dtype, s0_std=s0)
    check(d, chunk)


def test_two_segments():
    """Two segments: the second starts from the first's end state, no
    transition product is formed."""
    B, T, H, D = 1, 8 * 64, 32, 128
    assert kda.kda_chunk_fwd_segments(B, T, H, D, D, 64) == 2
    d = make_prefill(81, B, T, H, D, torch.bfloat16, s0_std=0.1)
    check(d, 64)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_segmented_equals_slice_chain(dtype):
    """The segment-parallel chain and the per-slice chain agree to rounding."""
    B, T, H, D, chunk = 1, 2000, 2, 64, 32
    assert kda.kda_chunk_fwd_segments(B, T, H, D, D, chunk, 0, dtype) > 1
    d = make_prefill(82, B, T, H, D, dtype, s0_std=0.1)
    o1, S1 = run(d, chunk)
    o2, S2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=chunk,
                               initial_state=d["S0"], chain_form="reg16")
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert rel_err(o1.cpu().numpy(), o2.double().cpu().numpy()) < tol
    assert rel_err(S1.cpu().numpy(), S2.double().cpu().numpy()) < tol


def test_segmented_in_place_state():
    """final_state aliasing initial_state: the first segment reads its copy of
    S0, so the last segment's write cannot race with it."""
    B, T, H, D = 1, 4096, 8, 128
    assert kda.kda_chunk_fwd_segments(B, T, H, D, D, 64) > 1
    d = make_prefill(83, B, T, H, D, torch.bfloat16, s0_std=0.1)
    o1, S1 = run(d, 64)
    st = d["S0"].clone()
    o2, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64,
                              initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, st)


def test_single_chain_many_segments():
    """One (sequence, head) chain cut into 32 segments (the cap): 30 combine
    steps, each segment rerun from its combined state."""
    B, T, H, D = 1, 32 * 4 * 64 - 20, 1, 128
    assert kda.kda_chunk_fwd_segments(B, T, H, D, D, 64) == 32
    d = make_prefill(90, B, T, H, D, torch.bfloat16, s0_std=0.1)
    check(d, 64)


# ---- one workgroup per whole (sequence, head) chain ----

@pytest.mark.parametrize("D,chunk,dtype", [(128, 64, torch.bfloat16), (64, 32, torch.bfloat16),
                                           (32, 16, torch.float32)])
@pytest.mark.parametrize("s0", [None, 0.1])
def test_whole_chain(D, chunk, dtype, s0):
    """B*H >= 128 chains too many to split: each runs whole in one workgroup
    over all columns; every output and state against the oracle."""
    B, T, H = 4, 3 * chunk + 7, 40
    assert kda.kda_chunk_fwd_segments(B, T, H, D, D, chunk, 0, dtype) == -1
    d = make_prefill(91 + D + chunk, B, T, H, D, dtype, s0_std=s0)
    check(d, chunk)


def _varlen_many(seed, H, D, dtype, lens):
    cu = kda_inputs.cu_seqlens_of(lens).cuda()
    d = make_prefill(seed, 1, sum(lens), H, D, dtype, s0_std=0.1, n_states=len(lens))
    return d, cu


def test_whole_chain_varlen():
    """Packed sequences with >= 128 chains: whole chains, longest first, with
    empty, one-token, partial-chunk and multi-chunk sequences."""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(0, 300, size=37)] + [0, 1, 63, 64, 65, 700]
    H, D = 4, 64
    assert kda.kda_chunk_fwd_segments(1, sum(lens), H, D, D, 64, len(lens)) == -1
    d, cu = _varlen_many(92, H, D, torch.bfloat16, lens)
    check(d, 64, cu=cu)


def test_whole_chain_equals_slice_chain():
    """The whole-chain form and the per-slice chain agree to rounding, for
    packed sequences and in place (final_state aliasing initial_state)."""
    lens = [200, 0, 64, 1000, 17, 333, 64 * 5, 90] * 5
    H, D = 4, 128
    d, cu = _varlen_many(93, H, D, torch.bfloat16, lens)
    assert kda.kda_chunk_fwd_segments(1, sum(lens), H, D, D, 64, len(lens)) == -1
    o1, S1 = run(d, 64, cu=cu)
    st = d["S0"].clone()
    o3, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64,
                              initial_state=st, final_state=st, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(S1, st)
    o2, S2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=64,
                               initial_state=d["S0"], cu_seqlens=cu, chain_form="reg16")
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert rel_err(o1.cpu().numpy(), o2.double().cpu().numpy()) < tol
    assert rel_err(S1.cpu().numpy(), S2.double().cpu().numpy()) < tol


def test_whole_chain_many_sequences_unordered():
    """More packed sequences than the length ranking covers (1100 > 1024): the
    whole-chain form runs them in the given order, still every output and
    state against the oracle."""
    rng = np.random.default_rng(6)
    lens = [int(x) for x in rng.integers(0, 40, size=1100)]
    H, D = 1, 32
    assert kda.kda_chunk_fwd_segments(1, sum(lens), H, D, D, 16, len(lens)) == -1
    d, cu = _varlen_many(94, H, D, torch.bfloat16, lens)
    check(d, 16, cu=cu)
