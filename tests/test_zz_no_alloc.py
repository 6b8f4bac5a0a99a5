"""kda_chunk_fwd_noalloc, the prefill entry point that allocates nothing (its
workspace is the library's fixed per-GPU scratch), called through the C ABI
and compared with kda_chunk_fwd on a caller-allocated workspace: the same
kernels on the same inputs give the same bits.  Two calls in a row, the
second smaller (the scratch keeps the first call's contents), each also
checked against the oracle at the input dtype's bound."""
import pytest
import torch

import linear_attention_sequence_chunkwise_amd as kda
from kda_testlib import TOL, make_prefill, oracle_prefill, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(d, chunk, cu=None):
    D = d["q"].shape[-1]
    o_ref, S_ref = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk=chunk,
                                     initial_state=d.get("S0"), cu_seqlens=cu)
    o = torch.full_like(o_ref, 3.0)
    S = torch.full_like(S_ref, 3.0)
    kda.kda_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], o, S, chunk=chunk,
                              initial_state=d.get("S0"), cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    ro, rS = oracle_prefill(d, D ** -0.5, cu=cu)
    tol = TOL[d["q"].dtype]
    assert rel_err(o.cpu().numpy(), ro) < tol and rel_err(S.cpu().numpy(), rS) < tol


def test_noalloc_two_calls_second_smaller():
    # segment-parallel chain, 32 chunks of 64 tokens x 8 heads at d = 128
    _pair(make_prefill(901, 1, 2000, 8, 128, torch.bfloat16, s0_std=0.1), 64)
    # then a smaller call with another plan (per-slice chain, d = 64)
    _pair(make_prefill(902, 2, 300, 4, 64, torch.bfloat16, s0_std=0.1), 32)


def test_noalloc_packed_and_fp32():
    lens = [70, 5, 300, 0, 33]
    cu = torch.tensor([0, 70, 75, 375, 375, 408], dtype=torch.int32, device="cuda")
    _pair(make_prefill(903, 1, sum(lens), 4, 128, torch.bfloat16, s0_std=0.1,
                       n_states=len(lens)), 64, cu=cu)
    _pair(make_prefill(904, 1, 200, 2, 32, torch.float32, s0_std=0.1), 16)


def test_noalloc_rejects_calls_beyond_the_scratch():
    # 32 heads x 8192 tokens at d = 128 needs far more than the fixed scratch
    need = kda.kda_chunk_fwd_workspace_bytes(1, 8192, 32, 128, 128, 64)
    assert need > kda.NOALLOC_SCRATCH_BYTES
    d = make_prefill(905, 1, 8192, 32, 128, torch.bfloat16)
    o = torch.zeros(1, 8192, 32, 128, device="cuda")
    with pytest.raises(kda.KDAError) as e:
        kda.kda_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], o)
    assert e.value.code == 7
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0
