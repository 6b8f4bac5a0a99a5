"""The Python binding's argument checks, on the CPU (no GPU call is made).

The C ABI receives bare pointers, so a tensor of the wrong shape would make
the kernels read or write past its end.  The binding therefore checks every
tensor's exact shape against q's sizes (and that the tensors live on a GPU)
before it calls the library; these tests hand it mis-shaped CPU tensors and
expect a ValueError naming the problem, raised before any device work.
"""
import pytest
import torch

import linear_attention_sequence_chunkwise_amd as kda

B, T, H, D = 1, 8, 2, 32


def prefill_args(**over):
    f = dict(dtype=torch.float32)
    a = dict(q=torch.zeros(B, T, H, D, dtype=torch.bfloat16),
             k=torch.zeros(B, T, H, D, dtype=torch.bfloat16),
             v=torch.zeros(B, T, H, D, dtype=torch.bfloat16),
             g=torch.zeros(B, T, H, D, **f), beta=torch.zeros(B, T, H, **f))
    a.update(over)
    return a


@pytest.fixture(autouse=True)
def _lib():
    try:
        kda.load_library()
    except (RuntimeError, OSError) as e:
        pytest.skip("libkda.so not loadable: %s" % e)


@pytest.mark.parametrize("name,bad", [
    ("k", torch.zeros(B, T, H, D + 1, dtype=torch.bfloat16)),
    ("v", torch.zeros(B, T + 1, H, D, dtype=torch.bfloat16)),
    ("g", torch.zeros(B, T, H, dtype=torch.float32)),          # a per-head scalar gate
    ("beta", torch.zeros(B, T, H, D, dtype=torch.float32)),
])
def test_prefill_rejects_misshaped_token_tensors(name, bad):
    a = prefill_args(**{name: bad})
    with pytest.raises(ValueError, match="shape"):
        kda.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"])


def test_prefill_rejects_misshaped_states_and_outputs():
    a = prefill_args()
    q, k, v, g, beta = (a[n] for n in ("q", "k", "v", "g", "beta"))
    with pytest.raises(ValueError, match="initial_state"):
        kda.kda_chunk_fwd(q, k, v, g, beta, initial_state=torch.zeros(B, H, D, D + 1))
    with pytest.raises(ValueError, match="shape"):
        kda.kda_chunk_fwd(q, k, v, g, beta, o=torch.zeros(B, T, H, D - 1))
    with pytest.raises(ValueError, match="final_state"):
        kda.kda_chunk_fwd(q, k, v, g, beta, final_state=torch.zeros(B + 1, H, D, D))
    cu = torch.tensor([0, 3, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="initial_state"):     # N = 2 sequences, one state
        kda.kda_chunk_fwd(q, k, v, g, beta, cu_seqlens=cu, initial_state=torch.zeros(1, H, D, D))
    q2 = torch.zeros(2, T, H, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="B == 1"):
        kda.kda_chunk_fwd(q2, q2, q2, torch.zeros(2, T, H, D), torch.zeros(2, T, H),
                          cu_seqlens=cu)


def test_prefill_rejects_host_tensors():
    a = prefill_args()
    with pytest.raises(ValueError, match="GPU"):
        kda.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"])


def test_prep_and_epilogue_shapes():
    a = prefill_args()
    args = (a["q"], a["k"], a["v"], a["g"], a["beta"])
    # the prep/epilogue tensors are checked when the structs are built
    with pytest.raises(ValueError, match="A_log"):
        kda.make_prep(dict(A_log=torch.zeros(H + 1)), H, D, torch.device("cpu"))
    with pytest.raises(ValueError, match="dt_bias"):
        kda.make_prep(dict(A_log=torch.zeros(H), dt_bias=torch.zeros(H * D)), H, D,
                      torch.device("cpu"))
    with pytest.raises(ValueError, match="weight"):
        kda.make_epilogue(dict(weight=torch.zeros(D - 1)), D, (B, T, H, D), torch.bfloat16,
                          torch.device("cpu"))
    with pytest.raises(ValueError, match="gate"):
        kda.make_epilogue(dict(gate=torch.zeros(B, T, H, D - 1, dtype=torch.bfloat16)), D,
                          (B, T, H, D), torch.bfloat16, torch.device("cpu"))
    assert args


def test_backward_rejects_misshaped_cotangents():
    a = prefill_args()
    args = (a["q"], a["k"], a["v"], a["g"], a["beta"])
    with pytest.raises(ValueError, match="grad_o"):
        kda.kda_chunk_bwd(*args, torch.zeros(B, T, H, D + 1))
    with pytest.raises(ValueError, match="grad_final_state"):
        kda.kda_chunk_bwd(*args, torch.zeros(B, T, H, D), grad_final_state=torch.zeros(H, D, D))


def test_dplr_rejects_misshaped_low_rank_vectors():
    a = prefill_args()
    bad = torch.zeros(B, T, H, D + 1, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        kda.kda_dplr_chunk_fwd(a["q"], a["k"], a["v"], bad, a["k"], a["g"])


@pytest.mark.parametrize("name", ["k", "v", "g", "beta", "slot_idx", "o"])
def test_decode_rejects_misshaped(name):
    N, S = 3, 5
    x = dict(q=torch.zeros(N, H, D, dtype=torch.bfloat16), k=torch.zeros(N, H, D, dtype=torch.bfloat16),
             v=torch.zeros(N, H, D, dtype=torch.bfloat16), g=torch.zeros(N, H, D),
             beta=torch.zeros(N, H), slot_idx=None, o=None)
    bad = dict(k=torch.zeros(N, H, D - 1, dtype=torch.bfloat16),
               v=torch.zeros(N + 1, H, D, dtype=torch.bfloat16),
               g=torch.zeros(N, H), beta=torch.zeros(N, H, 1),
               slot_idx=torch.zeros(N + 1, dtype=torch.int32), o=torch.zeros(N, H, D + 1))
    x[name] = bad[name]
    cache = torch.zeros(S, H, D, D)
    with pytest.raises(ValueError, match="shape|dimensions"):
        kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], cache,
                            slot_idx=x["slot_idx"], o=x["o"])


def test_decode_rejects_misshaped_cache():
    N = 2
    q = torch.zeros(N, H, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="state_cache"):
        kda.kda_decode_step(q, q, q, torch.zeros(N, H, D), torch.zeros(N, H),
                            torch.zeros(4, H, D, D + 1))


def test_every_entry_point_rejects_host_tensors():
    a = prefill_args()
    args = (a["q"], a["k"], a["v"], a["g"], a["beta"])
    for call in (lambda: kda.kda_chunk_fwd(*args),
                 lambda: kda.kda_chunk_bwd(*args, torch.zeros(B, T, H, D)),
                 lambda: kda.kda_dplr_chunk_fwd(a["q"], a["k"], a["v"], a["k"], a["k"], a["g"]),
                 lambda: kda.kda_decode_step(a["q"][0], a["k"][0], a["v"][0], a["g"][0],
                                             a["beta"][0], torch.zeros(T, H, D, D))):
        with pytest.raises(ValueError, match="GPU"):
            call()
