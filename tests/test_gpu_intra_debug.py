"""The intra-chunk kernel's own results (include/kda_debug.h), per chunk and
head, against the oracle's per-chunk quantities of the chunked form
(oracle.chunk_terms_np): the decayed key and query tiles, the decayed keys
seen from the chunk end, the k.k^T Gram, the UT transform T = (I + A)^-1, the
q.k^T Gram and exp(G_n) -- for fp32 inputs each one itself, for bf16 inputs
the folded products the fp16 records carry (the decayed keys times
T diag(beta), and M T diag(beta)).

Bounds (max |gpu - ref| over max |ref| of each quantity, the latter floored
at 1e-6): 2e-5 for fp32
inputs (fp32 arithmetic throughout); 4e-3 for bf16 inputs, whose records hold
fp16 values (relative rounding 2^-11) formed from fp16 matrix-core operands."""
import numpy as np
import pytest
import torch

import linear_attention_sequence_chunkwise_amd as kda
import oracle
from kda_testlib import make_prefill, np32

pytestmark = pytest.mark.gpu

BOUND = {torch.float32: 2e-5, torch.bfloat16: 4e-3}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rel(x, ref):
    # (a floor on the scale: under strong decay exp(G_n) is far below fp32's
    # range, so the kernel's 0 is exact to within that floor)
    m = max(float(np.max(np.abs(ref))), 1e-6)
    return float(np.max(np.abs(np.asarray(x, np.float64) - ref))) / m


def check(d, chunk):
    dtype = d["q"].dtype
    out = kda.kda_debug_chunk_intra(d["q"], d["k"], d["g"], d["beta"], chunk=chunk)
    torch.cuda.synchronize()
    got = {n: t.cpu().numpy() for n, t in out.items()}
    q, k, g, beta = (np32(d[n]) for n in ("q", "k", "g", "beta"))
    B, T, H, D = q.shape
    C = chunk
    worst = {}
    for b in range(B):
        for c in range((T + C - 1) // C):
            r0, r1 = c * C, min(T, (c + 1) * C)
            n = r1 - r0
            for h in range(H):
                t = oracle.chunk_terms_np(q[b, r0:r1, h].astype(np.float64),
                                          k[b, r0:r1, h].astype(np.float64),
                                          g[b, r0:r1, h].astype(np.float64),
                                          beta[b, r0:r1, h].astype(np.float64))
                bt = beta[b, r0:r1, h].astype(np.float64)
                pad = lambda x, rows=C, cols=None: np.pad(x, ((0, rows - x.shape[0]),
                                                              (0, (cols or x.shape[1]) - x.shape[1])))
                Tb = t["T"] * bt[None, :]
                ref = dict(KG=pad(t["KG"]), QG=pad(t["QG"]), GN=t["Gn"],
                           T=np.eye(C) + pad(t["T"] - np.eye(n), C, C),
                           P=pad(t["A"] / bt[:, None], C, C))
                if dtype == torch.float32:
                    ref.update(KP=pad(t["KE"]).T, TB=pad(Tb, C, C), MM=pad(t["M"], C, C))
                else:
                    ref.update(KP=np.pad(t["KE"].T @ Tb, ((0, 0), (0, C - n))),
                               TB=np.zeros((C, C)), MM=pad(t["M"] @ Tb, C, C))
                for name, r in ref.items():
                    e = rel(got[name][b, c, h], r)
                    worst[name] = max(worst.get(name, 0.0), e)
    print({kk: "%.1e" % v for kk, v in worst.items()}, flush=True)
    bad = {kk: v for kk, v in worst.items() if v > BOUND[dtype]}
    assert not bad, bad


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("chunk", [16, 64])
def test_intra_quantities(dtype, D, chunk):
    """Two rows, two full chunks and a ragged third, three heads."""
    d = make_prefill(600 + D + chunk, 2, 2 * chunk + 5, 3, D, dtype)
    check(d, chunk)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_intra_quantities_strong_and_mixed_decay(dtype):
    """Gates -U(0.1, 5) (every sub-block on the exact diagonal path) and gates
    straddling the exact-path threshold, d = 128, chunk 64."""
    check(make_prefill(610, 1, 130, 2, 128, dtype, g_range=(0.1, 5.0)), 64)
    gr = (0.001, 1.0) if dtype == torch.bfloat16 else (1.5, 3.5)
    check(make_prefill(611, 1, 130, 2, 128, dtype, g_range=gr), 64)
