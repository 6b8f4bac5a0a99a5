"""Pins for the fp64 oracle: each test checks the oracle against something
other than itself -- a hand-worked example, a closed form, an invariant the
method must satisfy, a special case that is a textbook algorithm, or brute
force on tiny inputs -- so that a dropped term, a wrong sign or index, or a
transposed operand anywhere in it fails at least one of them.

Method source: GeekNews summary of Kimi Linear (es.news.hada.io topic 31936),
sections "De la atencion lineal a Gated DeltaNet", "Control fino de memoria en
Kimi Delta Attention" and "Algoritmo paralelo por chunks".
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def rand_chain(rng, T, dk, dv, g_lo=0.001, g_hi=0.1, normalize=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if normalize:
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    g = -rng.uniform(g_lo, g_hi, (T, dk))
    # round to float32 once: every form below sees the same values
    return [x.astype(np.float32).astype(np.float64) for x in (q, k, v, g, beta)]


def c_chain(q, k, v, g, beta, scale, S0=None, drop_erase=False):
    """Run the C oracle on one chain (B = H = 1)."""
    s0 = None if S0 is None else S0[None, None]
    o, S = oracle.kda_fwd(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None],
                          beta[None, :, None], scale, S0=s0, drop_erase=drop_erase)
    return o[0, :, 0], S[0, 0]


def close(a, b, tol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    return float(np.max(np.abs(a - b))) <= tol * scale if a.size else True


# ---------------------------------------------------------------- hand-worked

@pytest.mark.parametrize("case", ["scalar", "two_channel"])
def test_hand_examples(case):
    ex = json.load(open(GOLD))[case]
    q = np.array(ex["q"], dtype=np.float64).reshape(len(ex["beta"]), -1)
    k = np.array(ex["k"], dtype=np.float64).reshape(q.shape)
    v = np.array(ex["v"], dtype=np.float64).reshape(q.shape[0], -1)
    g = np.log(np.array(ex["alpha"], dtype=np.float64)).reshape(q.shape)
    beta = np.array(ex["beta"], dtype=np.float64)
    S0 = np.array(ex["S0"], dtype=np.float64)
    o, S = c_chain(q, k, v, g, beta, 1.0, S0)
    assert np.allclose(o.reshape(-1), np.array(ex["o"]).reshape(-1), atol=1e-6, rtol=0)
    assert np.allclose(S, np.array(ex["S_final"]), atol=1e-6, rtol=0)


# ---------------------------------------------------------------- P0 brute force

@pytest.mark.parametrize("T,dk,dv", [(1, 4, 4), (7, 3, 5), (40, 8, 6), (33, 16, 16)])
def test_p0_bruteforce_matches(T, dk, dv):
    rng = np.random.default_rng(10 + T + dk)
    q, k, v, g, beta = rand_chain(rng, T, dk, dv, 0.0, 1.0)
    S0 = rng.standard_normal((dk, dv))
    scale = dk ** -0.5
    ob, Sb = oracle.bruteforce_np(q, k, v, g, beta, scale, S0)
    oc, Sc = c_chain(q, k, v, g, beta, scale, S0)
    on, Sn = oracle.recurrence_np(q, k, v, g, beta, scale, S0)
    assert close(oc, ob) and close(Sc, Sb)
    assert close(on, ob) and close(Sn, Sb)


# ---------------------------------------------------------------- P1 chunked form

@pytest.mark.parametrize("T,chunk", [(37, 1), (37, 3), (37, 5), (128, 16), (130, 64), (50, 50),
                                     (64, 64), (200, 16)])
def test_p1_chunked_form(T, chunk):
    rng = np.random.default_rng(100 + T + chunk)
    dk, dv = 16, 12
    q, k, v, g, beta = rand_chain(rng, T, dk, dv)
    S0 = 0.3 * rng.standard_normal((dk, dv))
    scale = dk ** -0.5
    oc, Sc = c_chain(q, k, v, g, beta, scale, S0)
    ok, Sk = oracle.chunked_np(q, k, v, g, beta, scale, S0, chunk=chunk)
    assert close(ok, oc, 1e-11) and close(Sk, Sc, 1e-11)


def test_forward_substitution_inverse():
    rng = np.random.default_rng(5)
    L = np.eye(20) + np.tril(rng.standard_normal((20, 20)) * 0.3, -1)
    X = oracle.forward_substitution_inverse(L)
    assert np.allclose(X @ L, np.eye(20), atol=1e-12)
    assert np.allclose(np.triu(X, 1), 0)


# ---------------------------------------------------------------- invariants

def test_i1_no_gate_no_write_keeps_state():
    """alpha = 1, beta = 0: the state never changes and o_t = scale S0^T q_t."""
    rng = np.random.default_rng(1)
    T, dk, dv = 25, 8, 8
    q, k, v, _, _ = rand_chain(rng, T, dk, dv)
    S0 = rng.standard_normal((dk, dv))
    o, S = c_chain(q, k, v, np.zeros((T, dk)), np.zeros(T), 0.5, S0)
    assert np.array_equal(S, S0)
    assert close(o, 0.5 * q @ S0)


def test_i2_linear_attention():
    """alpha = 1 and the k k^T erase term dropped: causal linear attention."""
    rng = np.random.default_rng(2)
    T, dk, dv = 30, 8, 6
    q, k, v, _, beta = rand_chain(rng, T, dk, dv)
    S0 = rng.standard_normal((dk, dv))
    scale = 0.7
    o, S = c_chain(q, k, v, np.zeros((T, dk)), beta, scale, S0, drop_erase=True)
    oe, Se = oracle.linear_attention_closed_form(q, k, v, beta, scale, S0)
    assert close(o, oe) and close(S, Se)


def test_i3_scalar_gate_is_gated_deltanet():
    """alpha equal across channels: scalar-gated DeltaNet (Diag(a) commutes)."""
    rng = np.random.default_rng(3)
    T, dk, dv = 40, 8, 5
    q, k, v, _, beta = rand_chain(rng, T, dk, dv)
    gs = -rng.uniform(0.0, 0.5, T).astype(np.float32).astype(np.float64)
    g = np.repeat(gs[:, None], dk, axis=1)
    S0 = rng.standard_normal((dk, dv))
    o, S = c_chain(q, k, v, g, beta, 0.9, S0)
    oe, Se = oracle.scalar_gated_deltanet_np(q, k, v, np.exp(gs), beta, 0.9, S0)
    assert close(o, oe) and close(S, Se)


def test_i4_orthonormal_keys_exact_retrieval():
    """beta = 1, alpha = 1, S0 = 0, orthonormal keys: S^T k_j = v_j exactly,
    querying with k_j returns scale v_j, and rewriting key j replaces v_j."""
    rng = np.random.default_rng(4)
    dk, dv, n = 16, 7, 10
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :n].T.copy()
    vals = rng.standard_normal((n, dv))
    vnew = rng.standard_normal(dv)
    # write all n keys, rewrite key 3 with vnew, then read key 3 and key 5
    k = np.vstack([keys, keys[3], np.zeros(dk), np.zeros(dk)])
    v = np.vstack([vals, vnew, np.zeros(dv), np.zeros(dv)])
    q = np.vstack([keys, keys[3], keys[3], keys[5]])
    T = k.shape[0]
    beta = np.r_[np.ones(n + 1), 0.0, 0.0]
    k32 = k.astype(np.float32).astype(np.float64)
    q32 = q.astype(np.float32).astype(np.float64)
    v32 = v.astype(np.float32).astype(np.float64)
    o, S = c_chain(q32, k32, v32, np.zeros((T, dk)), beta, 2.0)
    # float32 keys are orthonormal to ~1e-7
    for j in range(n):
        want = vnew if j == 3 else v32[j]
        assert np.allclose(S.T @ k32[j], want, atol=1e-5)
        assert np.allclose(o[j], 2.0 * v32[j], atol=1e-5)
    assert np.allclose(o[n + 1], 2.0 * v32[n], atol=1e-5)
    assert np.allclose(o[n + 2], 2.0 * v32[5], atol=1e-5)


def test_i5_basis_keys_per_channel_decay():
    """Keys e_j, beta = 1, arbitrary per-channel alpha: row j of the final
    state is v_j times the product of channel j's later gates (rows are key
    channels, and each channel decays on its own)."""
    rng = np.random.default_rng(5)
    dk, dv = 6, 4
    order = [2, 0, 5, 1, 4, 3]
    T = len(order) + 3
    k = np.zeros((T, dk))
    for t, j in enumerate(order):
        k[t, j] = 1.0
    v = rng.standard_normal((T, dv)).astype(np.float32).astype(np.float64)
    g = (-rng.uniform(0.0, 1.0, (T, dk))).astype(np.float32).astype(np.float64)
    beta = np.r_[np.ones(len(order)), np.zeros(3)]
    o, S = c_chain(np.zeros((T, dk)), k, v, g, beta, 1.0)
    for t, j in enumerate(order):
        decay = np.exp(g[t + 1:, j].sum())
        assert np.allclose(S[j], decay * v[t], rtol=1e-12, atol=1e-14)


def test_i6_single_token_and_scale():
    """T = 1 from zero state: o = scale beta (q.k) v."""
    rng = np.random.default_rng(6)
    dk, dv = 9, 4
    q, k, v, g, beta = rand_chain(rng, 1, dk, dv, 0.0, 2.0)
    o, S = c_chain(q, k, v, g, beta, 0.37)
    assert close(o[0], 0.37 * beta[0] * (q[0] @ k[0]) * v[0])
    assert close(S, beta[0] * np.outer(k[0], v[0]))


def test_i7_linearity_in_v_and_state():
    rng = np.random.default_rng(7)
    T, dk, dv = 20, 8, 6
    q, k, v1, g, beta = rand_chain(rng, T, dk, dv)
    v2 = rng.standard_normal((T, dv)).astype(np.float32).astype(np.float64)
    S1 = rng.standard_normal((dk, dv))
    S2 = rng.standard_normal((dk, dv))
    a, b = 0.75, -1.25
    o1, F1 = c_chain(q, k, v1, g, beta, 1.0, S1)
    o2, F2 = c_chain(q, k, v2, g, beta, 1.0, S2)
    vc = (a * v1 + b * v2).astype(np.float32).astype(np.float64)
    # use exactly representable combination by checking against the fp64 combination
    oc, Fc = oracle.recurrence_np(q, k, a * v1 + b * v2, g, beta, 1.0, a * S1 + b * S2)
    assert close(oc, a * o1 + b * o2, 1e-11) and close(Fc, a * F1 + b * F2, 1e-11)
    del vc


def test_i8_split_resume_and_varlen_and_decode():
    rng = np.random.default_rng(8)
    H, dk, dv = 3, 8, 8
    lens = [17, 1, 40, 0, 23]
    T = sum(lens)
    q = rng.standard_normal((1, T, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((1, T, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, H, dv))
    g = -rng.uniform(0.001, 0.1, (1, T, H, dk))
    beta = rng.uniform(0.1, 0.9, (1, T, H))
    S0 = rng.standard_normal((len(lens), H, dk, dv)) * 0.1
    cu = np.r_[0, np.cumsum(lens)].astype(np.int32)
    o, S = oracle.kda_fwd(q, k, v, g, beta, 0.3, S0=S0, cu_seqlens=cu)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        on, Sn = oracle.kda_fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], 0.3,
                                S0=S0[n:n + 1])
        assert np.array_equal(on, o[:, a:b]) and np.array_equal(Sn[0], S[n])
        if L >= 2:  # split-and-resume
            m = L // 2
            o1, S1 = oracle.kda_fwd(q[:, a:a + m], k[:, a:a + m], v[:, a:a + m], g[:, a:a + m],
                                    beta[:, a:a + m], 0.3, S0=S0[n:n + 1])
            o2, S2 = oracle.kda_fwd(q[:, a + m:b], k[:, a + m:b], v[:, a + m:b], g[:, a + m:b],
                                    beta[:, a + m:b], 0.3, S0=S1)
            assert close(np.concatenate([o1, o2], 1), o[:, a:b]) and close(S2[0], S[n])
        # decode x L from the same initial state == prefill
        st = np.ascontiguousarray(S0[n:n + 1].copy())
        for t in range(a, b):
            od = oracle.kda_decode_step(q[0, t:t + 1], k[0, t:t + 1], v[0, t:t + 1],
                                        g[0, t:t + 1], beta[0, t:t + 1], 0.3, st)
            assert close(od[0], o[0, t])
        assert close(st[0], S[n])


def test_decode_slot_indirection():
    rng = np.random.default_rng(9)
    N, H, dk, dv, slots = 3, 2, 4, 5, 6
    st = rng.standard_normal((slots, H, dk, dv))
    ref = st.copy()
    q = rng.standard_normal((N, H, dk)); k = rng.standard_normal((N, H, dk))
    v = rng.standard_normal((N, H, dv)); g = -rng.uniform(0, 1, (N, H, dk))
    b = rng.uniform(0, 1, (N, H))
    idx = np.array([4, 0, 99], dtype=np.int32)  # 99 is out of range: skipped
    o = oracle.kda_decode_step(q, k, v, g, b, 1.0, st, slot_idx=idx)
    for n, s in enumerate(idx):
        if s >= slots:
            assert np.all(o[n] == 0)
            continue
        for h in range(H):
            S1 = ref[s, h].copy()
            on, Sn = oracle.recurrence_np(q[n, h][None].astype(np.float32), k[n, h][None].astype(np.float32),
                                          v[n, h][None].astype(np.float32), g[n, h][None].astype(np.float32),
                                          b[n, h:h + 1].astype(np.float32), 1.0, S1)
            assert close(on[0], o[n, h]) and close(Sn, st[s, h])
    untouched = [1, 2, 3, 5]
    assert np.array_equal(st[untouched], ref[untouched])


# ---------------------------------------------------------------- sensitivity

def _mutant(q, k, v, g, beta, scale, S0, kind):
    """The recurrence with one planted mistake (CPU only)."""
    dk, dv = q.shape[1], v.shape[1]
    S = S0.copy()
    o = np.zeros((q.shape[0], dv))
    for t in range(q.shape[0]):
        a = np.exp(g[t])
        if kind == "erase_then_decay":
            S = S - beta[t] * np.outer(k[t], k[t] @ S)
            S = a[:, None] * S + beta[t] * np.outer(k[t], v[t])
        else:
            if kind == "decay_columns":
                S = S * a[None, :dv] if dk == dv else S
            else:
                S = a[:, None] * S
            u = S.T @ k[t]
            if kind == "sign":
                u = -u
            S = S + beta[t] * np.outer(k[t], v[t] - u)
            if kind == "output_before_update":
                o[t] = scale * ((S - beta[t] * np.outer(k[t], v[t] - u)).T @ q[t])
                continue
        o[t] = scale * (S.T @ q[t]) if kind != "transposed_read" else scale * (S @ q[t][:dv])
    return o, S


@pytest.mark.parametrize("kind", ["erase_then_decay", "decay_columns", "sign",
                                  "output_before_update", "transposed_read"])
def test_pins_detect_planted_mistakes(kind):
    """Each planted mistake must disagree with the brute-force pin by far more
    than the oracle does."""
    rng = np.random.default_rng(11)
    T, dk, dv = 12, 6, 6
    q, k, v, g, beta = rand_chain(rng, T, dk, dv, 0.05, 1.0)
    S0 = rng.standard_normal((dk, dv))
    ob, Sb = oracle.bruteforce_np(q, k, v, g, beta, 0.5, S0)
    om, Sm = _mutant(q, k, v, g, beta, 0.5, S0, kind)
    assert np.max(np.abs(om - ob)) > 1e-3


def test_chunk_terms_against_direct_sums():
    """The per-chunk quantities of the chunked form, against sums written out
    entry by entry with the decay between tokens as a product of per-token
    gates (no division), on a tiny chunk: A_ri = beta_r sum_c k_r k_i
    prod_{i<j<=r} alpha_j, M_ri likewise with q_r and i <= r, T (I + A) = I,
    KE = k * prod_{j>i} alpha_j, Gn = prod_j alpha_j."""
    rng = np.random.default_rng(77)
    n, dk = 6, 3
    Q, K = rng.standard_normal((n, dk)), rng.standard_normal((n, dk))
    g = -rng.uniform(0.05, 2.0, (n, dk))
    b = rng.uniform(0.1, 1.0, n)
    t = oracle.chunk_terms_np(Q, K, g, b)
    al = np.exp(g)
    A = np.zeros((n, n))
    M = np.zeros((n, n))
    for r in range(n):
        for i in range(r + 1):
            for c in range(dk):
                p = 1.0
                for j in range(i + 1, r + 1):
                    p *= al[j, c]
                M[r, i] += Q[r, c] * K[i, c] * p
                if i < r:
                    A[r, i] += b[r] * K[r, c] * K[i, c] * p
    assert np.allclose(t["A"], A, rtol=1e-12, atol=1e-14)
    assert np.allclose(t["M"], M, rtol=1e-12, atol=1e-14)
    assert np.allclose(t["T"] @ (np.eye(n) + A), np.eye(n), atol=1e-12)
    KE = K * np.array([[np.prod(al[i + 1:, c]) for c in range(dk)] for i in range(n)])
    assert np.allclose(t["KE"], KE, rtol=1e-12)
    assert np.allclose(t["Gn"], np.prod(al, axis=0), rtol=1e-12)
    assert np.allclose(t["KG"], K * np.cumprod(al, axis=0), rtol=1e-12)
    assert np.allclose(t["QG"], Q * np.cumprod(al, axis=0), rtol=1e-12)
