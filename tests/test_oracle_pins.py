"""Pins of the fp64 oracle to things other than itself (CPU only).

Each ``pin_*`` function checks an implementation of the per-query Parallax
output (``attend(q, rho, K, V, scale)``) or of the batched oracles against
an independent fact:

* a library routine: torch's scaled_dot_product_attention for rho = 0
  (softmax attention, with GQA and the causal mask), NumPy's weighted
  covariance for Sigma_KV, NumPy's least squares for the local linear fit;
* brute force: the d x d covariance built entry by entry in pure Python;
* closed forms: the two-key output, exact rational worked examples
  (``tests/golden/worked_examples.json``);
* invariants: key shift, value shift, identical keys, linearity in rho,
  permutation of the keys, one key, no key.

``test_mutants_are_caught`` plants plausible mistakes in copies of the
oracle (dropped correction, flipped sign, transposed covariance, uncentred
covariance, unnormalised weights, scaled probe, wrong GQA mapping, causal
off-by-one) and checks that every one fails at least one pin.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import parallax_oracle as po

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _case(rng, n, d, scale=1.0, rho_std=0.3, k_off=0.0):
    q = rng.standard_normal(d)
    K = rng.standard_normal((n, d)) + k_off
    V = rng.standard_normal((n, d))
    rho = rng.standard_normal(d) * rho_std
    return q, rho, K, V, scale


# --------------------------------------------------------------------------- pins


def pin_sdpa_rho0(attend, seed=0):
    """rho = 0 reduces to softmax attention (torch SDPA, fp64, CPU)."""
    rng = _rng(seed)
    for n, d, scale in [(1, 4, 1.0), (7, 8, 0.5), (40, 16, 0.25), (64, 64, 1 / 8)]:
        q, _, K, V, _ = _case(rng, n, d)
        got = attend(q, np.zeros(d), K, V, scale)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, None, None], torch.tensor(K)[None, None],
            torch.tensor(V)[None, None], scale=scale)[0, 0, 0].numpy()
        if not np.allclose(got, ref, rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_np_cov(sigma, seed=1):
    """Sigma_KV equals NumPy's weighted population covariance block."""
    rng = _rng(seed)
    for n, d in [(3, 2), (20, 5), (50, 16)]:
        K = rng.standard_normal((n, d))
        V = rng.standard_normal((n, d)) + 2.0
        w = rng.random(n)
        w /= w.sum()
        got = sigma(K, V, w)
        full = np.cov(np.vstack([V.T, K.T]), aweights=w, bias=True)
        ref = full[:d, d:]  # value rows, key columns
        if not np.allclose(got, ref, rtol=1e-12, atol=1e-13):
            return False
    return True


def brute_force(q, rho, K, V, scale):
    """Pure-Python evaluation: weights, means and the d x d matrix entry by entry."""
    n, dk = len(K), len(q)
    dv = len(V[0]) if n else len(q)
    if n == 0:
        return [0.0] * dv
    s = [scale * sum(q[a] * K[i][a] for a in range(dk)) for i in range(n)]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    tot = sum(e)
    w = [x / tot for x in e]
    mu_k = [sum(w[i] * K[i][a] for i in range(n)) for a in range(dk)]
    mu_v = [sum(w[i] * V[i][a] for i in range(n)) for a in range(dv)]
    sig = [[sum(w[i] * (V[i][r] - mu_v[r]) * (K[i][c] - mu_k[c]) for i in range(n))
            for c in range(dk)] for r in range(dv)]
    return [mu_v[r] - sum(sig[r][c] * rho[c] for c in range(dk)) for r in range(dv)]


def pin_brute(attend, seed=2):
    rng = _rng(seed)
    for n, d in [(1, 2), (2, 3), (5, 4), (17, 8), (33, 6)]:
        q, rho, K, V, scale = _case(rng, n, d, scale=0.7, k_off=0.3)
        got = attend(q, rho, K, V, scale)
        ref = brute_force(q.tolist(), rho.tolist(), K.tolist(), V.tolist(), scale)
        if not np.allclose(got, ref, rtol=1e-11, atol=1e-12):
            return False
    return True


def pin_two_key(attend, seed=3):
    """n = 2: out = w1 v1 + w2 v2 - w1 w2 ((k1 - k2).rho)(v1 - v2)."""
    rng = _rng(seed)
    for d in (2, 5, 16):
        q, rho, K, V, scale = _case(rng, 2, d, scale=1.3)
        s1, s2 = scale * K[0] @ q, scale * K[1] @ q
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        w2 = 1.0 - w1
        ref = w1 * V[0] + w2 * V[1] - w1 * w2 * ((K[0] - K[1]) @ rho) * (V[0] - V[1])
        if not np.allclose(attend(q, rho, K, V, scale), ref, rtol=1e-12, atol=1e-12):
            return False
    return True


def _frac(x):
    if isinstance(x[0], list):
        return np.array([_frac(r) for r in x])
    return x[0] / x[1]


def pin_worked(attend, sigma=None):
    """Exact rational worked examples (tests/golden/worked_examples.json)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)
        rho = _frac(c["rho"])
        K, V = _frac(c["K"]), _frac(c["V"])
        if not np.allclose(attend(q, rho, K, V, c["scale"]), _frac(c["out"]), rtol=0, atol=1e-14):
            return False
        if sigma is not None:
            w = np.full(len(K), 1.0 / len(K))
            if not np.allclose(sigma(K, V, w), _frac(c["sigma_kv"]), rtol=0, atol=1e-14):
                return False
    return True


def _wls_intercept(q, K, V, w):
    """Local linear regression at q: weighted least squares of v on [1, k - q]."""
    X = np.hstack([np.ones((len(K), 1)), K - q])
    sw = np.sqrt(w)[:, None]
    coef, *_ = np.linalg.lstsq(X * sw, V * sw, rcond=None)
    return coef[0]


def pin_lla(attend, seed=4):
    """With rho* = Sigma_KK^-1 (mu_k - q) the output is the local linear estimate.

    Textbook local linear regression (the estimate the pages say softmax's
    local-constant one is upgraded to) has intercept
    mu_v - Sigma_VK Sigma_KK^-1 (mu_k - q); the Parallax output with that
    probe must equal NumPy's weighted least-squares intercept, and on exactly
    linear data it must return the true value at the query while plain
    softmax (rho = 0) does not.
    """
    rng = _rng(seed)
    for n, d, scale in [(12, 3, 0.8), (40, 6, 0.5), (100, 8, 0.3)]:
        q = rng.standard_normal(d) + 1.5  # query near the edge of the key cloud
        K = rng.standard_normal((n, d))
        V = rng.standard_normal((n, d))
        s = scale * K @ q
        w = np.exp(s - s.max())
        w /= w.sum()
        mu_k = w @ K
        Skk = (K - mu_k).T @ (w[:, None] * (K - mu_k))
        rho_star = np.linalg.solve(Skk, mu_k - q)
        got = attend(q, rho_star, K, V, scale)
        if not np.allclose(got, _wls_intercept(q, K, V, w), rtol=1e-9, atol=1e-10):
            return False
        a0 = rng.standard_normal(d)
        B0 = rng.standard_normal((d, d))
        Vlin = a0 + (K - q) @ B0.T
        if not np.allclose(attend(q, rho_star, K, Vlin, scale), a0, rtol=1e-9, atol=1e-9):
            return False
        if np.allclose(attend(q, np.zeros(d), K, Vlin, scale), a0, atol=1e-3):
            return False  # softmax alone must show the boundary bias here
    return True


def pin_invariants(attend, seed=5):
    rng = _rng(seed)
    for n, d in [(9, 4), (30, 8)]:
        q, rho, K, V, scale = _case(rng, n, d, scale=0.9)
        base = attend(q, rho, K, V, scale)
        c = rng.standard_normal(d) * 3.0
        if not np.allclose(attend(q, rho, K + c, V, scale), base, rtol=1e-10, atol=1e-10):
            return False  # adding c to every key changes nothing
        cv = rng.standard_normal(d) * 3.0
        if not np.allclose(attend(q, rho, K, V + cv, scale), base + cv, rtol=1e-10, atol=1e-10):
            return False  # adding c to every value shifts the output by c
        Kid = np.repeat(K[:1], n, axis=0)
        if not np.allclose(attend(q, rho, Kid, V, scale), V.mean(axis=0), rtol=1e-12, atol=1e-12):
            return False  # identical keys: uniform weights, no correction
        r1, r2 = rng.standard_normal(d), rng.standard_normal(d)
        o0 = attend(q, np.zeros(d), K, V, scale)
        lhs = attend(q, 2.0 * r1 - 0.5 * r2, K, V, scale) - o0
        rhs = 2.0 * (attend(q, r1, K, V, scale) - o0) - 0.5 * (attend(q, r2, K, V, scale) - o0)
        if not np.allclose(lhs, rhs, rtol=1e-10, atol=1e-12):
            return False  # affine in rho
        p = rng.permutation(n)
        if not np.allclose(attend(q, rho, K[p], V[p], scale), base, rtol=1e-12, atol=1e-12):
            return False  # keys are a set
        if not np.allclose(attend(q, rho, K[:1], V[:1], scale), V[0], rtol=0, atol=0):
            return False  # one key: the value itself
        if not np.array_equal(attend(q, rho, K[:0], V[:0], scale), np.zeros(d)):
            return False  # no key: zeros
    return True


def _gqa_decode_case(seed, B=3, Hq=8, Hkv=2, d=16, S=40):
    rng = _rng(seed)
    q = rng.standard_normal((B, Hq, d))
    rho = rng.standard_normal((B, Hq, d)) * 0.2
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    lens = np.array([S, 1, 23][:B], dtype=np.int32)
    for b, n in enumerate(lens):
        k[b, :, n:] = np.nan
        v[b, :, n:] = np.nan
    return q, rho, k, v, lens


def pin_decode_sdpa(decode, seed=6):
    """Batched decode with rho = 0 and GQA equals torch SDPA (enable_gqa)."""
    q, rho, k, v, lens = _gqa_decode_case(seed)
    scale = 0.4
    got = decode(q, np.zeros_like(rho), k, v, lens, scale)
    for b, n in enumerate(lens):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[b])[None, :, None], torch.tensor(k[b, :, :n])[None],
            torch.tensor(v[b, :, :n])[None], scale=scale, enable_gqa=True)[0, :, 0].numpy()
        if not np.allclose(got[b], ref, rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_decode_matches_single(decode, seed=7):
    """Batched decode equals the single-query definition per (b, h) with h_kv = h // G."""
    q, rho, k, v, lens = _gqa_decode_case(seed)
    scale = 0.6
    got = decode(q, rho, k, v, lens, scale)
    G = q.shape[1] // k.shape[1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            n = lens[b]
            ref = brute_force(q[b, h].tolist(), rho[b, h].tolist(), k[b, h // G, :n].tolist(),
                              v[b, h // G, :n].tolist(), scale)
            if not np.allclose(got[b, h], ref, rtol=1e-10, atol=1e-11):
                return False
    return True


def _prefill_case(seed, B=2, Hq=4, Hkv=2, T=24, d=8):
    rng = _rng(seed)
    q = rng.standard_normal((B, Hq, T, d))
    rho = rng.standard_normal((B, Hq, T, d)) * 0.2
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    return q, rho, k, v, np.array([T, T], dtype=np.int32)


def pin_prefill_sdpa(prefill_full, seed=8):
    """Causal prefill with rho = 0 and GQA equals torch SDPA (is_causal, enable_gqa)."""
    q, rho, k, v, lens = _prefill_case(seed)
    scale = 0.5
    got = prefill_full(q, np.zeros_like(rho), k, v, lens, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), scale=scale, is_causal=True,
        enable_gqa=True).numpy()
    for (b, h), o in got.items():
        if not np.allclose(o, ref[b, h], rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_prefill_brute(prefill_full, seed=9):
    """Every prefill row equals the brute-force single-query output over keys 0..t."""
    q, rho, k, v, lens = _prefill_case(seed, T=12, d=4)
    scale = 0.8
    got = prefill_full(q, rho, k, v, lens, scale)
    G = q.shape[1] // k.shape[1]
    for (b, h), o in got.items():
        for t in range(q.shape[2]):
            ref = brute_force(q[b, h, t].tolist(), rho[b, h, t].tolist(),
                              k[b, h // G, : t + 1].tolist(), v[b, h // G, : t + 1].tolist(), scale)
            if not np.allclose(o[t], ref, rtol=1e-10, atol=1e-11):
                return False
    return True


# --------------------------------------------------------------------------- tests


def test_pin_sdpa_rho0():
    assert pin_sdpa_rho0(oracle.parallax_attend)


def test_pin_np_cov():
    assert pin_np_cov(oracle.sigma_kv)


def test_pin_brute_force():
    assert pin_brute(oracle.parallax_attend)


def test_pin_two_key_closed_form():
    assert pin_two_key(oracle.parallax_attend)


def test_pin_worked_examples():
    assert pin_worked(oracle.parallax_attend, oracle.sigma_kv)


def test_pin_local_linear_reduction():
    assert pin_lla(oracle.parallax_attend)


def test_pin_invariants():
    assert pin_invariants(oracle.parallax_attend)


def test_pin_decode_sdpa_gqa():
    assert pin_decode_sdpa(oracle.oracle_decode)


def test_pin_decode_per_head():
    assert pin_decode_matches_single(oracle.oracle_decode)


def test_pin_prefill_sdpa_causal_gqa():
    assert pin_prefill_sdpa(oracle.oracle_prefill_full)


def test_pin_prefill_brute():
    assert pin_prefill_brute(oracle.oracle_prefill_full)


def test_prefill_full_matches_explicit_rows():
    q, rho, k, v, lens = _prefill_case(10, T=40, d=8)
    lens = np.array([40, 29], dtype=np.int32)
    full = oracle.oracle_prefill_full(q, rho, k, v, lens, 0.7)
    rows = [(b, h, t) for b in range(2) for h in range(4) for t in (0, 1, 2, 17, 28, 29, 39)]
    ex = oracle.oracle_prefill_rows(q, rho, k, v, lens, 0.7, rows)
    for (b, h, t), o in ex.items():
        np.testing.assert_allclose(full[(b, h)][t], o, rtol=1e-12, atol=1e-12)
    assert np.array_equal(full[(1, 0)][29:], np.zeros((11, 8)))


def test_prefill_row0_is_v0():
    q, rho, k, v, lens = _prefill_case(11)
    full = oracle.oracle_prefill_full(q, rho, k, v, lens, 1.0)
    for (b, h), o in full.items():
        assert np.array_equal(o[0], v[b, h // 2, 0])


def test_decode_reads_no_padding():
    q, rho, k, v, lens = _gqa_decode_case(12)
    out = oracle.oracle_decode(q, rho, k, v, lens, 1.0)
    assert np.isfinite(out).all()


def test_torch_bf16_inputs_upcast_exactly():
    g = torch.Generator().manual_seed(0)
    K = torch.randn(10, 4, generator=g).to(torch.bfloat16)
    V = torch.randn(10, 4, generator=g).to(torch.bfloat16)
    q = torch.randn(4, generator=g).to(torch.bfloat16)
    rho = torch.randn(4, generator=g).to(torch.bfloat16)
    got = oracle.oracle_decode(q[None, None], rho[None, None], K[None, None], V[None, None],
                               torch.tensor([10]), 1.0)[0, 0]
    ref = brute_force(q.double().tolist(), rho.double().tolist(), K.double().tolist(),
                      V.double().tolist(), 1.0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@settings(max_examples=40, deadline=None)
@given(n=st.integers(0, 48), d=st.sampled_from([2, 3, 4, 8]), scale=st.floats(0.05, 3.0),
       rho_mag=st.floats(0.0, 2.0), k_off=st.floats(-4.0, 4.0), seed=st.integers(0, 2**31 - 1))
def test_hypothesis_brute_force(n, d, scale, rho_mag, k_off, seed):
    q, rho, K, V, _ = _case(_rng(seed), n, d, rho_std=rho_mag, k_off=k_off)
    got = oracle.parallax_attend(q, rho, K, V, scale)
    ref = brute_force(q.tolist(), rho.tolist(), K.tolist(), V.tolist(), scale)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-10)


# --------------------------------------------------------------- planted mistakes


def _m_drop(q, rho, K, V, scale):
    if len(K) == 0:
        return np.zeros(V.shape[1])
    w = po.softmax_weights(scale * (K @ q))
    return w @ V


def _m_sign(q, rho, K, V, scale):
    if len(K) == 0:
        return np.zeros(V.shape[1])
    w = po.softmax_weights(scale * (K @ q))
    return w @ V + po.sigma_kv(K, V, w) @ rho


def _m_transpose(q, rho, K, V, scale):
    if len(K) == 0:
        return np.zeros(V.shape[1])
    w = po.softmax_weights(scale * (K @ q))
    return w @ V - po.sigma_kv(K, V, w).T @ rho


def _sig_uncentred(K, V, w):
    return V.T @ (w[:, None] * K)


def _m_uncentred(q, rho, K, V, scale):
    if len(K) == 0:
        return np.zeros(V.shape[1])
    w = po.softmax_weights(scale * (K @ q))
    return w @ V - _sig_uncentred(K, V, w) @ rho


def _sig_unnormalised(K, V, w):
    w2 = w * len(w)  # weights summing to n
    mu_k, mu_v = w @ K, w @ V
    return (V - mu_v).T @ (w2[:, None] * (K - mu_k))


def _m_unnormalised(q, rho, K, V, scale):
    if len(K) == 0:
        return np.zeros(V.shape[1])
    w = po.softmax_weights(scale * (K @ q))
    return w @ V - _sig_unnormalised(K, V, w) @ rho


def _m_scaled_probe(q, rho, K, V, scale):
    # probe scaled like the query (scale applied to rho . k as well)
    return oracle.parallax_attend(q, scale * rho, K, V, scale)


def _m_gqa_decode(q, rho, k, v, lens, scale):
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            n = lens[b]
            out[b, h] = oracle.parallax_attend(q[b, h], rho[b, h], k[b, h % Hkv, :n],
                                               v[b, h % Hkv, :n], scale)
    return out


def _m_causal_prefill(q, rho, k, v, lens, scale):
    res = {}
    G = q.shape[1] // k.shape[1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            T = q.shape[2]
            o = np.zeros((T, v.shape[-1]))
            for t in range(T):
                o[t] = oracle.parallax_attend(q[b, h, t], rho[b, h, t], k[b, h // G, :t],
                                              v[b, h // G, :t], scale)  # excludes key t
            res[(b, h)] = o
    return res


def _attend_pins(attend, sigma=None):
    return [pin_sdpa_rho0(attend), pin_brute(attend), pin_two_key(attend),
            pin_worked(attend, sigma), pin_lla(attend), pin_invariants(attend)]


@pytest.mark.parametrize("mutant", [_m_drop, _m_sign, _m_transpose, _m_uncentred,
                                    _m_unnormalised, _m_scaled_probe])
def test_mutants_are_caught(mutant):
    assert not all(_attend_pins(mutant))


@pytest.mark.parametrize("sig", [_sig_uncentred, _sig_unnormalised,
                                 lambda K, V, w: po.sigma_kv(K, V, w).T])
def test_sigma_mutants_are_caught(sig):
    assert not pin_np_cov(sig)


def test_gqa_mutant_is_caught():
    assert not (pin_decode_sdpa(_m_gqa_decode) and pin_decode_matches_single(_m_gqa_decode))


def test_causal_mutant_is_caught():
    assert not (pin_prefill_sdpa(_m_causal_prefill) and pin_prefill_brute(_m_causal_prefill))


# ------------------------------------------------------------ chunked prefill


def _chunk_case(seed, B=2, Hq=4, Hkv=2, S=40, T=12, d=8):
    rng = _rng(seed)
    q_full = rng.standard_normal((B, Hq, S, d))
    rho_full = rng.standard_normal((B, Hq, S, d)) * 0.2
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    return q_full, rho_full, k, v


def pin_chunk_equals_prefill(chunk_rows, seed=20):
    """A chunk at offset p reproduces rows p.. of the (pinned) full causal prefill."""
    q_full, rho_full, k, v = _chunk_case(seed)
    S, T = q_full.shape[2], 12
    past = np.array([17, 5], dtype=np.int32)
    lens = np.array([T, 9], dtype=np.int32)
    qc = np.stack([q_full[b, :, past[b]:past[b] + T] for b in range(2)])
    rc = np.stack([rho_full[b, :, past[b]:past[b] + T] for b in range(2)])
    rows = [(b, h, t) for b in range(2) for h in range(4) for t in range(T)]
    got = chunk_rows(qc, rc, k, v, past, lens, 0.7, rows)
    ref = oracle.oracle_prefill_rows(q_full, rho_full, k, v, np.array([S, S]), 0.7,
                                     [(b, h, past[b] + t) for b, h, t in rows])
    for (b, h, t) in rows:
        want = np.zeros(8) if t >= lens[b] else ref[(b, h, past[b] + t)]
        if not np.allclose(got[(b, h, t)], want, rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_chunk_sdpa(chunk_full, seed=21):
    """rho = 0: torch SDPA with the shifted causal mask (GQA)."""
    q_full, rho_full, k, v = _chunk_case(seed)
    T, past = 12, np.array([20, 3], dtype=np.int32)
    qc = q_full[:, :, :T]
    got = chunk_full(qc, np.zeros_like(qc), k, v, past, np.array([T, T], dtype=np.int32), 0.5)
    for b in range(2):
        nk = past[b] + T
        mask = torch.tensor(np.arange(nk)[None, :] <= (past[b] + np.arange(T))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(qc[b])[None], torch.tensor(k[b, :, :nk])[None],
            torch.tensor(v[b, :, :nk])[None], attn_mask=mask, scale=0.5,
            enable_gqa=True)[0].numpy()
        for h in range(4):
            if not np.allclose(got[(b, h)], ref[h], rtol=1e-12, atol=1e-12):
                return False
    return True


def test_pin_chunk_equals_full_prefill():
    assert pin_chunk_equals_prefill(oracle.oracle_chunk_rows)


def test_pin_chunk_sdpa_shifted_mask():
    assert pin_chunk_sdpa(oracle.oracle_chunk_full)


def test_chunk_full_matches_rows_and_brute():
    q_full, rho_full, k, v = _chunk_case(22, S=30, T=10, d=4)
    qc, rc = q_full[:, :, :10], rho_full[:, :, :10]
    past = np.array([15, 0], dtype=np.int32)
    lens = np.array([10, 7], dtype=np.int32)
    full = oracle.oracle_chunk_full(qc, rc, k, v, past, lens, 0.9)
    rows = [(b, h, t) for b in range(2) for h in range(4) for t in range(10)]
    ex = oracle.oracle_chunk_rows(qc, rc, k, v, past, lens, 0.9, rows)
    for (b, h, t), o in ex.items():
        np.testing.assert_allclose(full[(b, h)][t], o, rtol=1e-12, atol=1e-12)
        if t < lens[b]:
            p = past[b] + t
            ref = brute_force(qc[b, h, t].tolist(), rc[b, h, t].tolist(),
                              k[b, h // 2, :p + 1].tolist(), v[b, h // 2, :p + 1].tolist(), 0.9)
            np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-11)


def test_chunk_with_no_past_is_prefill():
    q, rho, k, v, lens = _prefill_case(23)
    a = oracle.oracle_chunk_full(q, rho, k, v, np.zeros(2, dtype=np.int32), lens, 0.6)
    b = oracle.oracle_prefill_full(q, rho, k, v, lens, 0.6)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], rtol=1e-13, atol=1e-13)


def _m_chunk_offset(q, rho, k, v, past, lens, scale, rows):
    # off by one: row t sees keys 0..past + t - 1
    return oracle.oracle_chunk_rows(q, rho, k, v, np.asarray(past) - 1, lens, scale, rows)


def test_chunk_offset_mutant_is_caught():
    assert not pin_chunk_equals_prefill(_m_chunk_offset)
