"""GPU parity of the causal-prefill backward (and the training forward's saved
tensors) against the fp64 oracle, through the C ABI.

Error measure: per row of each gradient (a query row of dq / drho, a key
row of dk / dv), max |gpu - oracle| / max |oracle|, maximised over rows; bar
2e-3. Rows past the sequence (query rows t >= n, keys j >= n) must be exactly
zero. A row can also be zero for a mathematical reason (row 0 sees one key,
so its dq and drho vanish), where the GPU returns rounding noise; each row's
denominator is therefore floored at 1e-3 of the largest row of that tensor.
"""

import numpy as np
import pytest
import torch

import local_linear_attention_amd as pa
import oracle
from oracle import parallax_grad_oracle as go
from workloads import WORKLOADS, make_prefill_inputs, replace_shape

TOL = 2e-3
pytestmark = pytest.mark.gpu


def rel_err(got, ref, live=None):
    """live: boolean per row (flattened leading dims); rows not live must be 0."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    if live is None:
        live = np.abs(ref).max(axis=-1) > 0
    live = np.asarray(live).reshape(-1)
    assert np.all(got[~live] == 0), "rows past the sequence must be exactly zero"
    if not live.any():
        return 0.0
    den = np.abs(ref[live]).max(axis=-1)
    if den.max() == 0:  # an identically zero gradient (dq at scale 0)
        assert np.all(got[live] == 0)
        return 0.0
    den = np.maximum(den, 1e-3 * den.max())
    return float((np.abs(got[live] - ref[live]).max(axis=-1) / den).max())


def _live(lens, H, L):
    """[B, H, L] mask of positions below each sequence's length."""
    lens = np.asarray(lens)
    return np.arange(L)[None, None, :] < lens[:, None, None] + np.zeros((1, H, 1), dtype=int)


def _case(w, seed, lens=None, S_max=None, k_offset=0.0):
    inp = make_prefill_inputs(w, seed=seed, seq_lens=lens, S_max=S_max, nan_pad=False)
    if k_offset:
        inp["k"] = (inp["k"].float() + k_offset).to(inp["k"].dtype)
    g = torch.Generator().manual_seed(seed + 7)
    dout = torch.randn((w.B, w.H_q, w.T, w.d), generator=g, dtype=torch.float32)
    return inp, dout


def _run(inp, dout):
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out, mu, stats = pa.prefill_train(dev["q"], dev["rho"], dev["k"], dev["v"], dev["seq_lens"],
                                      dev["scale"])
    dq, drho, dk, dv = pa.prefill_backward(dev["q"], dev["rho"], dev["k"], dev["v"],
                                           dev["seq_lens"], out, mu, stats, dout.cuda(),
                                           dev["scale"])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (out, mu, stats, dq, drho, dk, dv)]


def check(w, *, seed=0, lens=None, S_max=None, k_offset=0.0, kv_heads=None):
    print(f"[backward parity] B={w.B} T={w.T} Hq={w.H_q} Hkv={w.H_kv} d={w.d} lens={lens} "
          f"S_max={S_max} koff={k_offset} seed={seed} kv_heads={kv_heads}", flush=True)
    inp, dout = _case(w, seed, lens, S_max, k_offset)
    out, mu, stats, dq, drho, dk, dv = _run(inp, dout)
    assert all(np.isfinite(x).all() for x in (out, mu, stats, dq, drho, dk, dv))
    ref = go.oracle_prefill_grads(inp["q"], inp["rho"], inp["k"], inp["v"], inp["seq_lens"],
                                  dout, inp["scale"], kv_heads=kv_heads)
    G = w.H_q // w.H_kv
    lens_np = inp["seq_lens"].numpy()
    lq = _live(lens_np, w.H_q, w.T)
    lk = _live(lens_np, w.H_kv, dk.shape[2])
    if kv_heads is None:
        errs = [rel_err(x, r, m) for x, r, m in zip((dq, drho, dk, dv), ref, (lq, lq, lk, lk))]
    else:
        errs = [0.0] * 4
        for b, hk in kv_heads:
            hs = slice(G * hk, G * hk + G)
            errs = [max(e, rel_err(x, r, m)) for e, x, r, m in zip(
                errs, (dq[b, hs], drho[b, hs], dk[b, hk], dv[b, hk]),
                (ref[0][b, hs], ref[1][b, hs], ref[2][b, hk], ref[3][b, hk]),
                (lq[b, hs], lq[b, hs], lk[b, hk], lk[b, hk]))]
    print(f"   max rel err dq {errs[0]:.2e} drho {errs[1]:.2e} dk {errs[2]:.2e} dv {errs[3]:.2e}",
          flush=True)
    assert max(errs) < TOL, errs
    return inp, out, mu, stats


def test_small_ragged():
    w = replace_shape(WORKLOADS[5], B=2, T=300, H_q=4, H_kv=2)
    check(w, seed=1, lens=[300, 173], S_max=320)


def test_head_dim_64():
    w = replace_shape(WORKLOADS[5], B=1, T=200, H_q=2, H_kv=1, d=64, q_std=64 ** -0.25,
                      k_std=64 ** -0.25)
    check(w, seed=2)


@pytest.mark.parametrize("H_q,H_kv", [(2, 2), (8, 2), (8, 1)])
def test_group_sizes(H_q, H_kv):
    w = replace_shape(WORKLOADS[5], B=1, T=150, H_q=H_q, H_kv=H_kv)
    check(w, seed=3 + H_q)


def test_edge_lengths():
    w = replace_shape(WORKLOADS[5], B=4, T=160, H_q=2, H_kv=1)
    check(w, seed=4, lens=[0, 1, 33, 128], S_max=200)


@pytest.mark.parametrize("scale", [-128 ** -0.5, 0.0])
def test_negative_and_zero_scale(scale):
    w = replace_shape(WORKLOADS[5], B=2, T=200, H_q=4, H_kv=2, scale=scale)
    check(w, seed=9, lens=[200, 141])


def _random_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        G = int(rng.choice([1, 2, 4, 8]))
        H_kv = int(rng.integers(1, 3))
        d = int(rng.choice([64, 128]))
        T = int(rng.integers(1, 260))
        S = T + int(rng.integers(0, 2)) * int(rng.integers(1, 90))
        B = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(0, T + 1, B)]
        cases.append((B, G, H_kv, d, T, S, lens))
    return cases


@pytest.mark.parametrize("case", _random_cases(6, 2027), ids=lambda c: f"B{c[0]}G{c[1]}Hkv{c[2]}d{c[3]}T{c[4]}S{c[5]}")
def test_random_shapes(case):
    """Seeded random shapes: group sizes, head dims, lengths (zero included),
    T not a multiple of any block, and caches longer than T."""
    B, G, H_kv, d, T, S, lens = case
    w = replace_shape(WORKLOADS[5], B=B, T=T, H_q=G * H_kv, H_kv=H_kv, d=d,
                      q_std=d ** -0.25, k_std=d ** -0.25)
    check(w, seed=11, lens=lens, S_max=S)


def test_large_key_offset():
    w = replace_shape(WORKLOADS[5], B=1, T=256, H_q=2, H_kv=1)
    check(w, seed=5, k_offset=4.0)


def test_training_forward_outputs():
    w = replace_shape(WORKLOADS[5], B=2, T=300, H_q=4, H_kv=2)
    inp, dout = _case(w, 6, lens=[300, 211])
    out, mu, stats, *_ = _run(inp, dout)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    plain = pa.prefill(dev["q"], dev["rho"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"])
    torch.cuda.synchronize()
    # The training forward contracts split bf16 weights, the inference prefill
    # fp16 ones: both outputs within the bar of the oracle, the training one
    # to the split weights' precision.
    ref = oracle.oracle_prefill_full(inp["q"], inp["rho"], inp["k"], inp["v"], inp["seq_lens"],
                                     inp["scale"])
    plain = plain.cpu().numpy()
    for (b, h), r in ref.items():
        n = int(inp["seq_lens"][b])
        den = np.abs(r[:n]).max(axis=-1)
        assert (np.abs(out[b, h, :n] - r[:n]).max(axis=-1) / den).max() < 1e-4
        assert (np.abs(plain[b, h, :n] - r[:n]).max(axis=-1) / den).max() < TOL
    q, k, v, rho = (inp[x].double().numpy() for x in ("q", "k", "v", "rho"))
    lens = inp["seq_lens"].tolist()
    G = w.H_q // w.H_kv
    for b in range(w.B):
        for h in range(w.H_q):
            n = lens[b]
            K, V = k[b, h // G, :n], v[b, h // G, :n]
            S = inp["scale"] * q[b, h, :n] @ K.T
            S[np.triu_indices(n, 1)] = -np.inf
            lse2 = (S.max(1) + np.log(np.exp(S - S.max(1, keepdims=True)).sum(1))) / np.log(2)
            W = np.exp(S - S.max(1, keepdims=True))
            W /= W.sum(1, keepdims=True)
            R = rho[b, h, :n] @ K.T
            c0 = R[:, 0]
            assert rel_err(mu[b, h, :n], W @ V) < 1e-4
            assert np.allclose(stats[b, h, :n, 0], lse2, rtol=1e-5, atol=1e-4)
            assert np.allclose(stats[b, h, :n, 1], c0, rtol=1e-5, atol=1e-5)
            assert np.allclose(stats[b, h, :n, 2], (W * R).sum(1) - c0, rtol=1e-4, atol=1e-5)
            assert np.all(stats[b, h, n:] == 0) and np.all(mu[b, h, n:] == 0)


def test_deterministic_bitwise():
    w = replace_shape(WORKLOADS[5], B=1, T=384, H_q=4, H_kv=2)
    inp, dout = _case(w, 8)
    a = _run(inp, dout)
    b = _run(inp, dout)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_workload5_full_size_sampled_heads():
    # the full causal-prefill workload on the GPU; the oracle on two KV heads
    # (and their query heads), every row and key of each
    w = WORKLOADS[5]
    check(w, seed=w.seed, kv_heads=[(0, 0), (3, 7)])
