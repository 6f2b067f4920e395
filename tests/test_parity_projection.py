"""GPU parity of the fused q, k, v, rho projection against the fp64 oracle.

The kernel rounds each fp32-accumulated dot product to bf16 (nearest even),
so the bar, element by element, is one bf16 unit in the last place of the
oracle's value plus the fp32 dot-product error bound d_model 2^-24
sum_c |x_c w_c| (which matters only for values near zero): where the fp32
sum and the exact value straddle a rounding boundary the two roundings
differ by one unit, and fewer than 1% of the elements may differ at all.
Cache rows outside [past, past + T) must be left untouched.
"""

import numpy as np
import pytest
import torch

import local_linear_attention_amd as pa
from oracle.projection_oracle import oracle_qkvr_projection

pytestmark = pytest.mark.gpu


def _inputs(B, T, C, H_q, H_kv, d, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((B, T, C), generator=g).to(torch.bfloat16)
    w = (torch.randn(((2 * H_q + 2 * H_kv) * d, C), generator=g) * C ** -0.5).to(torch.bfloat16)
    return x, w


def _ulp_check(got, ref, absref):
    """absref: the oracle with |x| and |w| (sum_c |x_c w_c| per element)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rb = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()  # oracle rounded to bf16
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(rb), 1e-30))) - 7)
    C = _ulp_check.d_model
    allow = ulp + C * 2.0 ** -24 * np.asarray(absref)
    diff = np.abs(got - rb)
    assert np.all(diff <= allow * 1.0001), float((diff / allow).max())
    frac = float(np.mean(diff > 0))
    assert frac < 0.01, frac
    return frac


def _random_shapes(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        H_kv = int(rng.integers(1, 4))
        H_q = H_kv * int(rng.choice([1, 2, 4]))
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 600)), 64 * int(rng.integers(1, 17)),
                    H_q, H_kv, int(rng.choice([64, 128]))))
    return out


@pytest.mark.parametrize("B,T,C,H_q,H_kv,d", [
    (2, 200, 256, 4, 2, 128),   # ragged token tile, GQA
    (1, 64, 128, 2, 2, 64),     # d = 64
    (3, 130, 512, 6, 2, 64),    # three KV heads' worth of odd sizes
    (2, 77, 192, 2, 1, 64),     # odd number of 64-wide d_model stages; a partial feature tile
    (1, 300, 64, 1, 1, 128),    # one stage; two token tiles, the second ragged
] + _random_shapes(5, 2028))
def test_projection_small(B, T, C, H_q, H_kv, d):
    print(f"[projection parity] B={B} T={T} d_model={C} Hq={H_q} Hkv={H_kv} d={d}", flush=True)
    x, w = _inputs(B, T, C, H_q, H_kv, d, seed=B * 1000 + T)
    q, k, v, r = pa.qkvr_projection(x.cuda(), w.cuda(), H_q, H_kv, d)
    torch.cuda.synchronize()
    ref = oracle_qkvr_projection(x, w, H_q, H_kv, d)
    absr = oracle_qkvr_projection(x.abs(), w.abs(), H_q, H_kv, d)
    _ulp_check.d_model = C
    fracs = [_ulp_check(t.float().cpu().numpy(), rr, ar) for t, rr, ar in zip((q, k, v, r), ref, absr)]
    print(f"   fraction one ulp off: {fracs}", flush=True)


def test_projection_into_cache_at_past_lengths():
    B, T, C, H_q, H_kv, d, S = 3, 48, 128, 4, 2, 128, 160
    x, w = _inputs(B, T, C, H_q, H_kv, d, seed=77)
    past = torch.tensor([0, 100, 150], dtype=torch.int32)  # the last overflows S_max
    kc = torch.full((B, H_kv, S, d), float("nan"), dtype=torch.bfloat16).cuda()
    vc = kc.clone()
    q, kc, vc, r = pa.qkvr_projection(x.cuda(), w.cuda(), H_q, H_kv, d, k_cache=kc, v_cache=vc,
                                      past_lens=past.cuda())
    torch.cuda.synchronize()
    _, kr, vr, _ = oracle_qkvr_projection(x, w, H_q, H_kv, d)
    _, ka, va, _ = oracle_qkvr_projection(x.abs(), w.abs(), H_q, H_kv, d)
    _ulp_check.d_model = C
    kc, vc = kc.float().cpu().numpy(), vc.float().cpu().numpy()
    for b, p in enumerate(past.tolist()):
        n = min(T, S - p)
        _ulp_check(kc[b, :, p:p + n], kr[b, :, :n], ka[b, :, :n])
        _ulp_check(vc[b, :, p:p + n], vr[b, :, :n], va[b, :, :n])
        rest = np.ones(S, dtype=bool)
        rest[p:p + n] = False
        assert np.all(np.isnan(kc[b][:, rest])) and np.all(np.isnan(vc[b][:, rest]))


def test_projection_full_size_sampled_tokens():
    # causal-prefill shapes (B=4, T=4096, H_q=16, H_kv=8, d=128) with
    # d_model = H_q d = 2048; the oracle on 512 seeded tokens
    B, T, C, H_q, H_kv, d = 4, 4096, 2048, 16, 8, 128
    print(f"[projection parity] full size B={B} T={T} d_model={C}", flush=True)
    x, w = _inputs(B, T, C, H_q, H_kv, d, seed=5)
    q, k, v, r = pa.qkvr_projection(x.cuda(), w.cuda(), H_q, H_kv, d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    tok = rng.choice(B * T, size=512, replace=False)
    bs, ts = tok // T, tok % T
    xs = x.reshape(B * T, C)[torch.from_numpy(tok)].reshape(1, 512, C)
    ref = oracle_qkvr_projection(xs, w, H_q, H_kv, d)
    absr = oracle_qkvr_projection(xs.abs(), w.abs(), H_q, H_kv, d)
    _ulp_check.d_model = C
    for t, rr, ar in zip((q, k, v, r), ref, absr):
        got = t.float().cpu().numpy()[bs, :, ts]  # [512, H, d]
        _ulp_check(got, rr[0].transpose(1, 0, 2), ar[0].transpose(1, 0, 2))
