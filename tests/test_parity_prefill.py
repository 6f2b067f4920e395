"""GPU parity of parallax_prefill (causal) against the fp64 oracle (through the C ABI).

Error measure: per output row (b, h, t), max_i |gpu_i - oracle_i| / max_i |oracle_i|,
maximised over rows; bar 2e-3 (bf16 inputs, fp32 accumulation). Rows at or
past a sequence's length must be exactly zero.
"""

import numpy as np
import pytest
import torch

import local_linear_attention_amd as pa
import oracle
from workloads import WORKLOADS, make_prefill_inputs, replace_shape

TOL = 2e-3
pytestmark = pytest.mark.gpu


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    zero = den == 0
    assert np.all(num[zero] == 0), "rows with no keys must be exactly zero"
    if np.all(zero):
        return 0.0
    return float((num[~zero] / den[~zero]).max())


def to_dev(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def run_prefill(dev):
    out = pa.prefill(dev["q"], dev["rho"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(w, *, seed=0, seq_lens=None, S_max=None, **kw):
    print(f"[prefill parity] B={w.B} T={w.T} Hq={w.H_q} Hkv={w.H_kv} d={w.d} seed={seed} "
          f"lens={seq_lens} S_max={S_max} {kw}", flush=True)
    cpu = make_prefill_inputs(w, seed=seed, seq_lens=seq_lens, S_max=S_max, **kw)
    ref = oracle.oracle_prefill_full(cpu["q"], cpu["rho"], cpu["k"], cpu["v"], cpu["seq_lens"],
                                     cpu["scale"])
    got = run_prefill(to_dev(cpu))
    assert np.isfinite(got).all()
    err = max(rel_err(got[b, h], r) for (b, h), r in ref.items())
    print(f"   max rel err {err:.3e}", flush=True)
    assert err < TOL
    return err


SMALL = replace_shape(WORKLOADS[5], B=2, T=200, H_q=4, H_kv=2)


def _random_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        G = int(rng.choice([1, 2, 3, 4, 8]))
        H_kv = int(rng.integers(1, 3))
        d = int(rng.choice([64, 128]))
        T = int(rng.integers(1, 400))
        S = T + int(rng.integers(0, 3)) * int(rng.integers(0, 100))
        B = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(0, T + 1, B)]
        cases.append((B, G, H_kv, d, T, S, lens))
    return cases


@pytest.mark.parametrize("case", _random_cases(8, 2025), ids=lambda c: f"B{c[0]}G{c[1]}Hkv{c[2]}d{c[3]}T{c[4]}S{c[5]}")
def test_random_shapes(case):
    """Seeded random shapes: group sizes, head dims, lengths (zero included),
    T not a multiple of any tile, and caches longer than T."""
    B, G, H_kv, d, T, S, lens = case
    w = replace_shape(WORKLOADS[5], B=B, T=T, H_q=G * H_kv, H_kv=H_kv, d=d,
                      q_std=d ** -0.25, k_std=d ** -0.25)
    check(w, seq_lens=lens, S_max=S)


def test_small_ragged_tail():
    check(SMALL, seq_lens=[200, 150])


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 127, 128, 129, 257, 384])
def test_lengths(T):
    w = replace_shape(WORKLOADS[5], B=1, T=T, H_q=2, H_kv=1)
    check(w)


def test_seq_lens_shorter_than_T_and_empty():
    w = replace_shape(SMALL, B=3)
    check(w, seq_lens=[200, 0, 65])


def test_cache_longer_than_T():
    check(SMALL, seq_lens=[200, 77], S_max=300)


@pytest.mark.parametrize("G,H_kv", [(1, 2), (2, 2), (4, 1)])
def test_group_sizes(G, H_kv):
    w = replace_shape(SMALL, H_q=G * H_kv, H_kv=H_kv, T=160)
    check(w)


def test_head_dim_64():
    w = replace_shape(SMALL, d=64, q_std=64 ** -0.25, k_std=64 ** -0.25)
    check(w, seq_lens=[200, 99])


def test_rho_zero_is_softmax_attention():
    check(replace_shape(SMALL, rho_std=0.0))


def test_sharp_softmax():
    check(replace_shape(SMALL, scale=8.0))


@pytest.mark.parametrize("rho_std,scale", [(0.5, 1.0), (1.0, 1.0), (1.0, 8.0)])
def test_strong_probe(rho_std, scale):
    """Probes 10-20x the workload's: the covariance correction dominates the
    output, and with a sharp softmax a few keys far from the probe reference
    carry the weight. The value contraction's fp16 weights are most exposed
    here."""
    w = replace_shape(SMALL, rho_std=rho_std, scale=scale, T=384)
    check(w, seq_lens=[384, 301])


def test_strong_probe_head_dim_64():
    """The fp16 value weights at d = 64 with a probe 20x the workload's and a
    sharp softmax."""
    w = replace_shape(SMALL, d=64, q_std=64 ** -0.25, k_std=64 ** -0.25, rho_std=1.0, scale=8.0,
                      T=384)
    check(w, seq_lens=[384, 257])


@pytest.mark.parametrize("v_std", [1e-2, 300.0])
def test_value_scale(v_std):
    """V is staged as fp16: values 100x smaller or 300x larger than the
    workload's stay inside fp16's normal range (2^-14 .. 65504), and the
    result scales with them."""
    check(replace_shape(SMALL, v_std=v_std), seq_lens=[200, 171])


def test_unscaled_dot_reading():
    check(replace_shape(SMALL, scale=128 ** -0.5))


@pytest.mark.parametrize("scale", [-128 ** -0.5, -4.0, 0.0])
def test_negative_and_zero_scale(scale):
    # scale < 0 weights the least similar keys most; scale = 0 is the uniform
    # average over the causal window (weights 1/(t+1))
    check(replace_shape(SMALL, scale=scale), seq_lens=[200, 131])


def test_large_key_offset():
    # keys with a large common component make rho . k carry a large offset
    w = SMALL
    cpu = make_prefill_inputs(w, seq_lens=[200, 180])
    cpu["k"] = (cpu["k"].float() + 4.0).to(torch.bfloat16)
    ref = oracle.oracle_prefill_full(cpu["q"], cpu["rho"], cpu["k"], cpu["v"], cpu["seq_lens"],
                                     cpu["scale"])
    got = run_prefill(to_dev(cpu))
    err = max(rel_err(got[b, h], r) for (b, h), r in ref.items())
    print(f"   large key offset: max rel err {err:.3e}", flush=True)
    assert err < TOL


def test_deterministic_bitwise():
    dev = to_dev(make_prefill_inputs(SMALL, seq_lens=[200, 150]))
    assert np.array_equal(run_prefill(dev), run_prefill(dev))


@pytest.mark.slow
def test_workload5_full_size():
    """Full-size causal prefill: every row of two heads, sampled rows of all heads."""
    w = WORKLOADS[5]
    print("[prefill parity] full-size causal-prefill", flush=True)
    dev = make_prefill_inputs(w, device="cuda")
    got = run_prefill(dev)
    assert np.isfinite(got).all()
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dev.items()}
    full = oracle.oracle_prefill_full(cpu["q"], cpu["rho"], cpu["k"], cpu["v"], cpu["seq_lens"],
                                      cpu["scale"], pairs=[(0, 0), (3, 15)])
    err_full = max(rel_err(got[b, h], r) for (b, h), r in full.items())
    rng = np.random.default_rng(5)
    T = w.T
    rows = []
    for b in range(w.B):
        for h in range(w.H_q):
            ts = {0, 1, 63, 64, 127, 128, T // 2, T - 1} | set(rng.integers(0, T, 2).tolist())
            rows += [(b, h, t) for t in ts]
    ex = oracle.oracle_prefill_rows(cpu["q"], cpu["rho"], cpu["k"], cpu["v"], cpu["seq_lens"],
                                    cpu["scale"], rows)
    err_rows = max(rel_err(got[b, h, t][None], o[None]) for (b, h, t), o in ex.items())
    print(f"   every row of 2 heads: {err_full:.3e}; {len(rows)} sampled rows: {err_rows:.3e}",
          flush=True)
    assert err_full < TOL and err_rows < TOL
