"""GPU parity of parallax_prefill_chunked (causal prefill against an existing
cache, also multi-token decode) against the fp64 oracle, through the C ABI.

Error measure as for prefill: per output row, max |gpu - oracle| / max |oracle|,
bar 2e-3; rows at or past a chunk's length must be exactly zero.
"""

import numpy as np
import pytest
import torch

import local_linear_attention_amd as pa
import oracle
from workloads import CHUNK_WORKLOAD, WORKLOADS, make_chunk_inputs, make_prefill_inputs, replace_shape

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


def run(dev):
    out = pa.prefill_chunked(dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"],
                             dev["past_lens"], dev["chunk_lens"], dev["scale"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(w, **kw):
    print(f"[chunked parity] B={w.B} T={w.T} past={w.past} Hq={w.H_q} Hkv={w.H_kv} d={w.d} {kw}",
          flush=True)
    cpu = make_chunk_inputs(w, **kw)
    ref = oracle.oracle_chunk_full(cpu["q"], cpu["rho"], cpu["k_cache"], cpu["v_cache"],
                                   cpu["past_lens"], cpu["chunk_lens"], cpu["scale"])
    got = run(to_dev(cpu))
    assert np.isfinite(got).all()
    err = max(rel_err(got[b, h], r) for (b, h), r in ref.items())
    print(f"   max rel err {err:.3e}", flush=True)
    assert err < TOL


SMALL = replace_shape(CHUNK_WORKLOAD, B=2, T=160, past=300, H_q=4, H_kv=2)


def _random_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        G = int(rng.choice([1, 2, 4, 8]))
        H_kv = int(rng.integers(1, 3))
        d = int(rng.choice([64, 128]))
        T = int(rng.integers(1, 200))
        B = int(rng.integers(1, 4))
        past = [int(x) for x in rng.integers(0, 600, B)]
        lens = [int(x) for x in rng.integers(0, T + 1, B)]
        # usually room for the chunk; sometimes a cache that cuts it short
        S = max(p + t for p, t in zip(past, lens))
        if rng.random() < 0.4:
            S -= int(rng.integers(1, 40))
        else:
            S += int(rng.integers(0, 50))
        S = max(S, T, 1)  # the chunk's query rows fit the cache (T <= S_max)
        cases.append((B, G, H_kv, d, T, S, past, lens))
    return cases


@pytest.mark.parametrize("case", _random_cases(8, 2026), ids=lambda c: f"B{c[0]}G{c[1]}Hkv{c[2]}d{c[3]}T{c[4]}S{c[5]}")
def test_random_shapes(case):
    """Seeded random shapes: past lengths, chunk lengths (zero included), group
    sizes, head dims, and caches that cut a chunk short (lengths clamped)."""
    B, G, H_kv, d, T, S, past, lens = case
    w = replace_shape(CHUNK_WORKLOAD, B=B, T=T, past=0, H_q=G * H_kv, H_kv=H_kv, d=d,
                      q_std=d ** -0.25, k_std=d ** -0.25)
    check(w, past_lens=past, chunk_lens=lens, S_max=S)


def test_small_chunk():
    check(SMALL)


@pytest.mark.parametrize("past", [0, 1, 31, 32, 33, 127, 500])
def test_past_offsets(past):
    check(replace_shape(SMALL, past=past, T=97))


@pytest.mark.parametrize("T", [1, 2, 4, 16])
def test_multi_token_decode(T):
    """A few new tokens against a long cache (speculative / multi-token decode)."""
    check(replace_shape(SMALL, T=T, past=2000))


@pytest.mark.parametrize("T", [1, 16, 17, 32, 33, 48, 64, 65, 127, 128, 129, 200, 256, 257])
def test_short_chunks(T):
    """Chunks of up to 256 rows split the keys of each row block into ranges
    and merge the ranges' states: 4 ranges of 16-row blocks up to 32 rows,
    4 of 32-row blocks up to 64, 2 of 64-row blocks up to 256; 257 rows take
    the one-range path."""
    check(replace_shape(SMALL, T=T, past=2000))


@pytest.mark.parametrize("T", [9, 32, 50, 100, 256])
def test_short_chunks_d64(T):
    w = replace_shape(SMALL, T=T, past=1500, d=64, q_std=64 ** -0.25, k_std=64 ** -0.25)
    check(w)


@pytest.mark.parametrize("T", [48, 160])
def test_short_chunks_ragged(T):
    """Split key ranges with chunk lengths and pasts that differ per sequence
    (one empty chunk, one whose keys fit in the first range)."""
    w = replace_shape(SMALL, B=4, T=T)
    check(w, past_lens=[1900, 0, 37, 700], chunk_lens=[T, 17, 0, T - 17], S_max=2000 + T)


def test_ragged_past_and_chunk_lengths():
    w = replace_shape(SMALL, B=3)
    check(w, past_lens=[300, 0, 41], chunk_lens=[160, 77, 0], S_max=500)


@pytest.mark.parametrize("scale", [-128 ** -0.5, 0.0])
def test_negative_and_zero_scale(scale):
    check(replace_shape(SMALL, scale=scale))


@pytest.mark.parametrize("T", [40, 130, 256])
@pytest.mark.parametrize("rho_std,scale", [(1.0, 1.0), (1.0, 8.0)])
def test_strong_probe(rho_std, scale, T):
    """Probes 20x the workload's, with a long past: the fp16 value weights are
    most exposed where the covariance correction dominates the output (four
    key ranges at 40 rows, two at 130 and 256)."""
    check(replace_shape(SMALL, rho_std=rho_std, scale=scale, past=1500, T=T))


def test_group_sizes_and_head_dim_64():
    check(replace_shape(SMALL, H_q=8, H_kv=2))
    check(replace_shape(SMALL, d=64, q_std=64 ** -0.25, k_std=64 ** -0.25))


def test_no_past_equals_prefill():
    """With every past length 0 the chunked call is the plain causal prefill."""
    w = replace_shape(WORKLOADS[5], B=2, T=200, H_q=4, H_kv=2)
    dev = to_dev(make_prefill_inputs(w, seq_lens=[200, 130]))
    a = pa.prefill(dev["q"], dev["rho"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"])
    zero = torch.zeros(2, dtype=torch.int32, device="cuda")
    b = pa.prefill_chunked(dev["q"], dev["rho"], dev["k"], dev["v"], zero, dev["seq_lens"],
                           dev["scale"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_chunks_reproduce_full_prefill():
    """Prefilling a sequence in three chunks gives the full prefill's rows.

    Chunks of up to 256 rows split their keys into ranges, each with its own
    running max and probe reference for the fp16 value weights, so their
    rounding differs from the one-range full prefill's (each weight within
    2^-10 of itself either way): rows agree to the per-row bar both meet
    against the oracle, not bit for bit.
    """
    w = replace_shape(WORKLOADS[5], B=1, T=384, H_q=4, H_kv=2)
    dev = to_dev(make_prefill_inputs(w))
    full = pa.prefill(dev["q"], dev["rho"], dev["k"], dev["v"], dev["seq_lens"], dev["scale"])
    for p0, p1 in [(0, 100), (100, 257), (257, 384)]:
        T = p1 - p0
        out = pa.prefill_chunked(dev["q"][:, :, p0:p1].contiguous(),
                                 dev["rho"][:, :, p0:p1].contiguous(), dev["k"], dev["v"],
                                 torch.tensor([p0], dtype=torch.int32, device="cuda"),
                                 torch.tensor([T], dtype=torch.int32, device="cuda"), dev["scale"])
        torch.cuda.synchronize()
        a = out.cpu().numpy()[0]
        b = full.cpu().numpy()[0, :, p0:p1]
        err = max(rel_err(a[h], b[h]) for h in range(w.H_q))
        print(f"   rows {p0}..{p1 - 1}: max rel difference {err:.3e}", flush=True)
        assert err < TOL


@pytest.mark.slow
def test_chunk_workload_full_size_sampled():
    w = CHUNK_WORKLOAD
    print("[chunked parity] full-size chunked-prefill", flush=True)
    dev = make_chunk_inputs(w, device="cuda")
    got = run(dev)
    assert np.isfinite(got).all()
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dev.items()}
    rng = np.random.default_rng(6)
    rows = [(b, h, t) for b in range(w.B) for h in range(w.H_q)
            for t in {0, 1, 511, w.T - 1} | set(rng.integers(0, w.T, 2).tolist())]
    ex = oracle.oracle_chunk_rows(cpu["q"], cpu["rho"], cpu["k_cache"], cpu["v_cache"],
                                  cpu["past_lens"], cpu["chunk_lens"], cpu["scale"], rows)
    err = max(rel_err(got[b, h, t][None], o[None]) for (b, h, t), o in ex.items())
    print(f"   {len(rows)} sampled rows: {err:.3e}", flush=True)
    assert err < TOL


@pytest.mark.slow
def test_longest_cache_accepted():
    """A 40-row chunk at the end of the longest cache the ABI accepts for prefill,
    (S_max + 256) d * 2 bytes just under 2^31 (d = 128): the chunk's keys sit at
    byte offsets next to 2^31. The sequence ends 3 rows before S_max; rows 40..47
    of the 48-row query tensor lie past the chunk and must be zero."""
    d = 128
    S = (1 << 31) // (d * 2) - 256 - 1
    past = S - 40 - 3
    w = replace_shape(CHUNK_WORKLOAD, B=1, T=48, past=past, H_q=2, H_kv=1)
    print(f"[chunked parity] longest cache S_max={S} past={past}", flush=True)
    dev = make_chunk_inputs(w, device="cuda", chunk_lens=[40], S_max=S)
    got = run(dev)
    assert np.isfinite(got).all()
    assert not got[0, :, 40:].any()
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dev.items()}
    rows = [(0, 0, 0), (0, 1, 39)]
    ex = oracle.oracle_chunk_rows(cpu["q"], cpu["rho"], cpu["k_cache"], cpu["v_cache"],
                                  cpu["past_lens"], cpu["chunk_lens"], cpu["scale"], rows)
    err = max(rel_err(got[b, h, t][None], o[None]) for (b, h, t), o in ex.items())
    print(f"   sampled rows {rows}: {err:.3e}", flush=True)
    assert err < TOL

