"""GPU parity of parallax_decode_tokens (multi-token decode: the chunked-prefill
result for a few new tokens per sequence, by the split-KV decode kernel)
against the fp64 oracle, through the C ABI.

Error measure as for the chunked prefill: per output row (b, h, t),
max |gpu - oracle| / max |oracle|, bar 2e-3; rows at or past a chunk's length
must be exactly zero.
"""

import numpy as np
import pytest
import torch

import local_linear_attention_amd as pa
import oracle
from workloads import CHUNK_WORKLOAD, WORKLOADS, make_chunk_inputs, make_decode_inputs, replace_shape

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


def run_tokens(dev, num_splits=0):
    out = pa.decode_tokens(dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"], dev["past_lens"],
                           dev["chunk_lens"], dev["scale"], num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(w, *, num_splits=(0, 1, 3), **kw):
    print(f"[decode_tokens parity] B={w.B} T={w.T} Hq={w.H_q} Hkv={w.H_kv} d={w.d} {w.dtype} "
          f"{kw} splits={num_splits}", flush=True)
    cpu = make_chunk_inputs(w, **kw)
    ref = oracle.oracle_chunk_full(cpu["q"], cpu["rho"], cpu["k_cache"], cpu["v_cache"],
                                   cpu["past_lens"], cpu["chunk_lens"], cpu["scale"])
    dev = to_dev(cpu)
    errs = []
    for ns in num_splits:
        got = run_tokens(dev, ns)
        assert np.isfinite(got).all()
        errs.append(max(rel_err(got[b, h], r) for (b, h), r in ref.items()))
    print(f"   max rel err {errs}", flush=True)
    assert max(errs) < TOL, errs


def small(**kw):
    base = dict(B=3, T=4, past=0, H_q=4, H_kv=2, d=128)
    base.update(kw)
    return replace_shape(CHUNK_WORKLOAD, **base)


@pytest.mark.parametrize("T", [1, 2, 4])
def test_group_of_two(T):
    """G = 2 (the gqa shape's group): T = 1, 2 fit one group of 4 (head, token)
    pairs; T = 4 fills one 8-pair workgroup (two probe tiles)."""
    check(small(T=T), past_lens=[700, 33, 256], chunk_lens=[T, max(T - 1, 0), T], S_max=720)


@pytest.mark.parametrize("G,H_kv,T", [(1, 3, 4), (4, 1, 1), (4, 2, 2), (8, 1, 2), (2, 2, 8),
                                      (2, 2, 3), (1, 2, 5), (2, 1, 5), (3, 2, 3)])
def test_group_sizes_and_tokens(G, H_kv, T):
    check(small(H_q=G * H_kv, H_kv=H_kv, T=T), past_lens=[400, 0, 129],
          chunk_lens=[T, T, 1], S_max=420)


@pytest.mark.parametrize("d,dtype", [(64, torch.bfloat16), (128, torch.float32)])
def test_head_dims_and_dtypes(d, dtype):
    w = small(d=d, dtype=dtype, q_std=d ** -0.25, k_std=d ** -0.25, T=2)
    check(w, past_lens=[500, 7, 64], chunk_lens=[2, 1, 2], S_max=510)


def test_zero_and_clamped_chunks():
    """A zero-length chunk writes zeros; a cache that ends inside the chunk
    clamps its length; a past beyond the cache clamps to it (no keys left)."""
    check(small(T=4), past_lens=[300, 318, 400], chunk_lens=[0, 4, 3], S_max=320)


def test_one_token_equals_decode():
    """T = 1 with chunk length 1 is the plain decode over past + 1 keys: same
    kernel arithmetic, so bitwise the same output."""
    w = replace_shape(WORKLOADS[2], B=3, S_max=700)
    cpu = make_decode_inputs(w, seq_lens=[700, 334, 98])
    dev = to_dev(cpu)
    ref = pa.decode(dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"], dev["seq_lens"],
                    dev["scale"], num_splits=4)
    past = (dev["seq_lens"] - 1).to(torch.int32)
    ones = torch.ones_like(past)
    got = pa.decode_tokens(dev["q"][:, :, None].contiguous(), dev["rho"][:, :, None].contiguous(),
                           dev["k_cache"], dev["v_cache"], past, ones, dev["scale"], num_splits=4)
    torch.cuda.synchronize()
    assert np.array_equal(got[:, :, 0].cpu().numpy(), ref.cpu().numpy())


def test_matches_chunked_prefill():
    """The same inputs through parallax_prefill_chunked agree to the bar."""
    w = small(B=2, T=3, H_q=16, H_kv=4)  # 12 (head, token) pairs per KV head
    dev = to_dev(make_chunk_inputs(w, past_lens=[600, 90], chunk_lens=[3, 2], S_max=640))
    a = run_tokens(dev)
    b = pa.prefill_chunked(dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"],
                           dev["past_lens"], dev["chunk_lens"], dev["scale"]).cpu().numpy()
    assert rel_err(a, b.astype(np.float64)) < TOL


def test_workspace_reuse_counts_return_to_zero():
    w = small(T=2)
    ns, _ = pa.decode_plan(w.B, w.H_q * w.T, w.H_kv, w.d, 720, 5)
    ws = torch.zeros(pa.decode_workspace_size(w.B, w.H_q * w.T, w.d, ns) // 4, device="cuda")
    rec_words = w.B * w.H_q * w.T * ns * (2 * w.d + 4)
    for past, clen in (([700, 33, 256], [2, 1, 2]), ([0, 718, 5], [2, 2, 0]), ([10, 10, 10], [0, 0, 0])):
        cpu = make_chunk_inputs(w, past_lens=past, chunk_lens=clen, S_max=720)
        dev = to_dev(cpu)
        out = pa.decode_tokens(dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"],
                               dev["past_lens"], dev["chunk_lens"], dev["scale"], num_splits=5,
                               workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.oracle_chunk_full(cpu["q"], cpu["rho"], cpu["k_cache"], cpu["v_cache"],
                                       cpu["past_lens"], cpu["chunk_lens"], cpu["scale"])
        got = out.cpu().numpy()
        assert max(rel_err(got[b, h], r) for (b, h), r in ref.items()) < TOL
        assert int(ws[rec_words:].view(torch.int32).abs().sum()) == 0


@pytest.mark.slow
def test_gqa_shape_four_tokens_sampled():
    """The gqa-decode shape (B=8, H_q=16, H_kv=8, d=128) with 4 new tokens
    after 4092 cached ones; sampled rows against the oracle."""
    w = replace_shape(CHUNK_WORKLOAD, B=8, T=4, past=4092, H_q=16, H_kv=8, d=128)
    dev = make_chunk_inputs(w, device="cuda")
    got = run_tokens(dev)
    assert np.isfinite(got).all()
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dev.items()}
    rows = [(0, 0, 0), (0, 1, 3), (3, 7, 1), (5, 10, 2), (7, 15, 3)]
    ex = oracle.oracle_chunk_rows(cpu["q"], cpu["rho"], cpu["k_cache"], cpu["v_cache"],
                                  cpu["past_lens"], cpu["chunk_lens"], cpu["scale"], rows)
    err = max(rel_err(got[b, h, t][None], o[None]) for (b, h, t), o in ex.items())
    print(f"   sampled rows: {err:.3e}", flush=True)
    assert err < TOL


def _random_cases(n=10, seed=20261203):
    """Seeded shapes that combine group size, token count, head dim, dtype,
    cache size, past and chunk lengths (past may run past the cache, which
    clamps the chunk) and split count."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 3, 4, 6, 8]))
        H_kv = int(rng.integers(1, 4))
        T = int(rng.integers(1, 9))
        d = int(rng.choice([64, 128]))
        dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
        B = int(rng.integers(1, 4))
        S = int(rng.integers(T, 900))
        past = [int(x) for x in rng.integers(0, S + 1, B)]
        clen = [int(x) for x in rng.integers(0, T + 1, B)]
        cases.append((G, H_kv, T, d, dtype, B, S, past, clen, int(rng.integers(2, 8))))
    return cases


@pytest.mark.parametrize("case", _random_cases(),
                         ids=lambda c: f"G{c[0]}-Hkv{c[1]}-T{c[2]}-d{c[3]}-S{c[6]}")
def test_random_shapes(case):
    G, H_kv, T, d, dtype, B, S, past, clen, ns = case
    w = small(B=B, T=T, H_q=G * H_kv, H_kv=H_kv, d=d, dtype=dtype, q_std=d ** -0.25,
              k_std=d ** -0.25)
    check(w, past_lens=past, chunk_lens=clen, S_max=S, num_splits=(0, 1, ns))
