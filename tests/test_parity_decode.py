"""GPU parity of parallax_decode against the fp64 oracle (through the C ABI).

Error measure: per output row (b, h), max_i |gpu_i - oracle_i| / max_i |oracle_i|,
maximised over rows; bar 2e-3 (bf16 or fp32 inputs, fp32 accumulation).
Rows whose oracle output is exactly zero (no keys) must be exactly zero.
"""

import math

import numpy as np
import pytest
import torch

import local_linear_attention_amd as pa
import oracle
from workloads import WORKLOADS, make_decode_inputs, replace_shape

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


def run_decode(inp, num_splits=0):
    out = pa.decode(inp["q"], inp["rho"], inp["k_cache"], inp["v_cache"], inp["seq_lens"],
                    inp["scale"], num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_all(inp):
    return oracle.oracle_decode(inp["q"], inp["rho"], inp["k_cache"], inp["v_cache"],
                                inp["seq_lens"], inp["scale"])


def check(w, *, seed=0, seq_lens=None, num_splits=(0,), **kw):
    print(f"[decode parity] {w.name} B={w.B} Hq={w.H_q} Hkv={w.H_kv} d={w.d} S={w.S_max} "
          f"{w.dtype} seed={seed} lens={seq_lens} splits={num_splits} {kw}", flush=True)
    cpu = make_decode_inputs(w, seed=seed, seq_lens=seq_lens, **kw)
    ref = oracle_all(cpu)
    dev = to_dev(cpu)
    errs = []
    for ns in num_splits:
        got = run_decode(dev, ns)
        assert np.isfinite(got).all()
        errs.append(rel_err(got, ref))
    print(f"   max rel err {errs}", flush=True)
    assert max(errs) < TOL, errs
    return errs


SMALL2 = replace_shape(WORKLOADS[2], B=3, S_max=700)


def test_workload1_full():
    """Single-head fp32 decode at its full size, every split plan."""
    check(WORKLOADS[1], num_splits=(0, 1, 2, 4))


def test_workload2_small_ragged_tail():
    check(SMALL2, seq_lens=[700, 333, 97], num_splits=(0, 1, 3, 6))


@pytest.mark.parametrize("n", [0, 1, 2, 31, 32, 33, 127, 128, 129, 255, 256, 257, 511])
def test_edge_lengths(n):
    w = replace_shape(WORKLOADS[2], B=2, S_max=512)
    check(w, seq_lens=[n, 512 - n], num_splits=(1, 2, 4))


@pytest.mark.parametrize("G,H_kv", [(1, 3), (2, 2), (3, 2), (4, 2), (5, 2), (6, 1), (7, 2),
                                    (8, 1), (10, 1), (12, 1), (13, 1)])
def test_group_sizes(G, H_kv):
    w = replace_shape(WORKLOADS[2], B=2, H_q=G * H_kv, H_kv=H_kv, S_max=300)
    check(w, seq_lens=[300, 161], num_splits=(0, 1))


@pytest.mark.parametrize("d,dtype", [(64, torch.bfloat16), (128, torch.float32),
                                     (64, torch.float32)])
def test_head_dims_and_dtypes(d, dtype):
    w = replace_shape(WORKLOADS[2], B=2, H_q=4, H_kv=2, d=d, S_max=400, dtype=dtype,
                      q_std=d ** -0.25, k_std=d ** -0.25)
    check(w, seq_lens=[400, 259], num_splits=(0, 1, 3))


def _random_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 10, 12]))
        H_kv = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
        S = int(rng.integers(1, 1500))
        B = int(rng.integers(1, 5))
        lens = [int(x) for x in rng.integers(0, S + 1, B)]
        splits = (0, 1, int(rng.integers(2, 8)))
        cases.append((B, G, H_kv, d, dtype, S, lens, splits))
    return cases


@pytest.mark.parametrize("case", _random_cases(10, 2024), ids=lambda c: f"B{c[0]}G{c[1]}Hkv{c[2]}d{c[3]}S{c[5]}")
def test_random_shapes(case):
    """Seeded random shapes: group sizes, head dims, dtypes, cache lengths,
    ragged lengths (zero included) and split counts together."""
    B, G, H_kv, d, dtype, S, lens, splits = case
    w = replace_shape(WORKLOADS[2], B=B, H_q=G * H_kv, H_kv=H_kv, d=d, S_max=S, dtype=dtype,
                      q_std=d ** -0.25, k_std=d ** -0.25)
    check(w, seq_lens=lens, num_splits=splits)


def test_head_groups_placed_together():
    """More than 4 query heads per KV head: one 8-head workgroup (two probe
    tiles) per KV head and split at G = 8, and several head groups at G = 12
    (8 + 4 heads) and G = 16 (8 + 8), whose workgroups are placed on one XCD
    when the grid size is divisible by 8 x groups."""
    for G in (6, 8, 12, 16):
        w = replace_shape(WORKLOADS[2], B=4, H_q=G * 4, H_kv=4, S_max=1024)
        check(w, seq_lens=[1024, 1000, 517, 3], num_splits=(0, 2, 4))


def test_rho_zero_is_softmax_attention():
    w = replace_shape(SMALL2, rho_std=0.0)
    check(w, seq_lens=[700, 5, 400])


def test_large_key_offset():
    # a common key offset shifts every r = rho . k by a large constant
    check(SMALL2, seq_lens=[700, 260, 64], k_offset=4.0, num_splits=(1, 5))


def test_sharp_softmax():
    check(SMALL2, seq_lens=[700, 300, 129], scale_mult=8.0, num_splits=(0, 1))


def test_unscaled_dot_reading():
    # the same q, k distributions with an extra 1/sqrt(d) bandwidth
    check(SMALL2, seq_lens=[700, 64, 640], scale_mult=1 / math.sqrt(128))


@pytest.mark.parametrize("scale_mult", [-1.0, -8.0, 0.0])
def test_negative_and_zero_scale(scale_mult):
    check(SMALL2, seq_lens=[700, 300, 129], scale_mult=scale_mult, num_splits=(0, 1, 5))


def test_deterministic_bitwise_static_paths():
    """One split, and the two-phase partial + combine, are bitwise repeatable."""
    w = SMALL2
    dev = to_dev(make_decode_inputs(w, seq_lens=[700, 333, 97]))
    assert np.array_equal(run_decode(dev, 1), run_decode(dev, 1))
    ns, _ = pa.decode_plan(w.B, w.H_q, w.H_kv, w.d, w.S_max, 4)
    ws = torch.empty(pa.decode_workspace_size(w.B, w.H_q, w.d, ns) // 4, device="cuda")
    outs = []
    for _ in range(2):
        out = torch.empty(w.B, w.H_q, w.d, device="cuda")
        pa.decode_partial(dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"], dev["seq_lens"],
                          dev["scale"], ws, num_splits=4)
        pa.decode_combine(dev["seq_lens"], out, ws, H_kv=w.H_kv, S_max=w.S_max, num_splits=4)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_fused_deterministic_bitwise():
    dev = to_dev(make_decode_inputs(SMALL2, seq_lens=[700, 333, 97]))
    assert np.array_equal(run_decode(dev, 6), run_decode(dev, 6))


def test_two_phase_equals_one_shot():
    w = SMALL2
    dev = to_dev(make_decode_inputs(w, seq_lens=[700, 333, 97]))
    ns, _ = pa.decode_plan(w.B, w.H_q, w.H_kv, w.d, w.S_max, 4)
    ws = torch.empty(pa.decode_workspace_size(w.B, w.H_q, w.d, ns) // 4, device="cuda")
    out = torch.empty(w.B, w.H_q, w.d, device="cuda")
    pa.decode_partial(dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"], dev["seq_lens"],
                      dev["scale"], ws, num_splits=4)
    pa.decode_combine(dev["seq_lens"], out, ws, H_kv=w.H_kv, S_max=w.S_max, num_splits=4)
    one = run_decode(dev, 4)
    torch.cuda.synchronize()
    # same splits, same records, same merge order: bitwise equal
    assert np.array_equal(out.cpu().numpy(), one)


@pytest.mark.parametrize("ns,H_q", [(2, 16), (3, 16), (5, 16), (8, 16), (12, 16), (16, 16), (32, 16),
                                     (5, 64), (12, 64)])
def test_two_phase_equals_one_shot_split_counts(ns, H_q):
    """Fused and two-phase merges agree bit for bit whatever the split count.

    The merging workgroup batches its record loads by the number of splits
    that hold keys (up to 8 at a time); the combine kernel does the same
    with other item widths. Lengths here give streams with 1 up to ns
    splits, so every batch size and a second batch are exercised.
    """
    w = replace_shape(WORKLOADS[2], B=3, H_q=H_q, S_max=4096)
    dev = to_dev(make_decode_inputs(w, seq_lens=[4096, 1029, 97]))
    nsr, _ = pa.decode_plan(w.B, w.H_q, w.H_kv, w.d, w.S_max, ns)
    assert nsr == (11 if ns == 12 else ns)  # the plan's chunks are multiples of 128 keys
    ws = torch.empty(pa.decode_workspace_size(w.B, w.H_q, w.d, nsr) // 4, device="cuda")
    out = torch.empty(w.B, w.H_q, w.d, device="cuda")
    pa.decode_partial(dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"], dev["seq_lens"],
                      dev["scale"], ws, num_splits=ns)
    pa.decode_combine(dev["seq_lens"], out, ws, H_kv=w.H_kv, S_max=w.S_max, num_splits=ns)
    one = run_decode(dev, ns)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), one)
    ref = oracle_all(dev)
    assert rel_err(one, ref) < TOL


def test_out_of_range_seq_lens_are_clamped():
    w = replace_shape(WORKLOADS[2], B=2, S_max=256)
    cpu = make_decode_inputs(w, seq_lens=[256, 0], nan_pad=False)
    dev = to_dev(cpu)
    dev["seq_lens"] = torch.tensor([100000, -5], dtype=torch.int32, device="cuda")
    got = run_decode(dev)
    ref = oracle_all(cpu)
    assert rel_err(got, ref) < TOL


# ------------------------------------------------------------- full-size workloads


def test_workload2_full():
    check(WORKLOADS[2])


def _sampled(w, heads, seed=None, gen_device="cuda"):
    print(f"[decode parity] full-size {w.name}, sampled heads {heads}", flush=True)
    dev = make_decode_inputs(w, seed=seed, device=gen_device)
    got = run_decode(dev)
    lens = dev["seq_lens"].cpu()
    errs = []
    G = w.H_q // w.H_kv
    for b, h in heads:
        n = int(lens[b])
        kk = dev["k_cache"][b, h // G, :n].cpu()
        vv = dev["v_cache"][b, h // G, :n].cpu()
        ref = oracle.parallax_attend(oracle.parallax_oracle._f64(dev["q"][b, h].cpu()),
                                     oracle.parallax_oracle._f64(dev["rho"][b, h].cpu()),
                                     oracle.parallax_oracle._f64(kk),
                                     oracle.parallax_oracle._f64(vv), dev["scale"])
        errs.append(rel_err(got[b, h][None], ref[None]))
    print(f"   max rel err {max(errs):.3e}", flush=True)
    assert max(errs) < TOL
    assert np.isfinite(got).all()


def test_gqa8_full_size_sampled():
    """The G = 8 decode (64 query heads on 8 KV heads, 8 x 4096 keys) in the
    automatic plan that the benchmark times: every head of two KV heads."""
    w = replace_shape(WORKLOADS[2], name="gqa8-decode", H_q=64)
    heads = [(0, h) for h in range(8)] + [(7, h) for h in range(56, 64)]
    _sampled(w, heads)


def test_gqa_d64_full_size_sampled():
    """The gqa-decode shape at head dim 64 (8 x 4096 keys, 16 query heads on 8
    KV heads) in the automatic plan the benchmark times (4 splits of 1024
    keys, 8-wave workgroups): every head of the first and last sequence."""
    w = replace_shape(WORKLOADS[2], name="gqa-decode-d64", d=64, q_std=64 ** -0.25,
                      k_std=64 ** -0.25)
    heads = [(0, h) for h in range(16)] + [(7, h) for h in range(16)]
    _sampled(w, heads)


@pytest.mark.slow
def test_workload3_full_sampled():
    w = WORKLOADS[3]
    heads = [(0, 0), (1, 15), (17, 6), (33, 9), (50, 2), (63, 14)]
    _sampled(w, heads)


@pytest.mark.slow
def test_workload4_full_sampled():
    w = WORKLOADS[4]
    heads = [(0, 0), (0, 5), (0, 18), (0, 31)]
    _sampled(w, heads)


def test_fused_workspace_reuse_counters_return_to_zero():
    """One zeroed workspace serves successive fused calls with different lengths."""
    w = SMALL2
    ns, _ = pa.decode_plan(w.B, w.H_q, w.H_kv, w.d, w.S_max, 6)
    nbytes = pa.decode_workspace_size(w.B, w.H_q, w.d, ns)
    ws = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    rec_words = w.B * w.H_q * ns * (2 * w.d + 4)
    for lens in ([700, 333, 97], [5, 700, 0], [129, 128, 700], [0, 0, 0]):
        cpu = make_decode_inputs(w, seq_lens=lens)
        dev = to_dev(cpu)
        out = pa.decode(dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"], dev["seq_lens"],
                        dev["scale"], num_splits=6, workspace=ws)
        torch.cuda.synchronize()
        assert rel_err(out.cpu().numpy(), oracle_all(cpu)) < TOL
        ctr = ws[rec_words:].view(torch.int32)
        assert int(ctr.abs().sum()) == 0


@pytest.mark.slow
@pytest.mark.parametrize("d", [128, 64])
def test_longest_cache_accepted(d):
    """The longest KV cache the ABI accepts, (S_max + 64) d * 2 bytes just under 2^31
    per (b, KV head) for bf16 (d = 128 and d = 64, whose workgroups have 8 waves):
    the last rows' byte offsets sit next to 2^31. The sequence ends 5 keys before
    S_max (NaN padding after it). Automatic plan, and one workgroup per head group
    streaming all of it."""
    S = (1 << 31) // (d * 2) - 64 - 1
    n = S - 5
    w = replace_shape(WORKLOADS[2], B=1, H_q=2, H_kv=1, d=d, S_max=S, q_std=d ** -0.25,
                      k_std=d ** -0.25)
    print(f"[decode parity] longest cache d={d} S_max={S} n={n}", flush=True)
    dev = make_decode_inputs(w, device="cuda", seq_lens=[n])
    outs = {ns: run_decode(dev, ns) for ns in (0, 1)}
    K = oracle.parallax_oracle._f64(dev["k_cache"][0, 0, :n].cpu())
    V = oracle.parallax_oracle._f64(dev["v_cache"][0, 0, :n].cpu())
    for h in range(2):
        ref = oracle.parallax_attend(oracle.parallax_oracle._f64(dev["q"][0, h].cpu()),
                                     oracle.parallax_oracle._f64(dev["rho"][0, h].cpu()),
                                     K, V, dev["scale"])
        errs = {ns: rel_err(o[0, h][None], ref[None]) for ns, o in outs.items()}
        print(f"   head {h}: max rel err {errs}", flush=True)
        assert max(errs.values()) < TOL

