"""The allocation-free decode (parallax_decode_noalloc, built-in per-device
scratch) against parallax_decode (caller's workspace), through the C ABI.

Two calls in a row, the second with a smaller input (fewer sequences and
heads, another head dim, ragged lengths), then the first shape again: the
scratch keeps the previous call's records, and its arrival counters must be
back at zero for every call to merge correctly. Each output must equal
parallax_decode's (the same kernels and plan) and lie within the 2e-3 bar
of the fp64 oracle.
"""

import numpy as np
import pytest
import torch

import local_linear_attention_amd as pa
import oracle
from workloads import WORKLOADS, make_decode_inputs, replace_shape

TOL = 2e-3
pytestmark = pytest.mark.gpu


def _rel(got, ref):
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    zero = den == 0
    assert np.all(num[zero] == 0)
    return float((num[~zero] / den[~zero]).max()) if np.any(~zero) else 0.0


def _case(w, seq_lens, seed):
    cpu = make_decode_inputs(w, seq_lens=seq_lens, seed=seed)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in cpu.items()}
    return cpu, dev


def _check(cpu, dev, num_splits=0):
    args = (dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"], dev["seq_lens"], dev["scale"])
    got = pa.decode_noalloc(*args, num_splits=num_splits)
    ref_gpu = pa.decode(*args, num_splits=num_splits)
    torch.cuda.synchronize()
    got, ref_gpu = got.cpu().numpy(), ref_gpu.cpu().numpy()
    assert np.array_equal(got, ref_gpu), "allocation-free decode differs from parallax_decode"
    ref = oracle.oracle_decode(cpu["q"], cpu["rho"], cpu["k_cache"], cpu["v_cache"],
                               cpu["seq_lens"], cpu["scale"])
    err = _rel(got, ref)
    print(f"   max rel err vs oracle {err:.3e}", flush=True)
    assert err < TOL
    return got


def test_noalloc_matches_decode_twice_then_again():
    big = replace_shape(WORKLOADS[2], B=4, S_max=2048)
    small = replace_shape(WORKLOADS[2], B=2, H_q=8, H_kv=2, d=64, S_max=700,
                          q_std=64 ** -0.25, k_std=64 ** -0.25)
    print("[noalloc] B=4 H_q=16 H_kv=8 d=128 S=2048", flush=True)
    cpu1, dev1 = _case(big, [2048, 1500, 1, 777], seed=31)
    first = _check(cpu1, dev1)
    print("[noalloc] B=2 H_q=8 H_kv=2 d=64 S=700 (smaller, after the first)", flush=True)
    cpu2, dev2 = _case(small, [700, 333], seed=32)
    _check(cpu2, dev2)
    print("[noalloc] first shape again, forced 7 splits, then automatic", flush=True)
    _check(cpu1, dev1, num_splits=7)
    again = _check(cpu1, dev1)
    assert np.array_equal(first, again)


def test_noalloc_empty_sequences_and_one_split():
    w = replace_shape(WORKLOADS[2], B=3, H_q=4, H_kv=2, S_max=512)
    print("[noalloc] empty sequences; one split", flush=True)
    cpu, dev = _case(w, [0, 512, 0], seed=33)
    _check(cpu, dev)
    _check(cpu, dev, num_splits=1)


def test_noalloc_rejects_plans_past_the_scratch():
    w = replace_shape(WORKLOADS[2], B=64, S_max=4096)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
           for k, v in make_decode_inputs(w, seed=34, device="cuda").items()}
    with pytest.raises(pa.ParallaxError, match="TOO_LARGE"):
        pa.decode_noalloc(dev["q"], dev["rho"], dev["k_cache"], dev["v_cache"], dev["seq_lens"],
                          dev["scale"], num_splits=32)
