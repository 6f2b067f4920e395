"""Seeded synthetic workloads for the Parallax forward pass.

This module holds shapes, value distributions and a seeded generator and
nothing of the method's arithmetic; both the HIP path and the oracle are fed
from it. The shapes and distributions are the five workloads the path is
measured and checked on:

1. single-head decode: B=1, H_q=H_kv=1, d=64, 512 keys, fp32;
   q, k, v ~ N(0,1), rho ~ N(0, 0.1^2).
2. GQA decode: B=8, H_q=16, H_kv=8, d=128, 4096 keys per sequence, bf16;
   q, k ~ N(0,1) * d^-1/4, v ~ N(0,1), rho ~ N(0, 0.05^2).
3. ragged-batch decode: B=64, H_q=16, H_kv=8, d=128, bf16, per-sequence key
   counts uniform on [1024, 32768]; distributions as in 2.
4. long-context split-KV decode: B=1, H_q=32, H_kv=8, d=128, 131072 keys,
   bf16; distributions as in 2.
5. causal prefill: B=4, T=4096, H_q=16, H_kv=8, d=128, bf16, per-token rho;
   distributions as in 2.

The softmax scale (the kernel bandwidth) is a workload parameter: 1/sqrt(d)
for workload 1, whose q and k are unit normals; 1 for the others, whose q and
k already carry a d^-1/4 factor each, which folds 1/sqrt(d) into q.k.

Draw order per workload, from one generator seeded with ``seed``:
sequence lengths (ragged only), then q, k, v, rho; each is drawn in fp32,
scaled by its standard deviation and rounded to the storage dtype with
round-to-nearest-even. Cache rows at or past a sequence's length are filled
with NaN so that any read of them poisons the result.
"""

from __future__ import annotations

import dataclasses
import math

import torch

__all__ = [
    "DecodeWorkload",
    "PrefillWorkload",
    "ChunkWorkload",
    "WORKLOADS",
    "CHUNK_WORKLOAD",
    "make_decode_inputs",
    "make_prefill_inputs",
    "make_chunk_inputs",
    "replace_shape",
]


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H_q: int
    H_kv: int
    d: int
    S_max: int
    dtype: torch.dtype
    q_std: float
    k_std: float
    v_std: float
    rho_std: float
    scale: float
    ragged: tuple | None = None  # (lo, hi) inclusive bounds of seq lens
    seed: int = 0

    def kv_bytes(self, seq_lens) -> int:
        """Bytes of K and V that lie inside the sequences (the KV stream)."""
        esz = torch.finfo(self.dtype).bits // 8
        return int(sum(int(n) for n in seq_lens)) * self.H_kv * self.d * esz * 2


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    T: int
    H_q: int
    H_kv: int
    d: int
    dtype: torch.dtype
    q_std: float
    k_std: float
    v_std: float
    rho_std: float
    scale: float
    seed: int = 0


@dataclasses.dataclass(frozen=True)
class ChunkWorkload:
    """Causal prefill of a chunk of T rows after `past` cached tokens."""
    name: str
    B: int
    T: int
    past: int
    H_q: int
    H_kv: int
    d: int
    dtype: torch.dtype
    q_std: float
    k_std: float
    v_std: float
    rho_std: float
    scale: float
    seed: int = 0


_D128 = 128 ** -0.25

WORKLOADS = {
    1: DecodeWorkload("single-head-decode", 1, 1, 1, 64, 512, torch.float32,
                      1.0, 1.0, 1.0, 0.1, 1.0 / math.sqrt(64), seed=1001),
    2: DecodeWorkload("gqa-decode", 8, 16, 8, 128, 4096, torch.bfloat16,
                      _D128, _D128, 1.0, 0.05, 1.0, seed=1002),
    3: DecodeWorkload("ragged-batch-decode", 64, 16, 8, 128, 32768, torch.bfloat16,
                      _D128, _D128, 1.0, 0.05, 1.0, ragged=(1024, 32768), seed=1003),
    4: DecodeWorkload("long-context-splitkv-decode", 1, 32, 8, 128, 131072, torch.bfloat16,
                      _D128, _D128, 1.0, 0.05, 1.0, seed=1004),
    5: PrefillWorkload("causal-prefill", 4, 4096, 16, 8, 128, torch.bfloat16,
                       _D128, _D128, 1.0, 0.05, 1.0, seed=1005),
}


# Chunked prefill (prefill against an existing cache): the last quarter of the
# causal-prefill workload, 1024 new rows after 3072 cached tokens.
CHUNK_WORKLOAD = ChunkWorkload("chunked-prefill", 4, 1024, 3072, 16, 8, 128, torch.bfloat16,
                               _D128, _D128, 1.0, 0.05, 1.0, seed=1006)


def replace_shape(w, **kw):
    """A copy of a workload with some fields changed (smaller test shapes)."""
    return dataclasses.replace(w, **kw)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, std, dtype, g, device, offset=0.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    if offset:
        x.add_(offset)
    return x.to(dtype)


def make_decode_inputs(w: DecodeWorkload, seed=None, device="cpu", seq_lens=None,
                       nan_pad=True, k_offset=0.0, scale_mult=1.0):
    """Seeded decode inputs for workload ``w``.

    Returns a dict of tensors on ``device``: q, rho [B, H_q, d];
    k_cache, v_cache [B, H_kv, S_max, d]; seq_lens int32 [B]; plus the
    float ``scale``. ``seq_lens`` overrides the drawn lengths (edge cases);
    ``k_offset`` adds a constant to every key before rounding (a large common
    key offset); ``scale_mult`` sharpens the softmax.

    K and V are drawn one batch entry at a time to bound peak memory.
    """
    seed = w.seed if seed is None else seed
    g = _gen(device, seed)
    B, Hq, Hkv, d, S = w.B, w.H_q, w.H_kv, w.d, w.S_max
    if seq_lens is None:
        if w.ragged is not None:
            lo, hi = w.ragged
            lens = torch.randint(lo, hi + 1, (B,), generator=g, device=device)
        else:
            lens = torch.full((B,), S, device=device, dtype=torch.int64)
    else:
        lens = torch.as_tensor(seq_lens, device=device)
    lens = lens.to(torch.int32)
    q = _normal((B, Hq, d), w.q_std, w.dtype, g, device)
    k = torch.empty((B, Hkv, S, d), dtype=w.dtype, device=device)
    v = torch.empty((B, Hkv, S, d), dtype=w.dtype, device=device)
    for b in range(B):
        k[b] = _normal((Hkv, S, d), w.k_std, w.dtype, g, device, offset=k_offset)
    for b in range(B):
        v[b] = _normal((Hkv, S, d), w.v_std, w.dtype, g, device)
    rho = _normal((B, Hq, d), w.rho_std, w.dtype, g, device)
    if nan_pad:
        lens_host = lens.cpu().tolist()
        for b, n in enumerate(lens_host):
            if n < S:
                k[b, :, n:] = float("nan")
                v[b, :, n:] = float("nan")
    return dict(q=q, rho=rho, k_cache=k, v_cache=v, seq_lens=lens,
                scale=float(w.scale * scale_mult))


def make_prefill_inputs(w: PrefillWorkload, seed=None, device="cpu", seq_lens=None,
                        S_max=None, nan_pad=True):
    """Seeded causal-prefill inputs for workload ``w``.

    Returns q, rho [B, H_q, T, d] (rho is per token); k, v [B, H_kv, S_max, d]
    with S_max >= T (default T); seq_lens int32 [B] (default T); ``scale``.
    """
    seed = w.seed if seed is None else seed
    g = _gen(device, seed)
    B, T, Hq, Hkv, d = w.B, w.T, w.H_q, w.H_kv, w.d
    S = T if S_max is None else int(S_max)
    if seq_lens is None:
        lens = torch.full((B,), T, device=device, dtype=torch.int32)
    else:
        lens = torch.as_tensor(seq_lens, device=device).to(torch.int32)
    q = _normal((B, Hq, T, d), w.q_std, w.dtype, g, device)
    k = _normal((B, Hkv, S, d), w.k_std, w.dtype, g, device)
    v = _normal((B, Hkv, S, d), w.v_std, w.dtype, g, device)
    rho = _normal((B, Hq, T, d), w.rho_std, w.dtype, g, device)
    if nan_pad:
        for b, n in enumerate(lens.cpu().tolist()):
            if n < S:
                k[b, :, n:] = float("nan")
                v[b, :, n:] = float("nan")
    return dict(q=q, rho=rho, k=k, v=v, seq_lens=lens, scale=float(w.scale))


def make_chunk_inputs(w: ChunkWorkload, seed=None, device="cpu", past_lens=None,
                      chunk_lens=None, S_max=None, nan_pad=True):
    """Seeded chunked-prefill inputs for workload ``w``.

    Returns q, rho [B, H_q, T, d] (the chunk's rows); k_cache, v_cache
    [B, H_kv, S_max, d] (S_max >= past + T, default exactly that) holding the
    past and the chunk's own keys and values; past_lens, chunk_lens int32 [B]
    (defaults: w.past and w.T for every sequence); ``scale``. Cache rows at or
    past past_lens[b] + chunk_lens[b] are NaN.
    """
    seed = w.seed if seed is None else seed
    g = _gen(device, seed)
    B, T, Hq, Hkv, d = w.B, w.T, w.H_q, w.H_kv, w.d
    past = torch.as_tensor([w.past] * B if past_lens is None else past_lens).to(torch.int32)
    lens = torch.as_tensor([T] * B if chunk_lens is None else chunk_lens).to(torch.int32)
    S = int(S_max) if S_max is not None else int(past.max()) + T
    q = _normal((B, Hq, T, d), w.q_std, w.dtype, g, device)
    k = _normal((B, Hkv, S, d), w.k_std, w.dtype, g, device)
    v = _normal((B, Hkv, S, d), w.v_std, w.dtype, g, device)
    rho = _normal((B, Hq, T, d), w.rho_std, w.dtype, g, device)
    if nan_pad:
        for b in range(B):
            end = int(past[b]) + int(lens[b])
            if end < S:
                k[b, :, end:] = float("nan")
                v[b, :, end:] = float("nan")
    return dict(q=q, rho=rho, k_cache=k, v_cache=v, past_lens=past.to(device),
                chunk_lens=lens.to(device), scale=float(w.scale))
