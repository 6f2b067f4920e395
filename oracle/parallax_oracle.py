"""fp64 NumPy oracle for the Parallax forward pass (decode and causal prefill).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

What is computed, per query (one query head h, one sequence b), over the keys
it may see, following the explicit definition and not any streaming form:

1. scores s_i = scale * (q . k_i); weights w = softmax(s) (max-subtracted).
   [blog "Parallax: Breaking the Boundary Bias with Parameterized Local Linear
   Attention", section "Context: Why 'Softmax' is Not Enough": softmax
   attention is the Nadaraya-Watson, local-constant estimate; the scale is the
   kernel bandwidth named in the paper page's "Abstract" as one axis of the
   family of mechanisms.]
2. weighted means mu_k = sum_i w_i k_i, mu_v = sum_i w_i v_i.
   (mu_v is the softmax-attention output.)
3. Sigma_KV = sum_i w_i (v_i - mu_v)(k_i - mu_k)^T, a d_v x d_k matrix formed
   entry by entry through one matrix product.
   [blog, section "The Core Insight: Covariance Correction", output equation;
   paper page "Abstract": rho is a second, query-like projection whose dot
   with the keys selects the covariance correction.] Readings taken where the pages are silent: rho lives in key
   space (it is dotted with keys, as a query is), so the matrix is
   value-rows x key-columns; it is centred at the softmax-weighted means; its
   weights are the same softmax weights, summing to one.
4. out = mu_v - Sigma_KV @ rho.  [blog, "The Core Insight", output equation:
   softmax attention minus the covariance applied to the probe.]

Edge readings: a query that sees no key (sequence length 0, or a prefill row
past the sequence length) outputs zeros; one key gives Sigma_KV = 0 so
out = v_0. GQA groups are contiguous: query head h reads KV head h // G with
G = H_q / H_kv. Decode has no mask (one new query against all n cached keys);
prefill row t sees keys 0..t inclusive.

All arithmetic is float64 on the exact values of the inputs (bf16 or fp32
tensors are upcast without rounding).
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast of a NumPy array or a CPU torch tensor (any float dtype)."""
    if hasattr(x, "detach"):  # torch tensor; bf16 has no NumPy dtype
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def softmax_weights(scores: np.ndarray) -> np.ndarray:
    """Softmax of a 1-D score vector, max-subtracted, in fp64 (step 1)."""
    scores = np.asarray(scores, dtype=np.float64)
    e = np.exp(scores - scores.max())
    return e / e.sum()


def sigma_kv(K: np.ndarray, V: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Softmax-weighted key/value cross-covariance, value rows x key columns.

    Sigma_KV = sum_i w_i (v_i - mu_v)(k_i - mu_k)^T   (steps 2 and 3)

    K: [n, d_k], V: [n, d_v], w: [n] non-negative weights summing to one.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    mu_k = w @ K
    mu_v = w @ V
    return (V - mu_v).T @ (w[:, None] * (K - mu_k))


def parallax_attend(q, rho, K, V, scale: float) -> np.ndarray:
    """Parallax output for one query over the keys K / values V it sees.

    out = mu_v - Sigma_KV @ rho   (steps 1-4). Zero keys give a zero vector.
    """
    q = np.asarray(q, dtype=np.float64)
    rho = np.asarray(rho, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    w = softmax_weights(scale * (K @ q))
    mu_v = w @ V
    return mu_v - sigma_kv(K, V, w) @ rho


def oracle_decode_heads(q, rho, k_cache, v_cache, seq_lens, scale, heads):
    """Decode oracle for a chosen list of (b, h) pairs; returns {(b, h): out}.

    q, rho: [B, H_q, d]; k_cache, v_cache: [B, H_kv, S_max, d];
    seq_lens: [B]. Only keys 0..seq_lens[b]-1 are read (padding is never
    touched, so NaN padding cannot leak in).
    """
    qd, rd = _f64(q), _f64(rho)
    lens = np.asarray(_f64(seq_lens), dtype=np.int64)
    H_q = qd.shape[1]
    H_kv = k_cache.shape[1]
    G = H_q // H_kv
    res = {}
    for b, h in heads:
        n = int(lens[b])
        hk = h // G
        K = _f64(k_cache[b, hk, :n])
        V = _f64(v_cache[b, hk, :n])
        res[(b, h)] = parallax_attend(qd[b, h], rd[b, h], K, V, scale)
    return res


def oracle_decode(q, rho, k_cache, v_cache, seq_lens, scale) -> np.ndarray:
    """Decode oracle for every (b, h): out [B, H_q, d] fp64."""
    B, H_q, d = q.shape
    heads = [(b, h) for b in range(B) for h in range(H_q)]
    res = oracle_decode_heads(q, rho, k_cache, v_cache, seq_lens, scale, heads)
    out = np.zeros((B, H_q, v_cache.shape[-1]), dtype=np.float64)
    for (b, h), o in res.items():
        out[b, h] = o
    return out


def oracle_prefill_rows(q, rho, k, v, seq_lens, scale, rows):
    """Causal-prefill oracle, explicit Sigma_KV, for chosen (b, h, t) rows.

    q, rho: [B, H_q, T, d]; k, v: [B, H_kv, S_max, d] with T <= S_max;
    seq_lens: [B]. Row t sees keys 0..t; rows t >= seq_lens[b] are zero.
    Returns {(b, h, t): out}.
    """
    lens = np.asarray(_f64(seq_lens), dtype=np.int64)
    H_q = q.shape[1]
    G = H_q // k.shape[1]
    res = {}
    for b, h, t in rows:
        if t >= lens[b]:
            res[(b, h, t)] = np.zeros(v.shape[-1], dtype=np.float64)
            continue
        hk = h // G
        K = _f64(k[b, hk, : t + 1])
        V = _f64(v[b, hk, : t + 1])
        res[(b, h, t)] = parallax_attend(_f64(q[b, h, t]), _f64(rho[b, h, t]), K, V, scale)
    return res


def oracle_prefill_full(q, rho, k, v, seq_lens, scale, pairs=None):
    """Every row of the causal prefill for chosen (b, h) pairs, fp64.

    The same centred definition as ``parallax_attend`` for all rows at once,
    with dense masked T x T matrices, and with Sigma_KV applied to rho by
    associativity instead of being formed as a d x d matrix per row:

        (Sigma_KV rho)_t = sum_j w_tj (v_j - mu_v,t) ((k_j - mu_k,t) . rho_t)

    Returns {(b, h): out [T, d]} (rows t >= seq_lens[b] are zero).
    """
    B, H_q, T, _ = q.shape
    G = H_q // k.shape[1]
    lens = np.asarray(_f64(seq_lens), dtype=np.int64)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H_q)]
    res = {}
    for b, h in pairs:
        n = int(min(lens[b], T))
        out = np.zeros((T, v.shape[-1]), dtype=np.float64)
        if n > 0:
            hk = h // G
            Q = _f64(q[b, h, :n])
            R = _f64(rho[b, h, :n])
            K = _f64(k[b, hk, :n])
            V = _f64(v[b, hk, :n])
            S = scale * (Q @ K.T)
            S[np.triu_indices(n, 1)] = -np.inf  # row t sees keys 0..t
            W = np.exp(S - S.max(axis=1, keepdims=True))
            W /= W.sum(axis=1, keepdims=True)
            mu_v = W @ V
            mu_k = W @ K
            # (k_j - mu_k,t) . rho_t for every (t, j)
            Rc = R @ K.T - np.sum(R * mu_k, axis=1, keepdims=True)
            WR = W * Rc
            corr = WR @ V - WR.sum(axis=1, keepdims=True) * mu_v
            out[:n] = mu_v - corr
        res[(b, h)] = out
    return res


def _chunk_bounds(past_lens, chunk_lens, T, S_max):
    """Per-sequence (past, n) with the clamping the chunked entry point applies."""
    past = np.clip(np.asarray(_f64(past_lens), dtype=np.int64), 0, S_max)
    n = np.minimum(np.clip(np.asarray(_f64(chunk_lens), dtype=np.int64), 0, T), S_max - past)
    return past, n


def oracle_chunk_rows(q, rho, k_cache, v_cache, past_lens, chunk_lens, scale, rows):
    """Chunked causal prefill, explicit Sigma_KV, for chosen (b, h, t) rows.

    Row t of the chunk sits at position p = past_lens[b] + t of the sequence
    and sees cache keys 0..p (the cache already holds the chunk's own keys);
    rows t >= chunk_lens[b] are zero. With past 0 this is the causal prefill.
    q, rho: [B, H_q, T, d]; k_cache, v_cache: [B, H_kv, S_max, d].
    Returns {(b, h, t): out}.
    """
    T = q.shape[2]
    S_max = k_cache.shape[2]
    past, n = _chunk_bounds(past_lens, chunk_lens, T, S_max)
    G = q.shape[1] // k_cache.shape[1]
    res = {}
    for b, h, t in rows:
        if t >= n[b]:
            res[(b, h, t)] = np.zeros(v_cache.shape[-1], dtype=np.float64)
            continue
        p = int(past[b]) + t
        K = _f64(k_cache[b, h // G, : p + 1])
        V = _f64(v_cache[b, h // G, : p + 1])
        res[(b, h, t)] = parallax_attend(_f64(q[b, h, t]), _f64(rho[b, h, t]), K, V, scale)
    return res


def oracle_chunk_full(q, rho, k_cache, v_cache, past_lens, chunk_lens, scale, pairs=None):
    """Every row of a chunked causal prefill for chosen (b, h) pairs, fp64.

    Same centred definition as ``oracle_prefill_full`` with the mask shifted
    by the past length: chunk row t sees keys j <= past + t.
    Returns {(b, h): out [T, d]}.
    """
    B, H_q, T, _ = q.shape
    S_max = k_cache.shape[2]
    past, n = _chunk_bounds(past_lens, chunk_lens, T, S_max)
    G = H_q // k_cache.shape[1]
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H_q)]
    res = {}
    for b, h in pairs:
        out = np.zeros((T, v_cache.shape[-1]), dtype=np.float64)
        nb, pb = int(n[b]), int(past[b])
        if nb > 0:
            nk = pb + nb
            Q = _f64(q[b, h, :nb])
            R = _f64(rho[b, h, :nb])
            K = _f64(k_cache[b, h // G, :nk])
            V = _f64(v_cache[b, h // G, :nk])
            S = scale * (Q @ K.T)
            S[np.arange(nk)[None, :] > (pb + np.arange(nb))[:, None]] = -np.inf
            W = np.exp(S - S.max(axis=1, keepdims=True))
            W /= W.sum(axis=1, keepdims=True)
            mu_v = W @ V
            mu_k = W @ K
            Rc = R @ K.T - np.sum(R * mu_k, axis=1, keepdims=True)
            WR = W * Rc
            out[:nb] = mu_v - (WR @ V - WR.sum(axis=1, keepdims=True) * mu_v)
        res[(b, h)] = out
    return res
