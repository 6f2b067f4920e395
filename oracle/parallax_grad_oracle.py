"""fp64 oracle for the gradients of the causal Parallax prefill.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the product path.

The forward is the explicit definition of ``parallax_oracle`` (blog
"Parallax: Breaking the Boundary Bias with Parameterized Local Linear
Attention", "The Core Insight: Covariance Correction", output equation):
per row t over keys j <= t,

    w = softmax(scale q_t . k_j),  mu_v = sum w v,  mu_k = sum w k,
    out_t = mu_v - S_KV rho_t,  S_KV = sum w (v - mu_v)(k - mu_k)^T,

written here in torch fp64 with dense masked T x T matrices (the same form
as ``oracle_prefill_full``: S_KV applied to rho by associativity, centring
explicit). The gradients (dq, drho, dk, dv) for an upstream gradient dO of
out are that function's derivatives, taken by torch autograd in fp64 (a
library routine used as one step). Rows t >= seq_lens[b] have zero output and
zero gradient; keys past seq_lens[b] get zero gradient. dk, dv sum over the
query heads of a GQA group. Training the probe is the pages' use of this
(paper page "Parallax: Parameterized Local Linear Attention for Language
Modeling", "Abstract": Parallax is pretrained with the learned probe).

Pins (tests/test_grad_oracle_pins.py): central finite differences of the
NumPy oracle, torch SDPA's gradients for rho = 0, the closed form
drho_t = -S_KV,t^T dO_t with NumPy's weighted covariance, and the key- and
value-shift invariances.
"""

from __future__ import annotations

import numpy as np
import torch


def _t64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to(device="cpu", dtype=torch.float64)
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def prefill_head_torch(Q, R, K, V, scale: float):
    """Causal Parallax output for one (b, h): Q, R [n, d], K, V [n, d] (torch
    fp64, rows and keys both 0..n-1). Differentiable."""
    n = Q.shape[0]
    S = scale * (Q @ K.T)
    mask = torch.triu(torch.ones(n, n, dtype=torch.bool), 1)  # key j > row t
    S = S.masked_fill(mask, float("-inf"))
    W = torch.softmax(S, dim=1)
    mu_v = W @ V
    mu_k = W @ K
    Rc = R @ K.T - (R * mu_k).sum(dim=1, keepdim=True)   # (k_j - mu_k,t) . rho_t
    WR = W * Rc
    return mu_v - (WR @ V - WR.sum(dim=1, keepdim=True) * mu_v)


def oracle_prefill_grads(q, rho, k, v, seq_lens, dout, scale: float, kv_heads=None):
    """Gradients of the causal prefill for upstream gradient `dout`.

    q, rho, dout: [B, H_q, T, d]; k, v: [B, H_kv, S_max, d]; seq_lens: [B].
    Returns (dq, drho, dk, dv) as fp64 NumPy arrays shaped like q, rho, k, v.
    `kv_heads` (list of (b, h_kv)) restricts the work to those KV heads and
    the query heads of their groups; everything else is left zero.
    """
    q, rho, k, v, dout = (_t64(x) for x in (q, rho, k, v, dout))
    lens = np.asarray(_t64(seq_lens).numpy(), dtype=np.int64)
    B, H_q, T, d = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    dq = torch.zeros_like(q)
    drho = torch.zeros_like(rho)
    dk = torch.zeros_like(k)
    dv = torch.zeros_like(v)
    for b in range(B):
        n = int(min(lens[b], T))
        if n <= 0:
            continue
        for h in range(H_q):
            hk = h // G
            if kv_heads is not None and (b, hk) not in kv_heads:
                continue
            Q = q[b, h, :n].clone().requires_grad_(True)
            R = rho[b, h, :n].clone().requires_grad_(True)
            K = k[b, hk, :n].clone().requires_grad_(True)
            V = v[b, hk, :n].clone().requires_grad_(True)
            out = prefill_head_torch(Q, R, K, V, scale)
            gq, gr, gk, gv = torch.autograd.grad(out, (Q, R, K, V), grad_outputs=dout[b, h, :n])
            dq[b, h, :n] = gq
            drho[b, h, :n] = gr
            dk[b, hk, :n] += gk
            dv[b, hk, :n] += gv
    return dq.numpy(), drho.numpy(), dk.numpy(), dv.numpy()
