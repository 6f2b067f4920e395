"""fp64 oracle for the fused q, k, v, rho projection.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the product path.

The probe rho is a learned projection of the layer input, like the query
(blog "Parallax: Breaking the Boundary Bias with Parameterized Local Linear
Attention", "The Core Insight: Covariance Correction" and "Architecture-
Optimizer Codesign": the W_R projection; paper page "Parallax: Parameterized
Local Linear Attention for Language Modeling", "Abstract"). With the packed
weight W = [W_Q; W_K; W_V; W_R] ((2 H_q + 2 H_kv) d rows of d_model
weights), every output feature f of token (b, t) is the dot product
x[b, t] . W[f]; the first H_q d features are q (head f // d, dim f % d), then
H_kv d of k, H_kv d of v and H_q d of rho. Computed with one fp64 matrix
product (a library routine as one step) on the exact input values; the
kernel rounds its fp32 sums to bf16, the test compares with that in mind.

Pinned in tests/test_projection_oracle_pins.py against a pure-Python
element-by-element evaluation of that definition.
"""

from __future__ import annotations

import numpy as np


def oracle_qkvr_projection(x, w, H_q: int, H_kv: int, d: int):
    """x [B, T, d_model], w [(2 H_q + 2 H_kv) d, d_model] (NumPy or torch, any
    float dtype). Returns fp64 (q, k, v, rho): q, rho [B, H_q, T, d];
    k, v [B, H_kv, T, d]."""
    if hasattr(x, "detach"):
        import torch

        x = x.detach().to("cpu", torch.float64).numpy()
        w = w.detach().to("cpu", torch.float64).numpy()
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, _ = x.shape
    y = x @ w.T  # [B, T, N]
    sizes = [H_q * d, H_kv * d, H_kv * d, H_q * d]
    heads = [H_q, H_kv, H_kv, H_q]
    outs = []
    f0 = 0
    for n, h in zip(sizes, heads):
        outs.append(y[:, :, f0:f0 + n].reshape(B, T, h, d).transpose(0, 2, 1, 3).copy())
        f0 += n
    return tuple(outs)
