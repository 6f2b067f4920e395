"""Accuracy and cost contrast of LLA (solved probe) and Parallax / softmax
attention on synthetic data, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (it calls nothing but this package and the seeded
input generator):

    python -m oracle.lla_contrast [--heads 8] [--keys 4096]

Keys and queries are those of the GQA decode workload (d = 128, q and k
~ N(0, 1) d^-1/4 rounded to bf16, softmax scale 1). Values follow a known
function of the keys, so the regression target at the query is known:

    linear:    v_i = c + M k_i + 0.1 eps_i
    nonlinear: v_i = c + M k_i + tanh(N k_i) + 0.1 eps_i

with c, M, N, eps seeded normals (M and N scaled by 1/sqrt(d)). The truth
at the query is f(q) (the noise-free function). Softmax attention (Parallax
with rho = 0) estimates f at the weighted key mean, hence its boundary bias
(blog "Parallax: Breaking the Boundary Bias with Parameterized Local Linear
Attention", "Context: Why 'Softmax' is Not Enough"); LLA solves for the
probe per query by conjugate gradient. Parallax with a learned probe sits
between the two; no trained probe exists here, so it is not measured.
"""

from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle.lla_oracle import lla_attend  # noqa: E402
from oracle.parallax_oracle import _f64, parallax_attend  # noqa: E402


def run(heads=8, keys=4096, lams=(1e-4, 1e-3, 1e-2), seed=7):
    from workloads import WORKLOADS, make_decode_inputs, replace_shape

    w = replace_shape(WORKLOADS[2], B=1, H_q=heads, H_kv=heads, S_max=keys)
    inp = make_decode_inputs(w, seed=seed, device="cpu", nan_pad=False)
    d = w.d
    rng = np.random.default_rng(seed)
    rows = []
    for kind in ("linear", "nonlinear"):
        errs = {"softmax": [], **{f"lla lam={lam:g}": [] for lam in lams}}
        iters = {lam: [] for lam in lams}
        t_sm = t_lla = 0.0
        for h in range(heads):
            q = _f64(inp["q"][0, h])
            K = _f64(inp["k_cache"][0, h])
            c = rng.standard_normal(d)
            M = rng.standard_normal((d, d)) / np.sqrt(d)
            N = rng.standard_normal((d, d)) / np.sqrt(d)
            f = (lambda x: c + x @ M.T) if kind == "linear" else \
                (lambda x: c + x @ M.T + np.tanh(x @ N.T))
            V = f(K) + 0.1 * rng.standard_normal((keys, d))
            truth = f(q[None])[0]
            norm = np.abs(truth).max()
            t0 = time.perf_counter()
            sm = parallax_attend(q, np.zeros(d), K, V, inp["scale"])
            t_sm += time.perf_counter() - t0
            errs["softmax"].append(np.abs(sm - truth).max() / norm)
            for lam in lams:
                t0 = time.perf_counter()
                out, _, it = lla_attend(q, K, V, inp["scale"], lam, tol=1e-10)
                t_lla += time.perf_counter() - t0
                errs[f"lla lam={lam:g}"].append(np.abs(out - truth).max() / norm)
                iters[lam].append(it)
        rows.append((kind, {k: float(np.median(v)) for k, v in errs.items()},
                     {lam: float(np.mean(v)) for lam, v in iters.items()},
                     t_sm / heads, t_lla / (heads * len(lams))))
    return rows, d, keys


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--heads", type=int, default=8)
    ap.add_argument("--keys", type=int, default=4096)
    args = ap.parse_args()
    rows, d, n = run(args.heads, args.keys)
    print(f"d = {d}, n = {n} keys, {args.heads} query heads; median over heads of "
          f"max|est - f(q)| / max|f(q)|")
    for kind, errs, iters, t_sm, t_lla in rows:
        print(f"\n{kind} values")
        for k, v in errs.items():
            print(f"  {k:16s} rel err {v:.3e}")
        for lam, it in iters.items():
            print(f"  CG iterations at lam={lam:g} (tol 1e-10): {it:.1f}")
        print(f"  oracle time per query: softmax/Parallax {t_sm * 1e3:.2f} ms, "
              f"LLA {t_lla * 1e3:.2f} ms")
    print(f"\nflops per query: Parallax streaming 8 d n = {8 * d * n / 1e6:.1f} M; "
          f"LLA key covariance 2 n d^2 = {2 * n * d * d / 1e6:.1f} M plus 2 d^2 per CG "
          f"iteration, and mu_k must be known before the covariance (a second pass or "
          f"a d x d running state per query)")


if __name__ == "__main__":
    main()
