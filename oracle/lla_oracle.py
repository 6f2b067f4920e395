"""fp64 oracle for Local Linear Attention (LLA), the solver-based variant that
Parallax replaces.

TEST INFRASTRUCTURE ONLY: imported by the tests and by the contrast script in
this package, never by the product path.

Sources (page titles and sections):

* Blog "Parallax: Breaking the Boundary Bias with Parameterized Local Linear
  Attention", section "Context: Why 'Softmax' is Not Enough": softmax attention
  is the local-constant (Nadaraya-Watson) estimate with a boundary bias; the
  earlier Local Linear Attention fixes it but solves a linear system per token
  with conjugate gradient, which is what kept it from scaling.
* Same post, "The Core Insight: Covariance Correction": the local linear
  estimate becomes an additive covariance correction to softmax attention; in
  Parallax a learned probe takes the place of the solved vector.
* Paper page "Parallax: Parameterized Local Linear Attention for Language
  Modeling", "Abstract": LLA has numerical-stability concerns; Parallax removes
  the numerical solver.

The pages print no LLA formula. The one used here is textbook local linear
regression (weighted least squares of the values on the keys, centred at the
query, the intercept being the estimate), with a ridge penalty on the slope as
the regularisation the stability concern calls for:

    min_{a, B}  sum_i w_i |v_i - a - B (k_i - q)|^2 + lam |B|_F^2

Its intercept is a = mu_v - S_KV rho* with

    rho* = (S_KK + lam I)^{-1} (mu_k - q),   S_KK = sum_i w_i (k_i - mu_k)(k_i - mu_k)^T,

i.e. the Parallax output (``parallax_attend``) at the probe rho*. rho* is found
by conjugate gradient on the symmetric positive (semi-)definite system, the
solver the blog names. With lam = 0 and n > d generic keys this is plain local
linear regression; as lam grows rho* -> 0 and the estimate tends to softmax
attention.
"""

from __future__ import annotations

import numpy as np

from .parallax_oracle import parallax_attend, softmax_weights


def conjugate_gradient(A, b, tol: float = 1e-12, maxiter: int | None = None):
    """Solves A x = b for symmetric positive (semi-)definite A by conjugate
    gradient (Hestenes-Stiefel), starting from x = 0.

    Stops when |r| <= tol |b| or after `maxiter` iterations (default: the
    dimension, the exact-arithmetic bound, times 4). Returns (x, iterations,
    final residual norm).
    """
    A = np.asarray(A, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n = b.shape[0]
    maxiter = 4 * n if maxiter is None else maxiter
    x = np.zeros(n)
    r = b.copy()           # residual b - A x
    p = r.copy()           # search direction
    rr = float(r @ r)
    bnorm = float(np.sqrt(b @ b))
    if bnorm == 0.0:
        return x, 0, 0.0
    it = 0
    while it < maxiter and np.sqrt(rr) > tol * bnorm:
        Ap = A @ p
        pAp = float(p @ Ap)
        if pAp <= 0.0:     # direction in the null space of a singular A
            break
        alpha = rr / pAp
        x += alpha * p
        r -= alpha * Ap
        rr_new = float(r @ r)
        p = r + (rr_new / rr) * p
        rr = rr_new
        it += 1
    return x, it, float(np.sqrt(rr))


def sigma_kk(K, w):
    """Softmax-weighted key covariance sum_i w_i (k_i - mu_k)(k_i - mu_k)^T."""
    K = np.asarray(K, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    Kc = K - w @ K
    return Kc.T @ (w[:, None] * Kc)


def lla_probe(q, K, scale: float, lam: float, solver: str = "cg", tol: float = 1e-12,
              maxiter: int | None = None):
    """The solved probe rho* = (S_KK + lam I)^{-1} (mu_k - q) for one query.

    solver: "cg" (conjugate gradient, the LLA solver) or "direct"
    (np.linalg.solve, for comparison). Returns (rho*, CG iterations or 0).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    w = softmax_weights(scale * (K @ q))
    A = sigma_kk(K, w) + lam * np.eye(K.shape[1])
    b = w @ K - q
    if solver == "direct":
        return np.linalg.solve(A, b), 0
    rho, it, _ = conjugate_gradient(A, b, tol=tol, maxiter=maxiter)
    return rho, it


def lla_attend(q, K, V, scale: float, lam: float, solver: str = "cg", tol: float = 1e-12,
               maxiter: int | None = None):
    """LLA output for one query: the ridge local-linear intercept at q.

    Equals ``parallax_attend(q, rho*, K, V, scale)`` with rho* from
    ``lla_probe``. Returns (out, rho*, CG iterations). No keys give zeros.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), np.zeros(K.shape[1]), 0
    rho, it = lla_probe(q, K, scale, lam, solver=solver, tol=tol, maxiter=maxiter)
    return parallax_attend(q, rho, K, V, scale), rho, it
