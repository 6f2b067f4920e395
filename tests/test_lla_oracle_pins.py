"""Pins of the LLA oracle extension (the solver-based Local Linear Attention
that Parallax replaces) to things other than itself (CPU only).

* conjugate gradient against NumPy's dense solve on random symmetric
  positive-definite systems, and against an exact 2 x 2 system solved by hand;
* the LLA output against NumPy's least squares: the weighted local linear fit
  at the query (lam = 0) and the same fit with a ridge penalty on the slope
  written as extra rows of the least-squares system (lam > 0);
* limits: exactly linear data is recovered at the query; a huge lam gives
  softmax attention (torch's scaled_dot_product_attention in fp64); one key
  gives v_0; no key gives 0.

``test_lla_mutants_are_caught`` plants plausible mistakes (flipped right-hand
side, uncentred key covariance, ridge added to the wrong matrix, a CG step
with a wrong sign) and checks that each fails a pin.
"""

import numpy as np
import pytest
import torch

from oracle import lla_oracle as lo
from oracle import parallax_oracle as po


def _rng(seed):
    return np.random.default_rng(seed)


def _spd(rng, d, cond):
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    ev = np.geomspace(1.0, 1.0 / cond, d)
    return (Q * ev) @ Q.T


def _case(rng, n, d, edge=1.5):
    q = rng.standard_normal(d) + edge  # query near the edge of the key cloud
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    return q, K, V


def _weights(q, K, scale):
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return w / w.sum()


def _ridge_intercept(q, K, V, w, lam):
    """Intercept of min sum_i w_i |v_i - a - B (k_i - q)|^2 + lam |B|^2 by
    least squares on the augmented system: rows sqrt(w_i) [1, k_i - q] with
    targets sqrt(w_i) v_i, plus rows sqrt(lam) [0, e_j] with target 0."""
    n, d = K.shape
    X = np.hstack([np.ones((n, 1)), K - q]) * np.sqrt(w)[:, None]
    Y = V * np.sqrt(w)[:, None]
    if lam > 0:
        X = np.vstack([X, np.hstack([np.zeros((d, 1)), np.sqrt(lam) * np.eye(d)])])
        Y = np.vstack([Y, np.zeros((d, V.shape[1]))])
    coef, *_ = np.linalg.lstsq(X, Y, rcond=None)
    return coef[0]


# ---- pins, each taking the functions under test so mutants can be fed in

def pin_cg(cg, seed=11):
    rng = _rng(seed)
    for d, cond in [(4, 10.0), (16, 1e3), (64, 1e4), (128, 1e3)]:
        A = _spd(rng, d, cond)
        b = rng.standard_normal(d)
        x, it, _ = cg(A, b, tol=1e-13)
        ref = np.linalg.solve(A, b)
        if not np.allclose(x, ref, rtol=1e-8, atol=1e-10 * np.abs(ref).max()):
            return False
    # exact 2 x 2: [[4, 1], [1, 3]] x = [1, 2] -> x = (1/11, 7/11); CG ends in 2 steps
    x, it, _ = cg(np.array([[4.0, 1.0], [1.0, 3.0]]), np.array([1.0, 2.0]), tol=1e-14)
    return np.allclose(x, [1 / 11, 7 / 11], rtol=0, atol=1e-15) and it == 2


def pin_lla_regression(lla, seed=12):
    rng = _rng(seed)
    for n, d, scale, lam in [(12, 3, 0.8, 0.0), (40, 6, 0.5, 0.0), (100, 8, 0.3, 0.0),
                             (40, 6, 0.5, 0.1), (100, 8, 0.3, 2.0), (300, 16, 0.25, 0.05)]:
        q, K, V = _case(rng, n, d)
        out, rho, _ = lla(q, K, V, scale, lam)
        w = _weights(q, K, scale)
        ref = _ridge_intercept(q, K, V, w, lam)
        if not np.allclose(out, ref, rtol=1e-8, atol=1e-9):
            return False
    return True


def pin_lla_limits(lla, seed=13):
    rng = _rng(seed)
    for n, d, scale in [(30, 4, 0.6), (200, 12, 0.3)]:
        q, K, V = _case(rng, n, d)
        # exactly linear values are recovered at the query (lam = 0)
        a0 = rng.standard_normal(d)
        B0 = rng.standard_normal((d, d))
        Vlin = a0 + (K - q) @ B0.T
        out, _, _ = lla(q, K, Vlin, scale, 0.0)
        if not np.allclose(out, a0, rtol=1e-8, atol=1e-8):
            return False
        # a huge ridge pins the slope to 0: softmax attention (torch SDPA, fp64)
        out, _, _ = lla(q, K, V, scale, 1e12)
        sdpa = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, None, None], torch.tensor(K)[None, None],
            torch.tensor(V)[None, None], scale=scale)[0, 0, 0].numpy()
        if not np.allclose(out, sdpa, rtol=1e-9, atol=1e-10):
            return False
    # one key: the fit is the key's value whatever the ridge
    q, K, V = _case(rng, 1, 5)
    for lam in (0.0, 0.3):
        out, _, _ = lla(q, K, V, 0.7, lam)
        if not np.allclose(out, V[0], rtol=0, atol=1e-12):
            return False
    out, _, _ = lla(q, K[:0], V[:0], 0.7, 0.1)
    return np.all(out == 0.0)


def test_cg_pins():
    assert pin_cg(lo.conjugate_gradient)


def test_lla_regression_pins():
    assert pin_lla_regression(lo.lla_attend)


def test_lla_limit_pins():
    assert pin_lla_limits(lo.lla_attend)


def test_cg_and_direct_solve_agree():
    rng = _rng(14)
    q, K, V = _case(rng, 500, 32, edge=0.5)
    for lam in (1e-3, 1e-1):
        a, ra, it = lo.lla_attend(q, K, V, 0.2, lam, solver="cg")
        b, rb, _ = lo.lla_attend(q, K, V, 0.2, lam, solver="direct")
        assert np.allclose(ra, rb, rtol=1e-8, atol=1e-10)
        assert np.allclose(a, b, rtol=1e-9, atol=1e-12)
        assert 0 < it <= 4 * 32


def test_lla_is_parallax_at_the_solved_probe():
    rng = _rng(15)
    q, K, V = _case(rng, 64, 8)
    out, rho, _ = lo.lla_attend(q, K, V, 0.5, 0.05)
    assert np.array_equal(out, po.parallax_attend(q, rho, K, V, 0.5))


# ---- mutants

def _cg_wrong_step(A, b, tol=1e-12, maxiter=None):
    A = np.asarray(A, float)
    x = np.zeros_like(b, dtype=float)
    r = b.astype(float).copy()
    p = r.copy()
    rr = r @ r
    for it in range(4 * len(b)):
        if np.sqrt(rr) <= tol * np.linalg.norm(b):
            break
        Ap = A @ p
        alpha = rr / (p @ Ap)
        x += alpha * p
        r -= alpha * Ap
        rr_new = r @ r
        p = r - (rr_new / rr) * p  # wrong sign in the direction update
        rr = rr_new
    return x, it, float(np.sqrt(rr))


def _lla_variant(kind):
    def lla(q, K, V, scale, lam):
        q = np.asarray(q, float)
        K = np.asarray(K, float)
        V = np.asarray(V, float)
        if len(K) == 0:
            return np.zeros(V.shape[1]), np.zeros(K.shape[1]), 0
        w = po.softmax_weights(scale * (K @ q))
        mu_k = w @ K
        if kind == "uncentred":
            S = K.T @ (w[:, None] * K)
        else:
            S = lo.sigma_kk(K, w)
        b = mu_k - q if kind != "flipped_rhs" else q - mu_k
        A = S + lam * np.eye(K.shape[1]) if kind != "ridge_on_rhs" else S
        if kind == "ridge_on_rhs":
            b = b + lam
        rho = np.linalg.lstsq(A, b, rcond=None)[0]
        return po.parallax_attend(q, rho, K, V, scale), rho, 0
    return lla


@pytest.mark.parametrize("kind", ["flipped_rhs", "uncentred", "ridge_on_rhs"])
def test_lla_mutants_are_caught(kind):
    m = _lla_variant(kind)
    assert not (pin_lla_regression(m) and pin_lla_limits(m))


def test_cg_mutant_is_caught():
    assert not pin_cg(_cg_wrong_step)


def test_unmutated_variant_passes():
    # control for the mutant test: the same harness without a planted mistake
    m = _lla_variant("none")
    assert pin_lla_regression(m) and pin_lla_limits(m)
