"""Pins of the prefill gradient oracle to things other than itself (CPU only).

* central finite differences of the NumPy oracle (``oracle_prefill_full``),
  a separate code path from the torch forward that autograd differentiates:
  directional derivatives along random directions of q, rho, k and v;
* rho = 0: torch's scaled_dot_product_attention gradients (fp64, causal, GQA);
* the closed form drho_t = -S_KV,t^T dO_t, with S_KV from NumPy's weighted
  covariance (the output is affine in rho with slope -S_KV);
* invariances: shifting every key by one vector leaves every output
  unchanged, so the key gradients of a KV head sum to zero; shifting every
  value by c shifts every output by c, so the value gradients sum to the sum
  of the upstream gradients of the rows that see keys.

``test_grad_mutants_are_caught`` differentiates plausible wrong forwards
(uncentred covariance, causal off-by-one, GQA gradients assigned instead of
summed) and checks each fails a pin.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import parallax_grad_oracle as go


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(rng, B=2, H_q=4, H_kv=2, T=9, d=5, lens=None, edge=0.0):
    q = rng.standard_normal((B, H_q, T, d)) * 0.7
    rho = rng.standard_normal((B, H_q, T, d)) * 0.4
    k = rng.standard_normal((B, H_kv, T, d)) + edge
    v = rng.standard_normal((B, H_kv, T, d))
    dout = rng.standard_normal((B, H_q, T, d))
    lens = np.array([T] * B if lens is None else lens)
    return q, rho, k, v, lens, dout


def _forward_np(q, rho, k, v, lens, scale):
    res = oracle.oracle_prefill_full(q, rho, k, v, lens, scale)
    B, H_q, T, d = q.shape
    out = np.zeros((B, H_q, T, d))
    for (b, h), o in res.items():
        out[b, h] = o
    return out


def pin_finite_differences(grads_fn, seed=31):
    rng = _rng(seed)
    scale = 0.8
    for lens in ([9, 6], [9, 0]):
        q, rho, k, v, lens, dout = _inputs(rng, lens=lens)
        dq, drho, dk, dv = grads_fn(q, rho, k, v, lens, dout, scale)
        args = [q, rho, k, v]
        grads = [dq, drho, dk, dv]
        for i in range(4):
            for _ in range(2):
                u = rng.standard_normal(args[i].shape)
                eps = 1e-5
                plus = list(args)
                minus = list(args)
                plus[i] = args[i] + eps * u
                minus[i] = args[i] - eps * u
                fd = np.sum(dout * (_forward_np(*plus, lens, scale) - _forward_np(*minus, lens, scale))) / (2 * eps)
                an = np.sum(grads[i] * u)
                if not abs(fd - an) <= 1e-7 * max(1.0, abs(fd)):
                    return False
    return True


def pin_sdpa_rho_zero(grads_fn, seed=32):
    rng = _rng(seed)
    q, rho, k, v, lens, dout = _inputs(rng, B=1, H_q=4, H_kv=2, T=12, d=6)
    rho[:] = 0.0
    dq, drho, dk, dv = grads_fn(q, rho, k, v, lens, dout, 0.6)
    Q = torch.tensor(q, requires_grad=True)
    K = torch.tensor(k, requires_grad=True)
    V = torch.tensor(v, requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=0.6,
                                                           enable_gqa=True)
    gq, gk, gv = torch.autograd.grad(out, (Q, K, V), grad_outputs=torch.tensor(dout))
    return (np.allclose(dq, gq.numpy(), rtol=1e-10, atol=1e-12)
            and np.allclose(dk, gk.numpy(), rtol=1e-10, atol=1e-12)
            and np.allclose(dv, gv.numpy(), rtol=1e-10, atol=1e-12))


def pin_drho_closed_form(grads_fn, seed=33):
    rng = _rng(seed)
    q, rho, k, v, lens, dout = _inputs(rng, B=1, H_q=2, H_kv=1, T=10, d=4)
    scale = 0.9
    _, drho, _, _ = grads_fn(q, rho, k, v, lens, dout, scale)
    for h in range(2):
        for t in range(10):
            K = k[0, 0, : t + 1]
            V = v[0, 0, : t + 1]
            s = scale * K @ q[0, h, t]
            w = np.exp(s - s.max())
            w /= w.sum()
            if t == 0:
                S = np.zeros((4, 4))
            else:
                S = np.cov(np.vstack([V.T, K.T]), aweights=w, bias=True)[:4, 4:]
            if not np.allclose(drho[0, h, t], -S.T @ dout[0, h, t], rtol=1e-10, atol=1e-12):
                return False
    return True


def pin_shift_invariances(grads_fn, seed=34):
    rng = _rng(seed)
    q, rho, k, v, lens, dout = _inputs(rng, B=2, H_q=4, H_kv=2, T=8, d=5, lens=[8, 5], edge=2.0)
    _, _, dk, dv = grads_fn(q, rho, k, v, lens, dout, 0.7)
    G = 2
    for b in range(2):
        n = lens[b]
        for hk in range(2):
            if not np.allclose(dk[b, hk].sum(axis=0), 0.0, atol=1e-10):
                return False
            want = dout[b, G * hk: G * hk + G, :n].sum(axis=(0, 1))
            if not np.allclose(dv[b, hk].sum(axis=0), want, rtol=1e-10, atol=1e-10):
                return False
            if np.any(dk[b, hk, n:] != 0) or np.any(dv[b, hk, n:] != 0):
                return False
    return True


PINS = (pin_finite_differences, pin_sdpa_rho_zero, pin_drho_closed_form, pin_shift_invariances)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_grad_oracle_pins(pin):
    assert pin(go.oracle_prefill_grads)


# ---- mutants: autograd of wrong forwards, or wrong accumulation

def _grads_with_forward(head_fn, accumulate=True):
    def grads(q, rho, k, v, seq_lens, dout, scale):
        q, rho, k, v, dout = (torch.as_tensor(np.asarray(x, float)) for x in (q, rho, k, v, dout))
        B, H_q, T, d = q.shape
        G = H_q // k.shape[1]
        dq, drho, dk, dv = (torch.zeros_like(x) for x in (q, rho, k, v))
        for b in range(B):
            n = int(min(seq_lens[b], T))
            if n <= 0:
                continue
            for h in range(H_q):
                hk = h // G
                Q, R, K, V = (x.clone().requires_grad_(True)
                              for x in (q[b, h, :n], rho[b, h, :n], k[b, hk, :n], v[b, hk, :n]))
                gq, gr, gk, gv = torch.autograd.grad(head_fn(Q, R, K, V, scale), (Q, R, K, V),
                                                     grad_outputs=dout[b, h, :n])
                dq[b, h, :n], drho[b, h, :n] = gq, gr
                if accumulate:
                    dk[b, hk, :n] += gk
                    dv[b, hk, :n] += gv
                else:
                    dk[b, hk, :n] = gk
                    dv[b, hk, :n] = gv
        return dq.numpy(), drho.numpy(), dk.numpy(), dv.numpy()
    return grads


def _uncentred(Q, R, K, V, scale):
    n = Q.shape[0]
    S = (scale * (Q @ K.T)).masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    W = torch.softmax(S, dim=1)
    return W @ V - (W * (R @ K.T)) @ V


def _off_by_one(Q, R, K, V, scale):
    n = Q.shape[0]
    # row t also sees key t + 1
    S = (scale * (Q @ K.T)).masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 2), float("-inf"))
    W = torch.softmax(S, dim=1)
    mu_v, mu_k = W @ V, W @ K
    WR = W * (R @ K.T - (R * mu_k).sum(1, keepdim=True))
    return mu_v - (WR @ V - WR.sum(1, keepdim=True) * mu_v)


@pytest.mark.parametrize("mutant", [
    _grads_with_forward(_uncentred),
    _grads_with_forward(_off_by_one),
    _grads_with_forward(go.prefill_head_torch, accumulate=False),
], ids=["uncentred", "causal_off_by_one", "gqa_assigned"])
def test_grad_mutants_are_caught(mutant):
    assert not all(pin(mutant) for pin in PINS)


def test_unmutated_harness_passes():
    good = _grads_with_forward(go.prefill_head_torch)
    assert all(pin(good) for pin in PINS)
