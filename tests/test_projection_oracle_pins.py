"""Pin of the projection oracle: a pure-Python, element-by-element evaluation
of the definition (each output feature of each token is the dot product of
the token's input with that feature's weight row, features laid out as q, k,
v, rho heads) on small inputs, plus a mutant (k and v swapped) that fails."""

import numpy as np

from oracle.projection_oracle import oracle_qkvr_projection


def brute(x, w, H_q, H_kv, d):
    B, T, C = x.shape
    out = {"q": {}, "k": {}, "v": {}, "rho": {}}
    blocks = [("q", H_q), ("k", H_kv), ("v", H_kv), ("rho", H_q)]
    f = 0
    for name, H in blocks:
        for h in range(H):
            for i in range(d):
                for b in range(B):
                    for t in range(T):
                        s = 0.0
                        for cc in range(C):
                            s += float(x[b, t, cc]) * float(w[f, cc])
                        out[name][(b, h, t, i)] = s
                f += 1
    return out


def pin(fn, seed=41):
    rng = np.random.default_rng(seed)
    for B, T, C, H_q, H_kv, d in [(1, 3, 4, 2, 1, 2), (2, 5, 6, 4, 2, 3)]:
        x = rng.standard_normal((B, T, C))
        w = rng.standard_normal(((2 * H_q + 2 * H_kv) * d, C))
        got = dict(zip(("q", "k", "v", "rho"), fn(x, w, H_q, H_kv, d)))
        ref = brute(x, w, H_q, H_kv, d)
        for name in ref:
            for (b, h, t, i), val in ref[name].items():
                if abs(got[name][b, h, t, i] - val) > 1e-12 * max(1.0, abs(val)):
                    return False
    return True


def test_projection_oracle_pin():
    assert pin(oracle_qkvr_projection)


def test_projection_mutant_is_caught():
    def swapped(x, w, H_q, H_kv, d):
        q, k, v, r = oracle_qkvr_projection(x, w, H_q, H_kv, d)
        return q, v, k, r
    assert not pin(swapped)
