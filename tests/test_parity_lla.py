"""GPU check of the LLA oracle extension through the HIP decode path.

LLA's output is the Parallax output at the solved probe
rho* = (S_KK + lam I)^{-1} (mu_k - q). With rho* found on the host by the
oracle's conjugate gradient and handed to ``parallax_decode`` as the probe
(fp32 inputs, so the probe reaches the kernel rounded only to fp32), the GPU
output must match the oracle's Parallax output at that same fp32 probe to
the 2e-3 bar (per-row max error over max |out|), and the oracle's LLA output
to the same bar.
"""

import numpy as np
import pytest
import torch

import local_linear_attention_amd as pa
import oracle
from oracle import lla_oracle
from workloads import WORKLOADS, make_decode_inputs, replace_shape

TOL = 2e-3
pytestmark = pytest.mark.gpu


def _rel(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())


@pytest.mark.parametrize("n,d,lam", [(512, 64, 1e-3), (2048, 128, 1e-2), (4096, 128, 1e-3)])
def test_decode_at_the_lla_probe(n, d, lam):
    print(f"[lla parity] n={n} d={d} lam={lam}", flush=True)
    w = replace_shape(WORKLOADS[1], B=1, H_q=4, H_kv=4, d=d, S_max=n, scale=1.0 / np.sqrt(d))
    inp = make_decode_inputs(w, seed=21, nan_pad=False)
    H = w.H_q
    rho = torch.empty_like(inp["rho"])
    want_lla = []
    for h in range(H):
        q = inp["q"][0, h].double().numpy()
        K = inp["k_cache"][0, h].double().numpy()
        V = inp["v_cache"][0, h].double().numpy()
        out, r, it = lla_oracle.lla_attend(q, K, V, inp["scale"], lam, tol=1e-10)
        assert it > 0
        rho[0, h] = torch.from_numpy(r).to(torch.float32)
        want_lla.append(out)
    want = oracle.oracle_decode(inp["q"], rho, inp["k_cache"], inp["v_cache"],
                                inp["seq_lens"], inp["scale"])
    got = pa.decode(inp["q"].cuda(), rho.cuda(), inp["k_cache"].cuda(), inp["v_cache"].cuda(),
                    inp["seq_lens"].cuda(), inp["scale"])
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    e_par = max(_rel(got[0, h], want[0, h]) for h in range(H))
    e_lla = max(_rel(got[0, h], want_lla[h]) for h in range(H))
    print(f"   vs Parallax at the fp32 probe {e_par:.2e}, vs LLA {e_lla:.2e}", flush=True)
    assert e_par < TOL
    assert e_lla < TOL
