"""Plain fp64 CPU oracle for the Parallax forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark do. The product path (the HIP library and its Python binding)
shares no code, constants or helpers with it, and it imports nothing from the
product package.

Sources the oracle follows (page titles and sections):

* "Parallax: Breaking the Boundary Bias with Parameterized Local Linear
  Attention" (explainer blog post), section "The Core Insight: Covariance
  Correction", the output equation: the output is the softmax-attention output
  minus the key/value covariance applied to a probe vector rho, and rho is a
  learned projection of the input.
* "Parallax: Parameterized Local Linear Attention for Language Modeling"
  (paper detail page), "Abstract": rho acts like a second query, dotted with
  the keys, and selects which direction of the key/value covariance corrects
  the output; softmax attention is the local-constant (Nadaraya-Watson)
  estimate that local linear attention improves on.
* Same blog post, section "Context: Why 'Softmax' is Not Enough": softmax
  attention is a Nadaraya-Watson estimator (local constant).

The pages do not define the covariance's orientation, centring or weights, the
softmax scale, GQA, masking or shapes. The readings taken are stated next to
each function and listed, with reasons, in the repository's design notes.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
something other than itself (a library routine, brute force, a closed form,
an exact worked example, invariants, and the textbook local-linear
regression it reduces to). No function is "parity unpinned".

``lla_oracle`` adds the solver-based Local Linear Attention that Parallax
replaces (conjugate gradient for the probe), pinned in
``tests/test_lla_oracle_pins.py``; ``lla_contrast`` measures its accuracy and
cost against softmax attention on synthetic data. ``parallax_grad_oracle``
gives the gradients of the causal prefill (fp64 autograd of the explicit
definition), pinned in ``tests/test_grad_oracle_pins.py``; ``projection_oracle``
gives the fused q, k, v, rho projection, pinned in
``tests/test_projection_oracle_pins.py``.
"""

from .parallax_oracle import (  # noqa: F401
    softmax_weights,
    sigma_kv,
    parallax_attend,
    oracle_decode,
    oracle_decode_heads,
    oracle_prefill_rows,
    oracle_prefill_full,
    oracle_chunk_rows,
    oracle_chunk_full,
)
from .parallax_grad_oracle import oracle_prefill_grads  # noqa: F401
from .projection_oracle import oracle_qkvr_projection  # noqa: F401
