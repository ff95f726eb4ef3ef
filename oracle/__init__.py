"""Plain fp64 CPU oracle for exact additive relative-position attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers or table generators).

What it computes is the dense definition of the score in "Fast and Exact
Relative-Position Attention via Structure-Aware Kernels" (Boychev, Petrov,
Dimitrov; arXiv 2611.01182), as digested on the nanless.github.io
audio-paper-digest page, section on the score formula, Eq. (1):

    S_ij = tau * (q_i.k_j + q_i.aQ[phi(i,j)] + k_j.aK[phi(i,j)] + b[phi(i,j)]) + M_ij

followed by a row softmax and O = P V, together with the exact gradients of
O with respect to every input.  The page presents the method as exact: every
reorganisation it makes leaves the result of Eq. (1) unchanged.  So the oracle
is the definition itself: it uses none of the method's structure (no
projection windows, no tiling, no unfolding of buckets, no per-offset
storage).

Modules
-------
phi        offset maps phi: truncated (Shaw, DeBERTa as configured), T5 buckets,
           DeBERTa log buckets, identity (Transformer-XL).
attention  forward (O, LSE) and backward (dQ, dK, dV, daQ, daK, db).
dropout    attention dropout: Philox4x32-10 random bytes and the keep mask.
"""

from .phi import phi_rows, num_rows, t5_bucket, log_bucket  # noqa: F401
from .attention import forward, backward  # noqa: F401
from .dropout import philox4x32_10, random_bytes, keep_mask  # noqa: F401
