"""CPU oracle for the MosaicQuant fused linear layer.

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by the
smoke check in ``__graft_entry__.py`` and by the CPU-baseline leg of
``bench.py``; nothing in the product path (``dense_sparse_w4a4_amd``) imports,
calls or links it, and it shares no code with the HIP kernels.

It is a plain, slow, step-by-step numpy implementation of what the method
computes, in the order the pages describe it:

  * MosaicQuant technical summary, gist.science/pt/paper/2606.15652
    (cited as [summary-pt]) - Metodologia 1 (the decomposition
    W_hat ~ Q(W_hat) + R into a dense 4-bit base and a sparse 4-bit residual),
    Metodologia 2 (block-level residual budget, Hessian-guided Delta-score,
    top-K blocks), Metodologia 3 (ZipperEngine: quantisation, dense compute,
    sparse compensation and reduce-sum in one pipeline);
  * the French page of the same summary, gist.science/fr/paper/2606.15652
    ([summary-fr]), same sections;
  * the authors' English abstract, fugumt.com/fugumt/paper_check/2606.15652v1
    ([abstract]).

Where the pages leave a step open the reading taken is stated at the function
(group size 128, symmetric codes in [-7, 7], round-half-to-even, fp16 weight
and residual scales, fp32 activation scales, the order of fp64 sums).

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
closed forms, invariants, special cases and brute force.  Parity unpinned:
whether the authors' own implementation used the same rounding and scale
conventions (the pages print no intermediate values), and the ">50% of output
distortion recovered at a 10% block budget" figure, which depends on data.
"""
from .mosaic import *  # noqa: F401,F403
