"""CPU fp64 oracle for sparse-linear attention (test infrastructure only).

This package is the checker, not the product.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the HIP library and
its Python binding never do, and the oracle never imports them.  It shares no
code with the GPU path: the only thing both sides consume is the seeded input
tensors from the ``workloads`` package.

Sources (page titles as printed; sections as on each page):

* SLA abstract ("SLA: Beyond Sparsity in Diffusion Transformers via
  Fine-Tunable Sparse-Linear Attention"): attention weights are split into
  critical (exact O(N^2) attention), marginal (O(N) linear attention) and
  negligible (skipped) parts, fused in one kernel.
* SLA2 technical summary, section 2.A: the output mixes the two branches per
  the equation O = alpha * O_s + (1 - alpha) * O_l.
* SLA2 technical summary, section 1 item 1: the sparse branch renormalises
  its softmax over the kept keys.
* SLA2 technical summary, section 2.B: the router sees only Q and K, pools
  adjacent tokens and uses a hard top-k at inference.
* PISA technical summary, "Algoritmo Central" and "Enrutamiento Consciente
  de la Covarianza": per-block first-order matrices H_j built from keys and
  values.
* SPLA technical summary, section 2.2: unselected blocks are compressed into
  a compact linear-attention state; section 2.3: a parameter-free
  exponential feature map.

Residual linear attention (SPLA technical summary, sections 2.2 and 2.3:
o_rla = o_bar - o_tilde over all and over the selected blocks, an RMS norm on
that branch, a gated sum, an exponential feature map) is in ``oracle.rla``.
The second-order block routing score (SPLA technical summary, section 2.1)
is in ``oracle.taylor``.  Piecewise exact-or-approximate attention (PISA
technical summary, section 2: exact terms on the selected blocks, a
zero-order centroid term per unselected block and one global first-order
correction inside a single softmax numerator and denominator) is in
``oracle.pisa``.

The block size (64), mean pooling, phi = softmax over the feature dimension,
H_j = phi(K_j)^T V_j, z_j = column sums of phi(K_j), and the per-head alpha
are the plain readings this build fixes where the pages leave the step open.

Every public function carries a "pinned by" note naming the tests that tie it
to something other than itself.  Functions with no such pin would say
"parity unpinned"; at present every function here is pinned.
"""
from . import sla, fp8  # noqa: F401
