"""Float64 CPU oracle for the affine linear recurrence and the S6 selective scan.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or link anything in this
package. The GPU library never uses it, and this package shares no code,
header, table or helper with the GPU library.

What is computed (plain definitions, evaluated in float64 from inputs that are
widened exactly from fp32 or bf16):

* ``linear.linear_scan``: h[-1] = h0 and h[t] = a[t]*h[t-1] + b[t] for every t,
  as stated by "Selective-scan CUDA kernels" (persus.netlify.app), the
  paragraph that introduces the recurrence and its reading as a prefix scan
  over affine pairs.
* ``linear.affine_combine`` / ``linear.affine_prefix``: that same recurrence as
  a prefix over affine maps, with the earlier map on the left; the paragraph
  above stresses that the operation is associative but not commutative.
* ``s6.selective_scan``: the forward pass of the POPCORNBENCH transcript
  FW-GLM-5-1 (level 2, problem 30), problem-statement summary: dA = exp(delta*A),
  dB = delta*B, x_db = u*dB, h = dA*h + x_db per step, y_t = sum_n h*C_t, then
  y + u*D; the transcript's sequential kernel starts the state at zero. The
  reverse and bidirectional forms follow "ARM-Scan — Optimized Mamba
  Selective-Scan Kernel" (sections "Approach" and "What broke"): the reverse
  recurrence reuses the same discretized terms, and the fused result must equal
  the two independent scans.
* ``s6.softplus``: log(1 + exp(x)), which the same transcript's model applies
  to the delta projection (with its bias) before the scan; ``selective_scan``
  applies it itself when asked to (delta_softplus=True, delta_bias).
* ``native``: a plain C twin of the same loops (``oracle_c.c``) used where the
  Python loops would be too slow (full-size parity checks, the CPU baseline).

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, exact rational brute force and invariants (not against itself).
"""
from .linear import linear_scan, affine_combine, affine_prefix, apply_affine  # noqa: F401
from .s6 import selective_scan, softplus  # noqa: F401
