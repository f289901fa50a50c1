"""CPU oracle of the routed-expert FP8 grouped matmul.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The HIP library and its Python binding never import it, and it
imports nothing from them: the two share no kernels, headers, helpers, tables,
constants or pre/post-processing.  Inputs come from the seeded generators in
``workloads``, which hold none of the method's arithmetic.

Modules
-------
formats   OCP e4m3fn / e5m2 decode and saturating round-to-nearest-even encode,
          bf16 rounding.
gmm       forward GMM (+SwiGLU), dequantization, dLHS and the in-kernel-quantized
          weight-gradient tgmm, each citing the page passage it restates.

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against
closed forms, a library cross-check, brute-force exact arithmetic on tiny
inputs, lossless constructions and invariants.  No pin comes from the pages'
printed numbers (the pages print no worked values for these functions).
"""
from . import formats, gmm  # noqa: F401
