"""Fused MaxSim late-interaction scoring for AMD MI355X (gfx950).

The operator lives in liblik.so (hand-written HIP kernels behind a C ABI,
declared in include/lik.h).  This package holds the thin ctypes binding
(``_lib``), the build script (``build``) and the seeded synthetic workloads
(``workloads``).
"""

from ._lib import (  # noqa: F401
    LikError,
    lik_maxsim_fwd,
    lik_maxsim_bwd,
    lik_maxsim_pairwise_fwd,
    lik_maxsim_pairwise_bwd,
    lik_maxsim_kd_fwd,
    lik_maxsim_kd_bwd,
)
