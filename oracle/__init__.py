"""CPU oracle for fused MaxSim late-interaction scoring.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
reference that the GPU library is checked against.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the library
under ``maxsim_scoring_02_amd`` never does, and this package imports nothing
from the library.

Sources (the pages, cited by title and section):

* "Late Interaction Kernels" README (Hugging Face Kernels package
  sentence-transformers/late-interaction-kernels), sections *What does it
  compute?*, *Scoring interface*, *Precision and compatibility*.
* Social thread announcing late-interaction-kernels, posts (2/N), (4/N), (5/N).
* colpali pull request "Add support for late-interaction-kernels (LIK)",
  sections *What this PR adds* and *Results*.

Modules:

* ``maxsim``  numpy float64 forward/backward for the all-pairs, pairwise and
  kd (per-query candidate) layouts, with tie information for parity checks.
* ``brute``   pure-Python loops with ``math.fsum``, for tiny inputs only; it
  pins ``maxsim`` independently of numpy's matmul.
* ``loss``    float64 row cross-entropy over a score matrix (the loss head
  the colpali pull request puts on the scores), with its gradient.

Every function here is pinned by the ``-m "not gpu"`` tests (brute force,
closed forms, finite differences, invariants, integer-exact inputs); none is
"parity unpinned".
"""

from .maxsim import (  # noqa: F401
    EMPTY_DOC_SCORE,
    TIE_GAP,
    ForwardResult,
    maxsim_allpairs,
    maxsim_allpairs_bwd,
    maxsim_pairwise,
    maxsim_pairwise_bwd,
    maxsim_kd,
    maxsim_kd_bwd,
    token_similarity,
    admissible_argmax,
    maxsim_block,
    scores_as_float32,
)
from .loss import ce_rows  # noqa: F401
from . import brute  # noqa: F401
