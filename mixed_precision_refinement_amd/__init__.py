"""msolve: repeated dense complex-symmetric solves Z(w) x = b to double
precision on an AMD Instinct MI355X (gfx950) -- single-precision LU plus
double-precision iterative refinement, in hand-written HIP kernels behind a
C-ABI library (include/msolve.h).

``from mixed_precision_refinement_amd import msolve`` loads libmsolve.so and
fails if it has not been built (``python mixed_precision_refinement_amd/build.py``).
"""

__all__ = ["msolve"]
