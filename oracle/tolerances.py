"""Parity bounds between the HIP path and this oracle, in one place (the GPU
tests and the smoke check both use them).

TEST INFRASTRUCTURE, like the rest of this package.

* O_ATOL: largest elementwise |O_gpu - O_ref| on the attention output.
* G_RELF: largest relative Frobenius error ||X_gpu - X_ref|| / ||X_ref|| on
  each of dq, dk, dv over the compared elements.
  (Both are the bounds stated for this path: max-abs 1e-2 on O, relative
  Frobenius 2e-2 on the gradients.)
* o_bound(ref): O is stored in bf16 (the BF16 training precision of the
  BioNeMo Recipes hub page, multi-precision training section), and storing
  even the exact O rounds it by up to half a bf16 ulp, which exceeds 1e-2
  once |O| >= 4 (an ulp there is 2^-5). The elementwise bound is therefore
  O_ATOL + ulp_bf16(ref) / 2; on inputs whose |O| stays below 2 this equals
  the literal 1e-2 plus at most 2^-8.
* LSE_ATOL: no tolerance is stated for the log-sum-exp, which the path
  returns for its own backward. Reading: with BF16 probabilities (the same
  multi-precision section) the P V product can only use bf16 values of P,
  each within a relative 2^-8 of the exact value (round to nearest even,
  8 significant bits); the invariant that each row of P sums to 1, applied
  to the P actually used, makes the softmax normaliser the sum of those
  values, whose log is then within ln(1 + 2^-8) of the exact LSE. 1e-4 more
  covers the float32 evaluation of the row maximum and the logarithm.
"""

import math

import numpy as np

O_ATOL = 1e-2
G_RELF = 2e-2
LSE_ATOL = math.log1p(2.0 ** -8) + 1e-4


def ulp_bf16(x):
    """Spacing of the bf16 grid at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def o_bound(ref):
    """Elementwise bound on |O_gpu - O_ref| (see the module docstring)."""
    return O_ATOL + 0.5 * ulp_bf16(ref)


def relf(a, b):
    """Relative Frobenius error of a against the reference b."""
    n = np.linalg.norm(b)
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / (n if n > 0 else 1.0))
