"""CPU oracle for bf16 RMSNorm -- TEST INFRASTRUCTURE ONLY.

Only the test suite and the benchmark may import this module; the product
library never does, and the two share no code.

What is computed (xDiT PR "LTX-2.5 optimizations: add parallel VAE decoding
and AITER RMSNorm", Changes, item 2: the transformer's block RMSNorm layers,
normalising in float32 with an optional elementwise weight): for every row r
of a (rows, dim) tensor

    y[r, j] = x[r, j] * w[j] / sqrt( (1/dim) * sum_k x[r, k]^2 + eps )

with w = 1 when there is no weight.  The inputs are the bf16 values upcast
exactly; everything here is float64.
"""
from __future__ import annotations

import numpy as np


def rms_norm(x, weight=None, eps: float = 1e-6):
    """x: (rows, dim) array-like (bf16 values as floats); weight: (dim,) or
    None.  Returns the float64 (rows, dim) result."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("x must be (rows, dim)")
    mean_sq = np.mean(x * x, axis=1, keepdims=True)
    y = x / np.sqrt(mean_sq + float(eps))
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)[None, :]
    return y
