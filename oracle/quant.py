"""INT8 quantisation of cached keys and values (test infrastructure only).

The pages say only that the single-GPU preset keeps the KV cache in INT8 and
computes in BF16 ("Hy-Nomas auf einer RTX 4090", inferencekey.com, section
"Das Single-GPU-Preset"; blog.authon.dev config excerpt
``kv_cache_quantization: int8``). The granularity and rounding are readings:

* one scale per (token, head) vector of D values, separately for K and V;
* symmetric: scale s = fp32(absmax / 127), the correctly rounded fp32 quotient;
* code q = round_half_even(fp32(x / s)), clamped to [-127, 127];
* an all-zero vector has s = 0 and q = 0;
* dequantisation is q * s (exact in float64).

Why float64 division followed by a cast to float32 gives the correctly rounded
float32 quotient: both operands are float32 values, and for division double
rounding from 53 to 24 bits is innocuous because 53 >= 2*24 + 2. The tests check
this claim against exact rational arithmetic instead of assuming it.
"""

import numpy as np


def quantise(x):
    """Quantise x[..., D] (float64 holding bf16 values) along the last axis.

    Returns (q int8 [..., D], s float32 [...]).
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.max(np.abs(x), axis=-1)
    s = (m / 127.0).astype(np.float32)
    s64 = s.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)[..., None]
    r = (x / safe).astype(np.float32).astype(np.float64)
    q = np.clip(np.rint(r), -127, 127)
    q = np.where((s64 > 0)[..., None], q, 0.0)
    return q.astype(np.int8), s


def dequantise(q, s):
    """x_hat = q * s as float64 (exact)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)[..., None]
