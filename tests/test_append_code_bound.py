"""CPU check of the numerical argument behind the INT8 append kernel's fast path.

The kernel forms the code of x (scale s = fp32(m / 127)) from the exact product
x * r with r = rcp(s), within one ulp of 1/s: f = fma(x, r, 1.5 * 2^23) rounds
x * r to an integer k (nearest, ties to even), and d = fma(x, r, -k) is the
distance of x * r from it. Only when |d| <= 1/2 - 2^-14 does it keep k; the
rest go to the IEEE quotient. The claim: every kept k equals the quantiser's
code RNE(fp32(x / s)) (oracle/quant.py). This test emulates those two fma
steps exactly (x * r is exact in float64: 8 + 24 significant bits) for every
bf16 x with |x| <= m, for reciprocals at and one ulp either side of 1/s, over
absmax values m that include the quantiser's tie cases, and checks the claim
and that the fallback stays rare. It checks the argument, not the GPU (the GPU
tests compare the kernel's bytes with the oracle)."""

import numpy as np
import pytest

from oracle import quant

C = np.float64(1.5 * 2 ** 23)
NEAR = 0.5 - 2.0 ** -14


def _bf16_values_upto(m):
    """All finite bf16 values x with 0 <= x <= m, as float64."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    v = bits.view(np.float32).astype(np.float64)
    return v[v <= m]


# absmax values (bf16 patterns): unit range, the x = m/2 tie cases of the
# quantiser pins, the outlier range, tiny normal values, and a spread
M_BITS = [0x3F80, 0x3F96, 0x3FB4, 0x3A8F, 0x4080, 0x42A0, 0x42A8, 0x0081, 0x1000, 0x7F00, 0x3FFF, 0x4049,
          0x40B6, 0x3E4D, 0x4170, 0x3C23]


@pytest.mark.parametrize("mbits", M_BITS, ids=hex)
def test_kept_codes_equal_the_quantiser(mbits):
    m = float(np.array([mbits << 16], np.uint32).view(np.float32)[0])
    s = np.float32(m / 127.0)
    if s < np.float32(2.0 ** -120):
        pytest.skip("scales below 2^-120 always take the IEEE quotient")
    xs = _bf16_values_upto(m)
    xs = np.concatenate([xs, -xs])
    # oracle codes: vectors [m, x] have absmax m
    vec = np.stack([np.full_like(xs, m), xs], axis=1)
    q_ref, s_ref = quant.quantise(vec)
    assert np.all(s_ref == s)
    ref = q_ref[:, 1].astype(np.int64)
    r0 = np.float32(1.0) / s          # float32 division: correctly rounded
    kept_total = 0
    for r in (np.nextafter(r0, np.float32(0)), r0, np.nextafter(r0, np.float32(np.inf))):
        p = xs * np.float64(r)          # exact
        k = np.rint(p)                  # fma(x, r, C) - C: p rounded to an integer, ties to even
        d = (p - k).astype(np.float32)  # fma(x, r, -k): one rounding of an exact float64 value
        keep = np.abs(d) <= NEAR
        assert np.array_equal(k[keep].astype(np.int64), ref[keep]), \
            f"m={m!r} r={r!r}: a kept code differs from the quantiser's"
        # the fallback is rare (about 2 * 2^-14 of uniformly spread quotients)
        assert np.mean(~keep) < 2e-3
        kept_total += keep.sum()
    assert kept_total > 0
