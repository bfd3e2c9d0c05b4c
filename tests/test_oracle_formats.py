"""Pins of oracle/formats.py against a library routine and brute force."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats


def _torch_bf16(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def test_to_bf16_matches_torch_on_float32_patterns():
    # every kind of float32: random bit patterns (incl. subnormals, huge values),
    # exact ties (low 16 bits 0x8000) and values next to ties
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, size=20_000).astype(np.uint32) << 16) | 0x8000
    near = np.concatenate([ties - 1, ties + 1])
    allbits = np.concatenate([bits, ties, near]).astype(np.uint32)
    x32 = allbits.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    ref = _torch_bf16(x32)
    got = formats.to_bf16(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_to_bf16_single_rounding_from_float64_brute_force():
    # values with more than 24 significant bits: compare with the nearest bf16
    # found among neighbouring bf16 patterns by exact rational distances
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-130, 120, 3000))
    got = formats.to_bf16(x)
    for xi, gi in zip(x, got):
        base = int((np.float32(xi).view(np.uint32) >> 16))
        cands = []
        for b in range(base - 3, base + 4):
            b &= 0xFFFF
            val = float(formats.from_bf16_bits(np.array([b], np.uint16))[0])
            if np.isfinite(val):
                cands.append((abs(Fraction(val) - Fraction(float(xi))), (b & 1), val))
        cands.sort(key=lambda c: (c[0], c[1]))   # nearest; on a tie the even pattern
        assert gi == cands[0][2], (xi, gi, cands[:2])


def test_bf16_bits_roundtrip_and_rejects_inexact():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2**16, 10000).astype(np.uint16)
    v = formats.from_bf16_bits(u)
    ok = np.isfinite(v)
    assert np.array_equal(formats.bf16_bits(v[ok]), u[ok])
    with pytest.raises(ValueError):
        formats.bf16_bits(np.array([1.0 + 2.0 ** -10]))


def test_bf16_ulp_examples():
    assert formats.bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert formats.bf16_ulp(np.array([1.5]))[0] == 2.0 ** -7
    assert formats.bf16_ulp(np.array([2.0]))[0] == 2.0 ** -6
    assert formats.bf16_ulp(np.array([0.75]))[0] == 2.0 ** -8
    assert formats.bf16_ulp(np.array([2.0 ** -130]))[0] == 2.0 ** -133
