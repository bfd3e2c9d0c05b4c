"""The oracle against its stored fixtures (tests/golden/tiny_oracle.json, written
by tests/golden/make_golden.py from oracle/ alone): bit patterns of the RoPE
outputs, INT8 codes and scales exactly, attention outputs and log-sum-exps to
1e-12 (BLAS summation order may differ between hosts). The pages print no worked
values; these fixtures only catch unintended changes of the oracle itself."""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_oracle_matches_its_fixtures():
    with open(os.path.join(HERE, "golden", "tiny_oracle.json")) as f:
        want = json.load(f)
    got = make_golden.compute()
    for key in ("rope_q_bf16_bits", "rope_k_bf16_bits", "k_codes_first_rows", "k_scales_f32_bits_first_rows",
                "v_codes_first_rows", "v_scales_f32_bits_first_rows"):
        assert got[key] == want[key], key
    for key in ("attention_out", "attention_lse"):
        a, b = np.array(got[key]), np.array(want[key])
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b))), key
