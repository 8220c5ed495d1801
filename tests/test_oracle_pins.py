"""The CPU oracle against what the pages and the mathematics fix (see pins.py)."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import pins
from importance_aware_kv_amd import workloads as W


@pytest.mark.parametrize("check", pins.ALL, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_bf16_rounding_nearest_even():
    # 1 + 2^-8 is a tie between 0x3F80 and 0x3F81 -> even 0x3F80;
    # 1 + 3*2^-8 ties between 0x3F81 and 0x3F82 -> even 0x3F82;
    # just above a tie rounds up; signs, zero and infinity pass through.
    x = np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -2.0, 0.0, np.inf],
                 dtype=np.float32)
    assert list(W.bf16_bits(x)) == [0x3F80, 0x3F82, 0x3F81, 0xC000, 0x0000, 0x7F80]
    assert np.array_equal(W.bf16_bits_to_f32(W.bf16_bits(x)),
                          np.array([1.0, 1.0 + 2**-6, 1.0 + 2**-7, -2.0, 0.0, np.inf], np.float32))


def test_workload_budgets_headkv():
    w = W.workload("headkv32k")
    b = w.budget_array()
    assert b.shape == (4, 8) and b.min() >= 64 and b.max() <= 8192
    assert np.all(b == b[0])                      # one draw shared across the batch
    assert abs(int(b[0].sum()) - 16384) < 2048    # clamping perturbs the total a little


def test_oracle_sanitized_selftest():
    """Build the oracle with ASan+UBSan into a native self-test and run it."""
    from oracle import build as ob
    with tempfile.TemporaryDirectory() as d:
        exe = ob.build_selftest(d)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        assert "selftest ok" in r.stdout
