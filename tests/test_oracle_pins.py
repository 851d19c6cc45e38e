"""CPU pins of the oracle (no GPU): golden fixtures, exhaustive format checks,
closed forms, brute force, linearity, one-hot and integer-exact products."""
import pytest

import oracle
from oracle_pins import ALL_PINS, golden_pack_files, pin_golden_pack
import oracle_pins as P


@pytest.mark.parametrize("fname", golden_pack_files())
def test_golden_pack(fname):
    pin_golden_pack(fname)


@pytest.mark.parametrize("pin", [f for f in ALL_PINS if getattr(f, "__name__", "") != "<lambda>"],
                         ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_tolerance_covers_any_fp32_order():
    """The largest kept-term count in the workloads is 14336 (K = 28672 at
    N/M = 1/2); any fp32 summation order of that many exact products errs by at
    most gamma_{n-1} * sum|terms|, which must sit below the 2e-3 factor."""
    assert oracle.max_terms_bound(14336) < 2e-3
    assert oracle.max_terms_bound(28672 * 7 // 8) < 2e-3


def test_ulp_values():
    import numpy as np
    assert oracle.ulp(1.0, "fp16") == 2.0 ** -10
    assert oracle.ulp(0.0, "fp16") == 2.0 ** -24
    assert oracle.ulp(65504.0, "fp16") == 32.0
    assert oracle.ulp(-3.0, "fp16") == 2.0 ** -9
    assert oracle.ulp(1.0, "bf16") == 2.0 ** -7
    assert oracle.ulp(2.0 ** -127, "bf16") == 2.0 ** -133
    assert oracle.ulp(0.0, "bf16") == 2.0 ** -133
    ok, worst, _ = oracle.check(np.array([[0x3C01]], np.uint16), np.array([[1.0]]), np.array([[0.0]]), "fp16")
    assert ok and worst == 1.0
    ok, _, _ = oracle.check(np.array([[0x3C02]], np.uint16), np.array([[1.0]]), np.array([[0.0]]), "fp16")
    assert not ok
