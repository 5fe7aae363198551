"""A seeded sweep of random small chunk steps (tests/fuzz_cases.py) through the
C ABI on the GPU, every output element against the fp64 oracle under the
official bars (parity.py): selection, O, LSE, dQ, dK, dV, and untouched pool
slots bitwise unchanged."""
import json

import pytest

import fuzz_cases
import gpu_harness as H

pytestmark = pytest.mark.gpu

CASES = fuzz_cases.cases()


@pytest.mark.parametrize("i", range(len(CASES)))
def test_fuzz_case(ora, i):
    seed, p = CASES[i]
    H.say(f"fuzz case {i} (seed {seed}): {p}")
    report, *_ = H.run_full(p, seed, ora)
    H.say(f"  {json.dumps(report, default=float)}")
