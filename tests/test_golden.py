"""The oracle still reproduces its committed regression record (tests/golden)."""
import json
import os

import numpy as np

from tests.golden.make_golden import compute

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_block_exact_regression():
    with open(os.path.join(HERE, "tiny_block_exact.json")) as f:
        ref = json.load(f)
    got = compute()
    for key in ("out", "x1", "mod_first8"):
        np.testing.assert_allclose(np.array(got[key]), np.array(ref[key]), rtol=1e-10, atol=1e-10)
