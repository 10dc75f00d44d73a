"""The oracle still reproduces its committed regression records (tests/golden)."""
import json
import os

import numpy as np
import pytest

from tests.golden.make_golden import compute

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("mode", ["exact", "contract"])
def test_tiny_block_regression(mode):
    with open(os.path.join(HERE, f"tiny_block_{mode}.json")) as f:
        ref = json.load(f)
    got = compute(mode)
    keys = ("out", "x1", "mod_first8") + (("h1", "o", "h2", "u") if mode == "contract" else ())
    for key in keys:
        np.testing.assert_allclose(np.array(got[key]), np.array(ref[key]), rtol=1e-10, atol=1e-10,
                                   err_msg=key)
