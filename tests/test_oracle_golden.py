"""The oracle still reproduces its committed regression fingerprint (CPU only)."""
import json
import os

import numpy as np
import pytest

from golden.make_golden import CASES, fingerprint

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("name", sorted(CASES))
def test_oracle_fingerprint_unchanged(name):
    with open(os.path.join(HERE, "golden", "oracle_tiny_fingerprint.json")) as f:
        want = json.load(f)[name]
    got = fingerprint(CASES[name])
    for key in ("row_sums", "samples", "lse"):
        np.testing.assert_allclose(got[key], want[key], rtol=0, atol=1e-12)
