"""The oracle reproduces the fixtures ``tests/golden/make_golden.py`` wrote from it: a
regression guard, so that a change to the oracle's arithmetic is a deliberate one (the
pages print no worked numeric example; the oracle's pins are in ``test_oracle.py``)."""
import os

import numpy as np

from tests.golden import make_golden as mg

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(HERE, name)) as f:
        return [line.split() for line in f if not line.startswith("#")]


def test_tiny_qk_prep_attn_fixture():
    want = np.array([[float(v) for v in r] for r in _rows("tiny_qk_prep_attn.txt")])
    np.testing.assert_allclose(mg.tiny_qk_prep_attn(), want, rtol=1e-13, atol=1e-15)


def test_quant_row_fixture():
    rows = _rows("quant_row.txt")
    x, (codes, scales, _) = mg.quant_row()
    assert np.float32(rows[0][0]) == scales[0]
    np.testing.assert_array_equal(codes, np.array([int(c) for c in rows[1]], np.int8))
