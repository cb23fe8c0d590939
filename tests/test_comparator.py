"""The parity comparator itself (no GPU): a defect confined to a few rows of
one chunk-head -- the kind a normwise bound over a whole tensor cannot see --
must fail the element-wise bounds, while rounding of every element to bf16
passes them."""
import numpy as np

from tests import gdr_cases as gc


def _bf16(x):
    # round-to-nearest-even to 8 significant bits (bf16), in float64
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def test_localized_defect_fails_the_row_bound_but_not_the_normwise_one():
    rng = np.random.default_rng(7)
    y = rng.standard_normal((1, 1024, 4, 128))          # an output like dv: [B, T, H, D]
    x = _bf16(y)
    lim = gc.ROW_TOL["bf16"]["dv"]
    assert gc.rel(x, y) < 2e-3
    assert gc.rel_row(x, y, "dv") < 1.5e-2 < lim
    bad = x.copy()
    bad[0, 3 * 64 + 48:3 * 64 + 64, 1, :16] += 0.2      # rows 48-63 of chunk 3, head 1, 16 columns
    assert gc.rel(bad, y) < gc.TOL["bf16"]              # invisible to the normwise bound
    assert gc.rel_row(bad, y, "dv") > lim               # caught by the row bound
    small = x.copy()
    small[0, 3 * 64 + 48:3 * 64 + 64, 1, :16] += 0.05   # a quarter of that is below it
    assert gc.rel_row(small, y, "dv") < lim


def test_scalar_outputs_use_64_token_rows():
    rng = np.random.default_rng(8)
    y = rng.standard_normal((2, 300, 3))                # dbeta: [B, T, H]
    x = _bf16(y)
    assert gc.rel_row(x, y, "dbeta") < 1.5e-2
    bad = x.copy()
    bad[1, 64 + 48:64 + 64, 2] += 0.3                   # 16 tokens of one chunk of one head
    assert gc.rel(bad, y) < 3e-2
    assert gc.rel_row(bad, y, "dbeta") > 0.1
    rows = gc._rows("dbeta", y)
    assert rows.shape == (2 * 3 * 5, 64)                # 300 tokens -> 5 blocks (zero-padded)


def test_near_zero_rows_are_measured_against_the_rms_floor():
    y = np.ones((10, 8))
    y[3] = 1e-9
    x = y.copy()
    x[3] += 1e-6                                        # tiny absolute error on a near-zero row
    assert gc.rel_row(x, y, "o") < 2e-5
