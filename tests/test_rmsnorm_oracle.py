"""Pins of the fp64 RMSNorm-backward oracle to facts outside itself (CPU
only): a two-row example worked by hand, central finite differences of both
gradients, the scale invariance of RMSNorm at eps = 0, the row-sum identity
of dw, a closed form, and agreement of the vectorised and the scalar-loop
formulations.  Planted mistakes (a dropped term, sum for mean, x for xhat, a
wrong power of r) must each fail a pin."""
import json
import os

import numpy as np
import pytest

from oracle import rmsnorm_oracle as ro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rmsnorm_bwd_handworked.json")


def rel(x, y):
    x, y = np.asarray(x, dtype=np.float64), np.asarray(y, dtype=np.float64)
    n = np.linalg.norm(y.ravel())
    d = np.linalg.norm((x - y).ravel())
    return d / n if n > 0 else d


def case(rng, M=3, N=5):
    x = rng.standard_normal((M, N))
    w = 1.0 + 0.3 * rng.standard_normal(N)
    dy = rng.standard_normal((M, N))
    return x, w, dy


def test_handworked_example():
    gd = json.load(open(GOLDEN))
    x = np.array(gd["inputs"]["x"], float)
    w = np.array(gd["inputs"]["w"], float)
    dy = np.array(gd["inputs"]["dy"], float)
    exp = gd["expected"]
    np.testing.assert_allclose(ro.rstd(x, 0.0), exp["rstd"], rtol=1e-15)
    for fn in (ro.backward, ro.backward_rows):
        dx, dw = fn(x, w, dy, eps=0.0)
        np.testing.assert_allclose(dx, exp["dx"], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(dw, exp["dw"], rtol=1e-14)


def loss(x, w, dy, eps):
    y, _ = ro.forward(x, w, eps)
    return float((y * dy).sum())


def fd_check(backward, eps=1e-3, seed=0, h=1e-6):
    """max relative error of backward's (dx, dw) against central differences"""
    rng = np.random.default_rng(seed)
    x, w, dy = case(rng)
    dx, dw = backward(x, w, dy, eps=eps)
    ndx = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        ndx[i] = (loss(xp, w, dy, eps) - loss(xm, w, dy, eps)) / (2 * h)
    ndw = np.zeros_like(w)
    for j in range(w.size):
        wp, wm = w.copy(), w.copy()
        wp[j] += h
        wm[j] -= h
        ndw[j] = (loss(x, wp, dy, eps) - loss(x, wm, dy, eps)) / (2 * h)
    return max(rel(dx, ndx), rel(dw, ndw))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_central_finite_differences(seed):
    assert fd_check(ro.backward, seed=seed) < 1e-7
    assert fd_check(ro.backward_rows, seed=seed) < 1e-7


def test_scale_invariance_at_zero_eps():
    # y(a x) = y(x) for a > 0 when eps = 0, so the gradient is orthogonal to x
    rng = np.random.default_rng(3)
    x, w, dy = case(rng, M=6, N=9)
    dx, _ = ro.backward(x, w, dy, eps=0.0)
    dots = (dx * x).sum(axis=1)
    assert np.abs(dots).max() < 1e-13 * np.abs(x).max() * np.abs(dx).max() * 9


def test_dw_is_the_sum_of_per_row_contributions():
    rng = np.random.default_rng(4)
    x, w, dy = case(rng, M=7, N=4)
    _, dw = ro.backward(x, w, dy, eps=1e-5)
    parts = [ro.backward(x[m:m + 1], w, dy[m:m + 1], eps=1e-5)[1] for m in range(7)]
    np.testing.assert_allclose(dw, np.sum(parts, axis=0), rtol=1e-14)


def test_cotangent_along_the_output_gives_zero_dx():
    # w = 1, eps = 0, dy = y: <dy, y> = |y|^2 = N whatever x is, so dx = 0
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 6))
    w = np.ones(6)
    y, _ = ro.forward(x, w, 0.0)
    dx, dw = ro.backward(x, w, y, eps=0.0)
    assert np.abs(dx).max() < 1e-14
    np.testing.assert_allclose(dw, (y * y).sum(axis=0), rtol=1e-14)


def test_vectorised_and_loop_forms_agree_and_given_rstd_is_used():
    rng = np.random.default_rng(6)
    x, w, dy = case(rng, M=7, N=13)
    a = ro.backward(x, w, dy, eps=1e-4)
    b = ro.backward_rows(x, w, dy, eps=1e-4)
    c = ro.backward(x, w, dy, r=ro.rstd(x, 1e-4))
    for u, v, z in zip(a, b, c):
        assert rel(u, v) < 1e-13
        np.testing.assert_array_equal(u, z)


# planted mistakes: each variant of the backward must fail a pin above
def _dropped_mean_term(x, w, dy, r=None, eps=0.0):
    r = ro.rstd(x, eps) if r is None else r
    xh = x * r[:, None]
    return r[:, None] * (w[None, :] * dy), (dy * xh).sum(axis=0)


def _sum_for_mean(x, w, dy, r=None, eps=0.0):
    r = ro.rstd(x, eps) if r is None else r
    xh = x * r[:, None]
    wdy = w[None, :] * dy
    c = (wdy * xh).sum(axis=1)
    return r[:, None] * (wdy - xh * c[:, None]), (dy * xh).sum(axis=0)


def _x_for_xhat_in_dw(x, w, dy, r=None, eps=0.0):
    dx, _ = ro.backward(x, w, dy, r=r, eps=eps)
    return dx, (dy * x).sum(axis=0)


def _r_squared(x, w, dy, r=None, eps=0.0):
    r = ro.rstd(x, eps) if r is None else r
    xh = x * r[:, None]
    wdy = w[None, :] * dy
    c = (wdy * xh).sum(axis=1) / x.shape[1]
    return (r * r)[:, None] * (wdy - xh * c[:, None]), (dy * xh).sum(axis=0)


@pytest.mark.parametrize("mutant", [_dropped_mean_term, _sum_for_mean, _x_for_xhat_in_dw, _r_squared])
def test_planted_mistakes_are_caught(mutant):
    assert fd_check(mutant) > 1e-3
