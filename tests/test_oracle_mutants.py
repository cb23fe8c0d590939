"""Planted mistakes in a copy of the oracle must be caught by its pins (CPU).

Each case copies ``oracle/gdr_oracle.c``, applies one plausible slip (a dropped
term, a flipped sign, a wrong operand), compiles the copy into a temporary
library and runs the pins of ``test_oracle.py`` that are cheap (the worked
example, the chunk-wise form, finite differences) against it.  At least one
must fail for every mutant; the unmodified source must pass them all.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

MUTANTS = {
    "forward_decay_dropped": ("Si[j] *= a;                 /* R1 */", "/* R1 dropped */"),
    "forward_delta_sign": ("d[i] = bt * (vt[i] - acc);    /* R3 */", "d[i] = bt * (vt[i] + acc);"),
    "forward_beta_dropped": ("d[i] = bt * (vt[i] - acc);    /* R3 */", "d[i] = (vt[i] - acc);"),
    "output_uses_key": ("acc += Si[j] * qt[j];", "acc += Si[j] * kt[j];"),
    "dq_uses_previous_state": ("acc += Snow[(size_t)i * DK + j] * dot[i];",
                               "acc += Sprev[(size_t)i * DK + j] * dot[i];"),
    "dk_erase_term_dropped": ("dk[th * DK + j] += acc;", "(void)acc;"),
    "dbeta_sign": ("db += dd[i] * (vt[i] - p[i]);", "db += dd[i] * (vt[i] + p[i]);"),
    "dg_before_erase_gradient": ("gg += dS[e] * St[e];", "gg += dS[e] * Sprev[e];"),
    "state_grad_not_decayed": ("for (size_t e = 0; e < SS; ++e) dS[e] *= a;", "(void)a;"),
    "dp_sign": ("dp[i] = -bt * dd[i];", "dp[i] = bt * dd[i];"),
}


def _build(text, tmpdir, name):
    c = os.path.join(tmpdir, name + ".c")
    so = os.path.join(tmpdir, name + ".so")
    with open(c, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so, c,
                           "-lm"])
    return oracle.load_variant(so)


def _pins_pass(lib):
    """Run cheap pins against `lib`; return the list of failed pin names."""
    failed = []
    gd, (q, k, v, beta, g, h0, do, dhT) = pins._golden()
    ex = gd["expected"]
    o, hT = oracle.fwd(q, k, v, beta, g, h0=h0, scale=1.0, layout="VK", lib=lib)
    if not (np.allclose(o.reshape(2, 2), ex["o"], atol=1e-12)
            and np.allclose(hT.reshape(2, 2), ex["hT"], atol=1e-12)):
        failed.append("golden_forward")
    r = oracle.bwd(q, k, v, beta, g, do, h0=h0, dhT=dhT, scale=1.0, layout="VK", lib=lib)
    ok = all(np.allclose(r[n].reshape(np.shape(ex[n])), ex[n], atol=1e-12)
             for n in ("dq", "dk", "dv", "dbeta", "dg", "dh0"))
    if not ok:
        failed.append("golden_backward")
    rng = np.random.default_rng(1)
    q, k, v, beta, g, _ = pins.rand_case(rng, B=1, T=70, H=1, DK=5, DV=4)
    o1, h1 = oracle.fwd(q, k, v, beta, g, layout="VK", lib=lib)
    o2, h2 = oracle.chunk_fwd(q, k, v, beta, g, layout="VK", chunk=16)
    if not (pins.rel(o1, o2) < 1e-12 and pins.rel(h1, h2) < 1e-12):
        failed.append("chunked_form")
    q, k, v, beta, g, _ = pins.rand_case(rng, B=1, T=4, H=1, DK=3, DV=3)
    h0 = rng.standard_normal((1, 1, 3, 3))
    do = rng.standard_normal(v.shape)
    dhT = rng.standard_normal((1, 1, 3, 3))
    r = oracle.bwd(q, k, v, beta, g, do, h0=h0, dhT=dhT, layout="VK", lib=lib)
    args = dict(q=q, k=k, v=v, beta=beta, g=g, h0=h0)
    grads = dict(q="dq", k="dk", v="dv", beta="dbeta", g="dg", h0="dh0")
    eps = 1e-6
    for name, x in args.items():
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = {kk: vv.copy() for kk, vv in args.items()}
            xm = {kk: vv.copy() for kk, vv in args.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fp = oracle.fwd(xp["q"], xp["k"], xp["v"], xp["beta"], xp["g"], h0=xp["h0"],
                            layout="VK", lib=lib)
            fm = oracle.fwd(xm["q"], xm["k"], xm["v"], xm["beta"], xm["g"], h0=xm["h0"],
                            layout="VK", lib=lib)
            num[idx] = ((np.sum(fp[0] * do) + np.sum(fp[1] * dhT))
                        - (np.sum(fm[0] * do) + np.sum(fm[1] * dhT))) / (2 * eps)
        if not pins.rel(r[grads[name]], num) < 1e-6:
            failed.append("fd_" + name)
    return failed


@pytest.fixture(scope="module")
def tmpdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


def test_unmodified_source_passes(tmpdir):
    with open(SRC) as f:
        text = f.read()
    assert _pins_pass(_build(text, tmpdir, "orig")) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmpdir):
    with open(SRC) as f:
        text = f.read()
    old, new = MUTANTS[name]
    assert text.count(old) == 1, "mutation site not found exactly once: " + old
    lib = _build(text.replace(old, new), tmpdir, name)
    failed = _pins_pass(lib)
    assert failed, "planted mistake %s was not caught by any pin" % name
