"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against something the recurrence or mathematics
fixes independently of the oracle's own code: a worked example in exact
arithmetic, the chunk-wise form of the same forward, closed forms in special
cases, invariants, and central finite differences for every gradient.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(x, y):
    x, y = np.asarray(x, dtype=np.float64), np.asarray(y, dtype=np.float64)
    d = np.linalg.norm((x - y).ravel())
    n = np.linalg.norm(y.ravel())
    return d / n if n > 0 else d


def rand_case(rng, B=1, T=8, H=1, DK=4, DV=4, unit_k=True, g_mean=0.0, lengths=None):
    if lengths is not None:
        B, T = 1, int(sum(lengths))
    q = rng.standard_normal((B, T, H, DK))
    k = rng.standard_normal((B, T, H, DK))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, DV))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    g = -np.log1p(np.exp(-(rng.standard_normal((B, T, H)) + g_mean)))
    cu = None
    if lengths is not None:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, k, v, beta, g, cu


# --------------------------------------------------------------------------
# worked example (exact rational arithmetic, derived by hand)


def _golden():
    with open(os.path.join(GOLDEN, "handworked_T2_D2.json")) as f:
        gd = json.load(f)
    inp = gd["inputs"]
    q = np.array(inp["q"], float).reshape(1, 2, 1, 2)
    k = np.array(inp["k"], float).reshape(1, 2, 1, 2)
    v = np.array(inp["v"], float).reshape(1, 2, 1, 2)
    beta = np.array(inp["beta"], float).reshape(1, 2, 1)
    g = np.array([0.0, np.log(0.5)]).reshape(1, 2, 1)
    h0 = np.array(inp["h0"], float).reshape(1, 1, 2, 2)
    do = np.array(inp["dO"], float).reshape(1, 2, 1, 2)
    dhT = np.array(inp["dhT"], float).reshape(1, 1, 2, 2)
    return gd, (q, k, v, beta, g, h0, do, dhT)


def test_golden_forward():
    gd, (q, k, v, beta, g, h0, do, dhT) = _golden()
    o, hT = oracle.fwd(q, k, v, beta, g, h0=h0, scale=gd["scale"], layout="VK")
    ex = gd["expected"]
    np.testing.assert_allclose(o.reshape(2, 2), ex["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hT.reshape(2, 2), ex["hT"], rtol=0, atol=1e-14)


def test_golden_backward():
    gd, (q, k, v, beta, g, h0, do, dhT) = _golden()
    r = oracle.bwd(q, k, v, beta, g, do, h0=h0, dhT=dhT, scale=gd["scale"], layout="VK")
    ex = gd["expected"]
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(r[name].reshape(2, 2), ex[name], rtol=0, atol=1e-14, err_msg=name)
    for name in ("dbeta", "dg"):
        np.testing.assert_allclose(r[name].reshape(2), ex[name], rtol=0, atol=1e-14, err_msg=name)
    np.testing.assert_allclose(r["dh0"].reshape(2, 2), ex["dh0"], rtol=0, atol=1e-14)


def test_golden_kv_layout_is_transpose():
    gd, (q, k, v, beta, g, h0, do, dhT) = _golden()
    o, hT = oracle.fwd(q, k, v, beta, g, h0=np.swapaxes(h0, -1, -2).copy(), scale=1.0, layout="KV")
    np.testing.assert_allclose(hT.reshape(2, 2), np.array(gd["expected"]["hT"]).T, atol=1e-14)
    np.testing.assert_allclose(o.reshape(2, 2), gd["expected"]["o"], atol=1e-14)


# --------------------------------------------------------------------------
# chunk-wise form == per-token form (two independent formulations)


@pytest.mark.parametrize("chunk", [4, 5, 64])
@pytest.mark.parametrize("layout", ["KV", "VK"])
def test_chunked_equals_recurrent_fixed(chunk, layout):
    rng = np.random.default_rng(10 + chunk)
    q, k, v, beta, g, _ = rand_case(rng, B=2, T=150, H=2, DK=8, DV=6)
    h0 = 0.1 * rng.standard_normal((2, 2, 8, 6) if layout == "KV" else (2, 2, 6, 8))
    o1, h1 = oracle.fwd(q, k, v, beta, g, h0=h0, layout=layout)
    o2, h2 = oracle.chunk_fwd(q, k, v, beta, g, h0=h0, layout=layout, chunk=chunk)
    assert rel(o2, o1) < 1e-12
    assert rel(h2, h1) < 1e-12


@pytest.mark.parametrize("chunk", [4, 64])
def test_chunked_equals_recurrent_varlen(chunk):
    rng = np.random.default_rng(3)
    lengths = [70, 0, 1, 64, 129]
    q, k, v, beta, g, cu = rand_case(rng, H=3, DK=5, DV=7, lengths=lengths)
    h0 = 0.1 * rng.standard_normal((len(lengths), 3, 7, 5))
    o1, h1 = oracle.fwd(q, k, v, beta, g, cu_seqlens=cu, h0=h0, layout="VK")
    o2, h2 = oracle.chunk_fwd(q, k, v, beta, g, cu_seqlens=cu, h0=h0, layout="VK", chunk=chunk)
    assert rel(o2, o1) < 1e-12
    assert rel(h2, h1) < 1e-12
    # zero-length sequence: the final state is the initial state
    np.testing.assert_array_equal(h1[1], h0[1])


# --------------------------------------------------------------------------
# invariants and closed forms


def test_beta0_g0_output_is_initial_state_readout():
    rng = np.random.default_rng(4)
    q, k, v, beta, g, _ = rand_case(rng, B=1, T=20, H=2, DK=6, DV=5)
    h0 = rng.standard_normal((1, 2, 5, 6))
    scale = 0.37
    o, hT = oracle.fwd(q, k, v, 0 * beta, 0 * g, h0=h0, scale=scale, layout="VK")
    ref = scale * np.einsum("hij,bthj->bthi", h0[0], q)
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(hT, h0, rtol=0, atol=0)


def test_unit_key_beta1_stores_value():
    # beta_t = 1 with |k_t| = 1 makes the state map k_t to v_t exactly, for any
    # decay (the erase term removes the old association along k_t).
    rng = np.random.default_rng(5)
    for T in range(1, 7):
        q, k, v, beta, g, _ = rand_case(rng, B=1, T=T, H=1, DK=6, DV=4)
        beta[:, -1] = 1.0
        g = rng.standard_normal(g.shape) * 2.0  # any sign
        h0 = rng.standard_normal((1, 1, 4, 6))
        _, hT = oracle.fwd(q, k, v, beta, g, h0=h0, layout="VK")
        np.testing.assert_allclose(hT[0, 0] @ k[0, -1, 0], v[0, -1, 0], rtol=1e-12, atol=1e-12)


def test_full_decay_resets_state():
    # exp(-1e4) underflows to exactly 0, so S_t = beta_t v_t k_t^T and nothing
    # before t can reach any later output.
    rng = np.random.default_rng(6)
    q, k, v, beta, g, _ = rand_case(rng, B=1, T=12, H=1, DK=5, DV=3)
    g[0, 6, 0] = -1e4
    h0 = rng.standard_normal((1, 1, 3, 5))
    o1, h1 = oracle.fwd(q, k, v, beta, g, h0=h0, layout="VK")
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, :6] += 1.0
    k2[:, :6] = rng.standard_normal(k2[:, :6].shape)
    v2[:, :6] *= -3.0
    o2, h2 = oracle.fwd(q2, k2, v2, beta, g, h0=2 * h0, layout="VK")
    np.testing.assert_allclose(o1[:, 6:], o2[:, 6:], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(h1, h2, rtol=1e-13, atol=1e-13)
    # the state right after the reset token
    _, h6 = oracle.fwd(q[:, :7], k[:, :7], v[:, :7], beta[:, :7], g[:, :7], h0=h0, layout="VK")
    ref = beta[0, 6, 0] * np.outer(v[0, 6, 0], k[0, 6, 0])
    np.testing.assert_allclose(h6[0, 0], ref, rtol=1e-13, atol=1e-14)


def test_single_token_product_form():
    # S_1 = a S_0 (I - b k k^T) + b v k^T, written as a product (the oracle
    # evaluates the expanded delta form).
    rng = np.random.default_rng(7)
    q, k, v, beta, g, _ = rand_case(rng, B=1, T=1, H=1, DK=5, DV=4, unit_k=False)
    h0 = rng.standard_normal((1, 1, 4, 5))
    o, hT = oracle.fwd(q, k, v, beta, g, h0=h0, scale=0.8, layout="VK")
    a, b = np.exp(g[0, 0, 0]), beta[0, 0, 0]
    kk, vv, qq = k[0, 0, 0], v[0, 0, 0], q[0, 0, 0]
    S1 = a * h0[0, 0] @ (np.eye(5) - b * np.outer(kk, kk)) + b * np.outer(vv, kk)
    np.testing.assert_allclose(hT[0, 0], S1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o[0, 0, 0], 0.8 * S1 @ qq, rtol=1e-13, atol=1e-13)


def test_joint_linearity_in_values_and_initial_state():
    rng = np.random.default_rng(8)
    q, k, v1, beta, g, _ = rand_case(rng, B=1, T=40, H=2, DK=6, DV=5)
    v2 = rng.standard_normal(v1.shape)
    a1, a2 = 0.7, -1.3
    s1 = rng.standard_normal((1, 2, 5, 6))
    s2 = rng.standard_normal((1, 2, 5, 6))
    oa, ha = oracle.fwd(q, k, v1, beta, g, h0=s1, layout="VK")
    ob, hb = oracle.fwd(q, k, v2, beta, g, h0=s2, layout="VK")
    oc, hc = oracle.fwd(q, k, a1 * v1 + a2 * v2, beta, g, h0=a1 * s1 + a2 * s2, layout="VK")
    assert rel(oc, a1 * oa + a2 * ob) < 1e-13
    assert rel(hc, a1 * ha + a2 * hb) < 1e-13


def test_segment_composition_forward_and_backward():
    # Running [0, T1) then [T1, T) with the state handed over equals one pass;
    # for the backward, dh0 of the second part is dh_T of the first.
    rng = np.random.default_rng(9)
    q, k, v, beta, g, _ = rand_case(rng, B=1, T=50, H=2, DK=6, DV=5)
    do = rng.standard_normal(v.shape)
    h0 = rng.standard_normal((1, 2, 5, 6))
    dhT = rng.standard_normal((1, 2, 5, 6))
    T1 = 23
    o, hT = oracle.fwd(q, k, v, beta, g, h0=h0, layout="VK")
    sl1 = lambda x: x[:, :T1]
    sl2 = lambda x: x[:, T1:]
    oA, hA = oracle.fwd(*(map(sl1, (q, k, v, beta, g))), h0=h0, layout="VK")
    oB, hB = oracle.fwd(*(map(sl2, (q, k, v, beta, g))), h0=hA, layout="VK")
    assert rel(np.concatenate([oA, oB], axis=1), o) < 1e-13
    assert rel(hB, hT) < 1e-13
    full = oracle.bwd(q, k, v, beta, g, do, h0=h0, dhT=dhT, layout="VK")
    rB = oracle.bwd(*(map(sl2, (q, k, v, beta, g, do))), h0=hA, dhT=dhT, layout="VK")
    rA = oracle.bwd(*(map(sl1, (q, k, v, beta, g, do))), h0=h0, dhT=rB["dh0"], layout="VK")
    for name in ("dq", "dk", "dv", "dbeta", "dg"):
        assert rel(np.concatenate([rA[name], rB[name]], axis=1), full[name]) < 1e-12, name
    assert rel(rA["dh0"], full["dh0"]) < 1e-12


def test_beta0_closed_form_gradients():
    # With beta = 0 the state only decays: S_t = exp(G_t) S_0 with G_t the
    # inclusive sum of g, so o_t = scale exp(G_t) S_0 q_t and
    #   dq_t  = scale exp(G_t) S_0^T do_t
    #   dg_t  = sum_{t' >= t} scale exp(G_t') do_t'.(S_0 q_t') + <dh_T, h_T>
    #   dh0   = sum_t scale exp(G_t) do_t q_t^T + exp(G_T) dh_T
    #   dv    = 0
    rng = np.random.default_rng(11)
    T, DK, DV = 9, 4, 3
    q, k, v, beta, g, _ = rand_case(rng, B=1, T=T, H=1, DK=DK, DV=DV)
    beta[:] = 0.0
    S0 = rng.standard_normal((1, 1, DV, DK))
    do = rng.standard_normal((1, T, 1, DV))
    dhT = rng.standard_normal((1, 1, DV, DK))
    sc = 0.6
    r = oracle.bwd(q, k, v, beta, g, do, h0=S0, dhT=dhT, scale=sc, layout="VK")
    G = np.cumsum(g[0, :, 0])
    S = S0[0, 0]
    hT = np.exp(G[-1]) * S
    terms = np.array([sc * np.exp(G[t]) * do[0, t, 0] @ (S @ q[0, t, 0]) for t in range(T)])
    dg = np.array([terms[t:].sum() for t in range(T)]) + np.sum(dhT[0, 0] * hT)
    dq = np.stack([sc * np.exp(G[t]) * S.T @ do[0, t, 0] for t in range(T)])
    dh0 = sum(sc * np.exp(G[t]) * np.outer(do[0, t, 0], q[0, t, 0]) for t in range(T))
    dh0 = dh0 + np.exp(G[-1]) * dhT[0, 0]
    np.testing.assert_allclose(r["dg"][0, :, 0], dg, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dq"][0, :, 0], dq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dh0"][0, 0], dh0, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(r["dv"], 0.0)


# --------------------------------------------------------------------------
# central finite differences of every gradient


def _loss(q, k, v, beta, g, h0, do, dhT, cu, scale, layout):
    o, hT = oracle.fwd(q, k, v, beta, g, cu_seqlens=cu, h0=h0, scale=scale, layout=layout)
    return float(np.sum(o * do) + np.sum(hT * dhT))


def _fd_check(q, k, v, beta, g, h0, do, dhT, cu=None, scale=None, layout="VK", eps=1e-6):
    r = oracle.bwd(q, k, v, beta, g, do, cu_seqlens=cu, h0=h0, dhT=dhT, scale=scale,
                   layout=layout)
    args = dict(q=q, k=k, v=v, beta=beta, g=g, h0=h0)
    grads = dict(q=r["dq"], k=r["dk"], v=r["dv"], beta=r["dbeta"], g=r["dg"], h0=r["dh0"])
    for name, x in args.items():
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {kk: vv.copy() for kk, vv in args.items()}
            xm = {kk: vv.copy() for kk, vv in args.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            num[idx] = (_loss(do=do, dhT=dhT, cu=cu, scale=scale, layout=layout, **xp)
                        - _loss(do=do, dhT=dhT, cu=cu, scale=scale, layout=layout, **xm)) / (2 * eps)
        err = rel(grads[name], num)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("layout", ["VK", "KV"])
def test_finite_differences_fixed(layout):
    rng = np.random.default_rng(12)
    q, k, v, beta, g, _ = rand_case(rng, B=1, T=8, H=1, DK=4, DV=4)
    h0 = 0.5 * rng.standard_normal((1, 1, 4, 4))
    do = rng.standard_normal(v.shape)
    dhT = rng.standard_normal((1, 1, 4, 4))
    _fd_check(q, k, v, beta, g, h0, do, dhT, layout=layout)


def test_finite_differences_varlen_nonsquare():
    rng = np.random.default_rng(13)
    q, k, v, beta, g, cu = rand_case(rng, H=2, DK=3, DV=5, lengths=[3, 5])
    h0 = 0.5 * rng.standard_normal((2, 2, 5, 3))
    do = rng.standard_normal(v.shape)
    dhT = rng.standard_normal((2, 2, 5, 3))
    _fd_check(q, k, v, beta, g, h0, do, dhT, cu=cu, scale=0.9)


def test_finite_differences_non_unit_keys_positive_g():
    # the backward must not rely on |k| = 1 or g <= 0
    rng = np.random.default_rng(14)
    q, k, v, beta, g, _ = rand_case(rng, B=1, T=6, H=1, DK=4, DV=3, unit_k=False)
    g = 0.3 * rng.standard_normal(g.shape)
    h0 = rng.standard_normal((1, 1, 3, 4))
    do = rng.standard_normal(v.shape)
    dhT = rng.standard_normal((1, 1, 3, 4))
    _fd_check(q, k, v, beta, g, h0, do, dhT)


def test_backward_without_dhT_equals_zero_dhT():
    rng = np.random.default_rng(15)
    q, k, v, beta, g, _ = rand_case(rng, B=1, T=30, H=2, DK=4, DV=4)
    do = rng.standard_normal(v.shape)
    r1 = oracle.bwd(q, k, v, beta, g, do, layout="KV")
    r2 = oracle.bwd(q, k, v, beta, g, do, dhT=np.zeros((1, 2, 4, 4)), h0=np.zeros((1, 2, 4, 4)),
                    layout="KV")
    for name in r1:
        np.testing.assert_array_equal(r1[name], r2[name])


def test_threads_do_not_change_results():
    rng = np.random.default_rng(16)
    q, k, v, beta, g, _ = rand_case(rng, B=2, T=70, H=3, DK=8, DV=8)
    do = rng.standard_normal(v.shape)
    a = oracle.bwd(q, k, v, beta, g, do, nthreads=1)
    b = oracle.bwd(q, k, v, beta, g, do, nthreads=4)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name])
