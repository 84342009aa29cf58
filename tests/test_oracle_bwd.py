"""Pins of the oracle's backward by central finite differences of its own
forward in float64 (the pages print no gradient formulas).  Loss L = <dy, Y>
with random dy; every gradient the backward returns is checked at random
coordinates and along random directions."""
import math

import numpy as np
import pytest

from oracle import diff_attn_bwd, diff_attn_fwd, diff_attn_lambda_grad, lambda_init, lambda_value

H_STEP = 1e-6
TOL = 1e-6


def _setup(seed, B=1, S=32, H=2, d=64, dv=128, in_scale=0.35):
    rng = np.random.default_rng(seed)
    x = {k: rng.standard_normal((B, S, H, d)) * in_scale for k in ("q1", "k1", "q2", "k2")}
    x["v"] = rng.standard_normal((B, S, H, dv))
    vecs = tuple(rng.standard_normal(64) * 0.1 for _ in range(4))
    dy = rng.standard_normal((B, S, H, dv))
    return x, vecs, dy


def _loss(x, vecs, dy, li, causal, norm, eps, lam_fixed=None):
    lam = lam_fixed if lam_fixed is not None else lambda_value(*vecs, li)
    y = diff_attn_fwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], lam, li,
                      causal=causal, norm=norm, eps=eps)
    return math.fsum((dy * y).ravel())


def _fd(f, base, direction):
    return (f(base + H_STEP * direction) - f(base - H_STEP * direction)) / (2 * H_STEP)


def _rel(a, b):
    return abs(a - b) / max(abs(a), abs(b), 1e-8)


@pytest.mark.parametrize("causal,norm", [(True, True), (True, False), (False, True)])
def test_backward_matches_finite_differences(causal, norm):
    """The 2-head, 32-token float64 copy of the training workload (d 64, value
    width 128, lambda_init at layer 12), plus the un-normalised and
    non-causal variants."""
    li, eps = lambda_init(12), 1e-5
    x, vecs, dy = _setup(11)
    g = diff_attn_bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], dy, lam_init=li,
                      lam_vectors=vecs, causal=causal, norm=norm, eps=eps)
    rng = np.random.default_rng(5)
    for name in ("q1", "k1", "q2", "k2", "v"):
        def f(t, name=name):
            y = dict(x)
            y[name] = t
            return _loss(y, vecs, dy, li, causal, norm, eps)
        grad = g["d" + name]
        for _ in range(6):                       # random coordinates
            idx = tuple(rng.integers(0, n) for n in x[name].shape)
            e = np.zeros_like(x[name])
            e[idx] = 1.0
            assert _rel(_fd(f, x[name], e), grad[idx]) < TOL, (name, idx)
        for _ in range(2):                       # random directions
            u = rng.standard_normal(x[name].shape)
            assert _rel(_fd(f, x[name], u), float(np.sum(grad * u))) < TOL, name
    for i, name in enumerate(("dlq1", "dlk1", "dlq2", "dlk2")):
        def f(t, i=i):
            vv = list(vecs)
            vv[i] = t
            return _loss(x, vv, dy, li, causal, norm, eps)
        u = rng.standard_normal(64)
        assert _rel(_fd(f, vecs[i], u), float(np.dot(g[name], u))) < TOL, name
        for j in rng.integers(0, 64, 3):
            e = np.zeros(64)
            e[j] = 1.0
            assert _rel(_fd(f, vecs[i], e), g[name][j]) < TOL, (name, j)


def test_fixed_lambda_gradient():
    """With lambda passed as a fixed scalar the backward returns dL/dlambda."""
    li, eps, lam = 0.2, 1e-5, 0.8
    x, vecs, dy = _setup(2, S=24, d=16, dv=32)
    g = diff_attn_bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], dy, lam_init=li,
                      lam_fixed=lam, causal=True, norm=True, eps=eps)
    f = lambda t: _loss(x, vecs, dy, li, True, True, eps, lam_fixed=float(t))  # noqa: E731
    fd = (f(lam + H_STEP) - f(lam - H_STEP)) / (2 * H_STEP)
    assert _rel(fd, g["dlambda"]) < TOL


def test_lambda_vector_gradients_share_one_scalar():
    """All four vector gradients come from the one scalar dL/dlambda (lambda
    is shared by every head): dlq1 = c1 lk1, dlk1 = c1 lq1, dlq2 = c2 lk2,
    dlk2 = c2 lq2 with c1 / c2 = -exp(<lq1,lk1>) / exp(<lq2,lk2>)."""
    li = lambda_init(12)
    x, vecs, dy = _setup(4, S=16, d=16, dv=32)
    g = diff_attn_bwd(x["q1"], x["k1"], x["q2"], x["k2"], x["v"], dy, lam_init=li,
                      lam_vectors=vecs, causal=True, norm=True)
    c1 = g["dlq1"] / vecs[1]
    c2 = g["dlq2"] / vecs[3]
    np.testing.assert_allclose(c1, c1[0], rtol=1e-10)
    np.testing.assert_allclose(g["dlk1"] / vecs[0], c1[0], rtol=1e-10)
    np.testing.assert_allclose(g["dlk2"] / vecs[2], c2[0], rtol=1e-10)
    assert c1[0] / c2[0] == pytest.approx(-math.exp(np.dot(vecs[0], vecs[1])) / math.exp(np.dot(vecs[2], vecs[3])), rel=1e-10)


@pytest.mark.parametrize("causal,norm", [(True, True), (False, True), (True, False)])
def test_lambda_only_gradient_matches_finite_differences(causal, norm):
    """diff_attn_lambda_grad (the lambda part of the backward on its own, used
    where the full backward is too slow): dL/dlambda by central differences
    in lambda, the vector gradients along a random direction of each vector,
    and agreement with the full backward."""
    li, eps = lambda_init(12), 1e-5
    x, vecs, dy = _setup(7, B=2, S=20, H=2, d=16, dv=32)
    X = (x["q1"], x["k1"], x["q2"], x["k2"], x["v"])
    lam = lambda_value(*vecs, li)
    gf = diff_attn_lambda_grad(*X, dy, lam_init=li, lam_fixed=lam, causal=causal, norm=norm, eps=eps)
    f = lambda t: _loss(x, vecs, dy, li, causal, norm, eps, lam_fixed=float(t))  # noqa: E731
    assert _rel((f(lam + H_STEP) - f(lam - H_STEP)) / (2 * H_STEP), gf["dlambda"]) < TOL
    gv = diff_attn_lambda_grad(*X, dy, lam_init=li, lam_vectors=vecs, causal=causal, norm=norm, eps=eps)
    rng = np.random.default_rng(8)
    for i, name in enumerate(("dlq1", "dlk1", "dlq2", "dlk2")):
        u = rng.standard_normal(64)
        def fv(t, i=i, u=u):
            vv = list(vecs)
            vv[i] = vecs[i] + t * u
            return _loss(x, vv, dy, li, causal, norm, eps)
        fd = (fv(H_STEP) - fv(-H_STEP)) / (2 * H_STEP)
        assert _rel(fd, float(np.dot(gv[name], u))) < TOL, name
    full = diff_attn_bwd(*X, dy, lam_init=li, lam_vectors=vecs, causal=causal, norm=norm, eps=eps)
    for name in ("dlambda", "dlq1", "dlk1", "dlq2", "dlk2"):
        np.testing.assert_allclose(gv[name], full[name], rtol=1e-12, atol=0)
