"""Pins of the oracle's DIFF V2 prefill backward (CPU only, float64).

The pages print no gradient formulas, so the backward is pinned to things it
does not share: central finite differences of the oracle's own forward
(v2_prefill_fwd), reverse-mode autodiff of an independent torch forward written
with torch's attention primitive, and invariants of softmax gradients (keys
shifted by a constant vector leave the output unchanged, so each head's dK
sums to zero over the keys; equal keys give dQ = 0)."""
import math

import numpy as np
import pytest
import torch

from oracle import sigmoid, v2_prefill_bwd, v2_prefill_fwd

H_STEP = 1e-6
TOL = 1e-6


def _case(seed, B=1, S=12, Hq=4, Hkv=2, D=8, scale=0.6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, Hq, D)) * scale
    k = rng.standard_normal((B, S, Hkv, D)) * scale
    v = rng.standard_normal((B, S, Hkv, D))
    lam = rng.standard_normal((B, S, Hq // 2))
    dout = rng.standard_normal((B, S, Hq // 2, D))
    return q, k, v, lam, dout


def _loss(x, dout, causal):
    return math.fsum((dout * v2_prefill_fwd(x["q"], x["k"], x["v"], x["lam"], causal=causal)).ravel())


def _rel(a, b):
    return abs(a - b) / max(abs(a), abs(b), 1e-8)


@pytest.mark.parametrize("causal,Hkv", [(True, 2), (False, 2), (True, 1)])
def test_backward_matches_finite_differences(causal, Hkv):
    """Random coordinates and random directions of every input, including a
    group of four query heads per KV head (two pairs sharing it)."""
    q, k, v, lam, dout = _case(3, Hkv=Hkv)
    x = {"q": q, "k": k, "v": v, "lam": lam}
    g = v2_prefill_bwd(q, k, v, lam, dout, causal=causal)
    rng = np.random.default_rng(9)
    for name in ("q", "k", "v", "lam"):
        grad = g["d" + name]

        def f(t, name=name):
            y = dict(x)
            y[name] = t
            return _loss(y, dout, causal)

        for _ in range(5):
            idx = tuple(rng.integers(0, n) for n in x[name].shape)
            e = np.zeros_like(x[name])
            e[idx] = 1.0
            fd = (f(x[name] + H_STEP * e) - f(x[name] - H_STEP * e)) / (2 * H_STEP)
            assert _rel(fd, grad[idx]) < TOL, (name, idx, fd, grad[idx])
        d = rng.standard_normal(x[name].shape)
        fd = (f(x[name] + H_STEP * d) - f(x[name] - H_STEP * d)) / (2 * H_STEP)
        assert _rel(fd, float(np.sum(grad * d))) < TOL, name


def _torch_forward(q, k, v, lam, causal):
    """The V2 forward written with torch's attention primitive (float64)."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    kk = k.repeat_interleave(Hq // Hkv, dim=2)
    vv = v.repeat_interleave(Hq // Hkv, dim=2)
    att = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(1, 2), kk.transpose(1, 2), vv.transpose(1, 2), is_causal=causal).transpose(1, 2)
    return att[:, :, 0::2] - torch.sigmoid(lam)[..., None] * att[:, :, 1::2]


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_autograd_of_torch_forward(causal):
    q, k, v, lam, dout = _case(4, B=2, S=20, Hq=8, Hkv=2, D=16)
    t = {n: torch.tensor(a, requires_grad=True) for n, a in (("q", q), ("k", k), ("v", v), ("lam", lam))}
    out = _torch_forward(t["q"], t["k"], t["v"], t["lam"], causal)
    (out * torch.tensor(dout)).sum().backward()
    g = v2_prefill_bwd(q, k, v, lam, dout, causal=causal)
    for n in ("q", "k", "v", "lam"):
        np.testing.assert_allclose(g["d" + n], t[n].grad.numpy(), rtol=0, atol=1e-12)


def test_key_shift_invariance():
    """softmax(s q (K + 1 c^T)^T) = softmax(s q K^T): shifting every key by one
    vector changes nothing, so the sum of dK over the keys is zero."""
    q, k, v, lam, dout = _case(5, S=16)
    for causal in (True, False):
        g = v2_prefill_bwd(q, k, v, lam, dout, causal=causal)
        np.testing.assert_allclose(g["dk"].sum(axis=1), 0.0, atol=1e-12)


def test_equal_keys_give_zero_dq():
    q, k, v, lam, dout = _case(6, S=10)
    k[:] = k[:, :1]
    g = v2_prefill_bwd(q, k, v, lam, dout)
    np.testing.assert_allclose(g["dq"], 0.0, atol=1e-13)


def test_dlam_closed_form_on_constant_values():
    """V = 1 everywhere: out = 1 - sigmoid(lam), so dL/dlam = -sigma (1 - sigma)
    sum_c dout."""
    q, k, v, lam, dout = _case(7)
    v = np.ones_like(v)
    g = v2_prefill_bwd(q, k, v, lam, dout)
    s = sigmoid(lam)
    np.testing.assert_allclose(g["dlam"], -s * (1 - s) * dout.sum(axis=-1), atol=1e-13)
    np.testing.assert_allclose(g["dq"], 0.0, atol=1e-13)   # constant values: scores do not matter
    np.testing.assert_allclose(g["dk"], 0.0, atol=1e-13)
