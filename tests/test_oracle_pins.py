"""Pins of the float64 oracle's forward against facts the pages and the
mathematics fix (CPU only).  None of these re-types the oracle's formulas: each
checks a printed value, an invariant, a special case that reduces to a library
routine, or a scalar brute-force twin."""
import json
import math
import os

import numpy as np
import pytest
import torch

from differential_attention_02_amd import workloads
from oracle import (brute_diff_attn_fwd, diff_attn_fwd, diff_weights, lambda_init,
                    lambda_value)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v, causal):
    """torch's own scaled-dot-product attention in float64 on the CPU; q, k, v
    in [B, S, H, c] layout."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    return o.numpy().transpose(0, 2, 1, 3)


# ---- the glossary page's worked example ------------------------------------

def test_worked_example_printed_values():
    """Seed 0, n=6, d=8, lambda=0.8 prints row sum 0.20 and 13 of 36 negative
    weights (glossary page, 'How differential attention works')."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    q1, k1, q2, k2, v = workloads.worked_example_inputs(g["n"], g["d"], g["seed"])
    w = diff_weights(q1.numpy(), k1.numpy(), q2.numpy(), k2.numpy(), g["lambda"])
    assert f"{w.sum(axis=-1)[0]:.2f}" == g["row0_sum_printed"]
    assert int((w < 0).sum()) == g["negative_weights"]
    assert w.size == g["total_weights"]


def test_worked_example_draw_matches_global_seed():
    """The seeded generator gives the same first draw as torch's global
    generator seeded with 0 (which the page seeds)."""
    torch.manual_seed(0)
    ref = torch.randn(4, 6, 8)
    q1, k1, q2, k2, _ = workloads.worked_example_inputs()
    assert torch.equal(torch.stack([q1, k1, q2, k2]), ref)


@pytest.mark.parametrize("scale,expect_13", [(1.0, False), (1.0 / 4.0, False), (1.0 / math.sqrt(8), True)])
def test_worked_example_fixes_the_scale(scale, expect_13):
    """Only the 1/sqrt(d) scale reproduces the printed count: dropping the
    scale or using 1/sqrt(2d) changes it, so the pin catches a scale slip."""
    q1, k1, q2, k2, _ = workloads.worked_example_inputs()
    w = diff_weights(q1.numpy(), k1.numpy(), q2.numpy(), k2.numpy(), 0.8, scale=scale)
    assert (int((w < 0).sum()) == 13) == expect_13


# ---- invariants of the combine ----------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one_minus_lambda(causal):
    """Each softmax map sums to 1 per row, so map1 - lam*map2 sums to 1 - lam
    (glossary page)."""
    n, d = 17, 8
    q1, k1, q2, k2 = (_rand((n, d), s) for s in range(4))
    for lam in (0.0, 0.3, 0.8, 1.3, -0.4):
        w = diff_weights(q1, k1, q2, k2, lam, causal=causal)
        np.testing.assert_allclose(w.sum(axis=-1), 1.0 - lam, rtol=0, atol=1e-14)
        if causal:
            assert np.all(w[np.triu_indices(n, 1)] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_values(causal):
    """V = 1 gives O = 1 - lam in every channel; with the per-head norm the
    output is (1 - lam_init)(1 - lam)/sqrt((1 - lam)^2 + eps)."""
    B, S, H, d, dv = 2, 9, 3, 8, 16
    q1, k1, q2, k2 = (_rand((B, S, H, d), s) for s in range(4))
    v = np.ones((B, S, H, dv))
    lam, li, eps = 0.77, 0.4, 1e-5
    y = diff_attn_fwd(q1, k1, q2, k2, v, lam, li, causal=causal, norm=False)
    np.testing.assert_allclose(y, 1.0 - lam, rtol=0, atol=1e-14)
    y = diff_attn_fwd(q1, k1, q2, k2, v, lam, li, causal=causal, norm=True, eps=eps)
    expect = (1 - li) * (1 - lam) / math.sqrt((1 - lam) ** 2 + eps)
    np.testing.assert_allclose(y, expect, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_lambda_zero_is_softmax_attention(causal):
    """lam = 0 leaves map1 alone: the output is ordinary attention, checked
    against torch's scaled_dot_product_attention in float64."""
    B, S, H, d, dv = 2, 13, 2, 8, 16
    q1, k1, q2, k2 = (_rand((B, S, H, d), s) for s in range(4))
    v = _rand((B, S, H, dv), 9)
    y = diff_attn_fwd(q1, k1, q2, k2, v, 0.0, 0.5, causal=causal, norm=False)
    np.testing.assert_allclose(y, _sdpa(q1, k1, v, causal), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_maps_scale_attention(causal):
    """Q2 = Q1 and K2 = K1 make both maps equal: O = (1 - lam) * attention."""
    B, S, H, d, dv = 1, 11, 2, 8, 16
    q1, k1 = _rand((B, S, H, d), 1), _rand((B, S, H, d), 2)
    v = _rand((B, S, H, dv), 3)
    lam = 0.62
    y = diff_attn_fwd(q1, k1, q1, k1, v, lam, 0.5, causal=causal, norm=False)
    np.testing.assert_allclose(y, (1 - lam) * _sdpa(q1, k1, v, causal), rtol=1e-12, atol=1e-13)


def test_causal_ignores_future_keys():
    """Changing keys/values after position i leaves row i unchanged."""
    B, S, H, d, dv = 1, 12, 1, 8, 16
    x = [_rand((B, S, H, d), s) for s in range(4)] + [_rand((B, S, H, dv), 5)]
    y0 = diff_attn_fwd(*x, 0.7, 0.3, causal=True)
    x2 = [t.copy() for t in x]
    for t in x2[1::2] + [x2[4]]:
        t[:, 7:] += 5.0
    y1 = diff_attn_fwd(*x2, 0.7, 0.3, causal=True)
    np.testing.assert_array_equal(y0[:, :7], y1[:, :7])
    assert not np.allclose(y0[:, 7:], y1[:, 7:])


# ---- lambda ------------------------------------------------------------------

def test_lambda_init_schedule():
    """lambda_init(1) = 0.8 - 0.6 = 0.2; deeper layers start nearer 0.8
    (glossary page; news write-up); every value lies in (0, 1)."""
    assert lambda_init(1) == pytest.approx(0.2, abs=1e-15)
    vals = [lambda_init(l) for l in range(1, 200)]
    assert all(b > a for a, b in zip(vals[:100], vals[1:100]))
    assert all(b >= a for a, b in zip(vals, vals[1:]))
    assert all(0.0 < x <= 0.8 for x in vals)
    assert vals[-1] == pytest.approx(0.8, abs=1e-12)
    with pytest.raises(ValueError):
        lambda_init(0)


def test_lambda_init_values_at_the_workload_layers():
    """lambda_init at layers 1, 2, 12 and 24 equals the pages' printed schedule
    evaluated in 40-digit decimal arithmetic (tests/golden/lambda_init.json,
    cited there), and the gaps to 0.8 shrink by exactly exp(-0.3) per layer,
    which fixes the decay rate (a 0.3 -> 0.03 slip gives a ratio of 0.97)."""
    rec = json.load(open(os.path.join(GOLDEN, "lambda_init.json")))
    for layer, val in rec["lambda_init"].items():
        assert lambda_init(int(layer)) == pytest.approx(float(val), abs=2e-16), layer
    q = float(rec["gap_ratio_exp_minus_0.3"])
    for layer in range(1, 24):   # deeper, 0.8 - lambda_init loses digits to cancellation
        ratio = (0.8 - lambda_init(layer + 1)) / (0.8 - lambda_init(layer))
        assert ratio == pytest.approx(q, rel=1e-10), layer


def test_lambda_value_special_cases():
    """Zero vectors, or equal (q, k) pairs, leave lambda = lambda_init; with
    the second pair zero, lambda rises above lambda_init exactly when
    <lq1, lk1> > 0; swapping the pairs mirrors lambda around lambda_init."""
    rng = np.random.default_rng(3)
    z = np.zeros(64)
    assert lambda_value(z, z, z, z, 0.37) == 0.37
    a, b = rng.standard_normal(64) * 0.1, rng.standard_normal(64) * 0.1
    assert lambda_value(a, b, a, b, 0.37) == pytest.approx(0.37, abs=1e-15)
    up = lambda_value(np.abs(a), np.abs(b), z, z, 0.37)
    down = lambda_value(np.abs(a), -np.abs(b), z, z, 0.37)
    assert up > 0.37 > down
    c, e = rng.standard_normal(64) * 0.1, rng.standard_normal(64) * 0.1
    l1 = lambda_value(a, b, c, e, 0.37)
    l2 = lambda_value(c, e, a, b, 0.37)
    assert (l1 - 0.37) == pytest.approx(-(l2 - 0.37), abs=1e-15)
    # exp(<a,b>) - 1 with the second pair zero: at a tiny dot product this
    # is the dot product itself to first order.
    t = lambda_value(a * 1e-4, b * 1e-4, z, z, 0.0)
    assert t == pytest.approx(float(np.dot(a, b)) * 1e-8, rel=1e-6)


# ---- per-head RMSNorm ----------------------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 1e-5, 1e-3])
def test_rmsnorm_row_rms(eps):
    """Per-head normalisation: each row of Y has RMS |1 - lam_init| scaled by
    sqrt(m / (m + eps)), m the row mean square of the un-normalised output."""
    B, S, H, d, dv = 2, 10, 3, 8, 16
    x = [_rand((B, S, H, d), s) for s in range(4)] + [_rand((B, S, H, dv), 4)]
    lam, li = 0.55, 0.2
    o = diff_attn_fwd(*x, lam, li, causal=True, norm=False)
    y = diff_attn_fwd(*x, lam, li, causal=True, norm=True, eps=eps)
    m = np.mean(o * o, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)),
                               abs(1 - li) * np.sqrt(m / (m + eps)), rtol=1e-13)
    # the norm only rescales rows: direction unchanged
    np.testing.assert_allclose(y / np.linalg.norm(y, axis=-1, keepdims=True),
                               o / np.linalg.norm(o, axis=-1, keepdims=True), rtol=1e-12, atol=1e-14)


# ---- scalar brute-force twin -----------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("norm", [False, True])
def test_brute_force_agrees_on_tiny_config(causal, norm):
    """The tiny single-head float32 workload (64 tokens, d 8, dv 16, lambda
    0.8, lambda_init at layer 1) through the vectorised oracle and the
    scalar loops."""
    t = workloads.make_attn_inputs("tiny_f32")
    x = [t[k].double().numpy() for k in ("q1", "k1", "q2", "k2", "v")]
    li = lambda_init(1)
    y = diff_attn_fwd(*x, 0.8, li, causal=causal, norm=norm, eps=1e-5)
    yb = np.array(brute_diff_attn_fwd(*x, 0.8, li, causal=causal, norm=norm, eps=1e-5))
    np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-12)


def test_brute_force_agrees_at_large_logits():
    """Logits spanning about +-40 (the page's largest reported attention
    logit is 38.8): the max-shifted oracle matches the unshifted twin."""
    B, S, H, d, dv = 1, 20, 2, 8, 16
    x = [_rand((B, S, H, d), s, 3.0) for s in range(4)] + [_rand((B, S, H, dv), 4)]
    s1 = x[0][0, :, 0] @ x[1][0, :, 0].T / math.sqrt(d)
    assert np.abs(s1).max() > 20
    y = diff_attn_fwd(*x, 0.9, 0.5, causal=True, norm=True)
    yb = np.array(brute_diff_attn_fwd(*x, 0.9, 0.5, causal=True, norm=True))
    np.testing.assert_allclose(y, yb, rtol=1e-10, atol=1e-12)


def test_row_subset_and_aux():
    """rows= evaluates the same rows; aux holds O = A1 - lam A2, and the
    partition functions match a scalar log-sum-exp."""
    B, S, H, d, dv = 1, 15, 2, 8, 16
    x = [_rand((B, S, H, d), s) for s in range(4)] + [_rand((B, S, H, dv), 4)]
    lam = 0.66
    y, aux = diff_attn_fwd(*x, lam, 0.3, causal=True, return_aux=True)
    rows = np.array([0, 3, 14])
    ys = diff_attn_fwd(*x, lam, 0.3, causal=True, rows=rows)
    np.testing.assert_allclose(ys, y[:, rows], rtol=1e-14, atol=0)
    np.testing.assert_allclose(aux["O"], aux["A1"] - lam * aux["A2"], rtol=1e-12, atol=1e-14)
    b, h, i = 0, 1, 9
    sc = [math.fsum(a * c for a, c in zip(x[2][b, i, h], x[3][b, j, h])) / math.sqrt(d) for j in range(i + 1)]
    assert aux["lse2"][b, h, i] == pytest.approx(math.log(math.fsum(math.exp(t) for t in sc)), rel=1e-13)
