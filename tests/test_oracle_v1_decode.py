"""Pins of the oracle's DIFF V1 decode step (CPU only): one new token over a
K1/K2/V cache equals the last row of the causal prefill forward over the same
sequence (an independent code path: the prefill forward masks and slices a
full score matrix), sequence lengths cut the cache, lambda = 0 with equal maps
reduces to torch attention, V = 1 gives the normalised 1 - lambda, and an
empty sequence gives zeros."""
import numpy as np
import torch

from oracle import diff_attn_fwd, lambda_init, v1_decode


def _cache(seed, B=2, L=11, H=3, d=8, dv=16):
    rng = np.random.default_rng(seed)
    k1, k2 = rng.standard_normal((2, B, L, H, d)) * 0.7
    v = rng.standard_normal((B, L, H, dv))
    q1, q2 = rng.standard_normal((2, B, H, d)) * 0.7
    return q1, q2, k1, k2, v


def test_matches_last_row_of_causal_prefill():
    q1, q2, k1, k2, v = _cache(0)
    li = lambda_init(5)
    for norm in (True, False):
        # the new token's query sits at the last position of the prefill inputs
        Q1, Q2 = np.zeros_like(k1), np.zeros_like(k2)
        Q1[:, -1], Q2[:, -1] = q1, q2
        ref = diff_attn_fwd(Q1, k1, Q2, k2, v, 0.7, li, causal=True, norm=norm, eps=1e-5)[:, -1]
        np.testing.assert_allclose(v1_decode(q1, q2, k1, k2, v, 0.7, li, norm=norm), ref, atol=1e-12)


def test_seqlens_cut_the_cache():
    q1, q2, k1, k2, v = _cache(1)
    li = lambda_init(3)
    out = v1_decode(q1, q2, k1, k2, v, 0.5, li, seqlens=[7, 0])
    np.testing.assert_allclose(out[0], v1_decode(q1[:1], q2[:1], k1[:1, :7], k2[:1, :7], v[:1, :7], 0.5, li)[0],
                               atol=1e-13)
    assert np.all(out[1] == 0.0)


def test_lambda_zero_is_torch_attention():
    q1, q2, k1, k2, v = _cache(2, B=1)
    out = v1_decode(q1, q2, k1, k2, v, 0.0, 0.2, norm=False)
    for h in range(3):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q1[0, h])[None, None], torch.from_numpy(k1[0, :, h])[None],
            torch.from_numpy(v[0, :, h])[None])[0, 0].numpy()
        np.testing.assert_allclose(out[0, h], ref, atol=1e-12)


def test_constant_values_give_one_minus_lambda():
    q1, q2, k1, k2, v = _cache(3)
    ones = np.ones_like(v)
    np.testing.assert_allclose(v1_decode(q1, q2, k1, k2, ones, 0.8, 0.2, norm=False), 0.2, atol=1e-14)
    li, eps = lambda_init(4), 1e-5
    want = (1 - li) * 0.2 / np.sqrt(0.04 + eps)
    np.testing.assert_allclose(v1_decode(q1, q2, k1, k2, ones, 0.8, li, eps=eps), want, atol=1e-12)
