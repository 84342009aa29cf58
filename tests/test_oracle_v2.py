"""Pins of the oracle's DIFF V2 decode (CPU only): special cases that reduce
to ordinary attention, the 1 - sigmoid(lambda) row-sum identity, the even/odd
pairing inside a GQA group, sequence lengths, and the scalar twin."""
import numpy as np
import pytest
import torch

from oracle import brute_v2_decode, sigmoid, v2_decode


def _case(seed, B=3, Hq=8, Hkv=4, D=16, L=11):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, L, Hkv, D))
    v = rng.standard_normal((B, L, Hkv, D))
    lam = rng.standard_normal(Hq // 2)
    return q, k, v, lam


def _sdpa_head(q, k, v):
    """torch's scaled_dot_product_attention in float64 for one query vector."""
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])
    return o[0, 0].numpy()


def test_brute_force_agrees():
    q, k, v, lam = _case(0)
    lens = np.array([11, 5, 1])
    np.testing.assert_allclose(v2_decode(q, k, v, lam, lens),
                               np.array(brute_v2_decode(q, k, v, lam, lens)), rtol=1e-12, atol=1e-13)
    lam_b = np.random.default_rng(1).standard_normal((3, 4))
    np.testing.assert_allclose(v2_decode(q, k, v, lam_b),
                               np.array(brute_v2_decode(q, k, v, lam_b)), rtol=1e-12, atol=1e-13)


def test_sigmoid_to_zero_leaves_even_heads():
    """sigmoid(lambda) -> 0 removes the odd head: output = even head's
    ordinary attention over its KV head (library routine)."""
    q, k, v, _ = _case(2, Hq=8, Hkv=2)
    lam = np.full(4, -60.0)
    out = v2_decode(q, k, v, lam)
    for b in range(q.shape[0]):
        for p in range(4):
            t = 2 * p
            j = t // 4
            np.testing.assert_allclose(out[b, p], _sdpa_head(q[b, t], k[b, :, j], v[b, :, j]), rtol=1e-12, atol=1e-13)


def test_equal_pair_queries():
    """Identical even and odd queries: (1 - sigmoid(lambda)) * attention."""
    q, k, v, lam = _case(3, Hq=4, Hkv=2)
    q[:, 1::2] = q[:, 0::2]
    out = v2_decode(q, k, v, lam)
    for b in range(q.shape[0]):
        for p in range(2):
            ref = _sdpa_head(q[b, 2 * p], k[b, :, p], v[b, :, p])
            np.testing.assert_allclose(out[b, p], (1 - sigmoid(lam[p])) * ref, rtol=1e-12, atol=1e-13)


def test_all_ones_values():
    """V = 1: every head's attention is 1, so each output is 1 - sigmoid(lambda)."""
    q, k, _, lam = _case(4)
    v = np.ones_like(k)
    out = v2_decode(q, k, v, lam)
    np.testing.assert_allclose(out, np.broadcast_to((1 - sigmoid(lam))[None, :, None], out.shape), rtol=1e-14)


def test_pairs_share_their_kv_head():
    """Even/odd pairs subtract heads of the same KV head (GQA compatibility
    section).  With KV head 1's values zero, pair 1 (query heads 2, 3 on KV
    head 1) is exactly zero; a first-half/second-half split would have paired
    head 1 (KV head 0) with head 3 and left it non-zero."""
    q, k, v, lam = _case(5, Hq=4, Hkv=2)
    v[:, :, 1] = 0.0
    out = v2_decode(q, k, v, lam)
    assert np.all(out[:, 1] == 0.0)
    assert np.all(np.abs(out[:, 0]).max(axis=-1) > 1e-3)


def test_sequence_lengths():
    """Keys past seqlens[b] never contribute (even NaN there); length 0
    yields zeros."""
    q, k, v, lam = _case(6)
    lens = np.array([7, 11, 0])
    k2, v2 = k.copy(), v.copy()
    k2[0, 7:] = np.nan
    v2[0, 7:] = np.nan
    out = v2_decode(q, k2, v2, lam, lens)
    ref0 = v2_decode(q[:1], k[:1, :7], v[:1, :7], lam)
    np.testing.assert_allclose(out[0], ref0[0], rtol=1e-14)
    assert np.all(out[2] == 0.0)


def test_rejects_pairs_across_kv_heads():
    q, k, v, lam = _case(7, Hq=6, Hkv=2)      # group of 3: pairs would straddle
    with pytest.raises(ValueError):
        v2_decode(q, k, v, lam)
