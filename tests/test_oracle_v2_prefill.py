"""Pins of the oracle's DIFF V2 prefill forward (CPU only): the scalar twin,
special cases that reduce to torch's attention, the 1 - sigmoid(lambda)
identity, the even/odd pairing inside a GQA group, causality, per-token
lambda, and agreement with the decode step on the last token."""
import numpy as np
import torch

from oracle import brute_v2_prefill_fwd, sigmoid, v2_decode, v2_prefill_fwd


def _case(seed, B=2, S=9, Hq=8, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    lam = rng.standard_normal((B, S, Hq // 2))
    return q, k, v, lam


def _sdpa(q, k, v, causal):
    """torch's scaled_dot_product_attention in float64: q [S, D], k, v [S, D]."""
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], is_causal=causal)
    return o[0].numpy()


def test_brute_force_agrees():
    for causal in (True, False):
        q, k, v, lam = _case(0)
        np.testing.assert_allclose(v2_prefill_fwd(q, k, v, lam, causal=causal),
                                   np.array(brute_v2_prefill_fwd(q, k, v, lam, causal)), rtol=0, atol=1e-12)


def test_very_negative_lambda_is_plain_attention_of_even_heads():
    """sigmoid(lambda) -> 0: every pair's output is its even head's ordinary
    (GQA) attention."""
    q, k, v, _ = _case(1)
    lam = np.full((2, 9, 4), -800.0)
    out = v2_prefill_fwd(q, k, v, lam)
    for b in range(2):
        for p in range(4):
            t = 2 * p
            j = t // 4
            np.testing.assert_allclose(out[b, :, p], _sdpa(q[b, :, t], k[b, :, j], v[b, :, j], True), atol=1e-12)


def test_equal_even_odd_queries_scale_by_one_minus_sigmoid():
    q, k, v, lam = _case(2)
    q[:, :, 1::2] = q[:, :, 0::2]
    out = v2_prefill_fwd(q, k, v, lam)
    for b in range(2):
        for p in range(4):
            att = _sdpa(q[b, :, 2 * p], k[b, :, p // 2], v[b, :, p // 2], True)
            np.testing.assert_allclose(out[b, :, p], (1 - sigmoid(lam[b, :, p]))[:, None] * att, atol=1e-12)


def test_constant_values_give_one_minus_sigmoid():
    """V = 1 everywhere: each head's attention is exactly 1, so every output
    entry is 1 - sigmoid(lambda) of its token and pair."""
    q, k, v, lam = _case(3)
    out = v2_prefill_fwd(q, k, np.ones_like(v), lam)
    np.testing.assert_allclose(out, np.broadcast_to((1 - sigmoid(lam))[..., None], out.shape), atol=1e-14)


def test_pairs_share_their_kv_head():
    """Zeroing KV head 1's values zeroes exactly the pairs whose heads read it
    (query heads 4..7 at group size 4), not the others."""
    q, k, v, lam = _case(4)
    v0 = v.copy()
    v0[:, :, 1] = 0.0
    out, ref = v2_prefill_fwd(q, k, v0, lam), v2_prefill_fwd(q, k, v, lam)
    assert np.all(out[:, :, 2:] == 0.0)
    np.testing.assert_allclose(out[:, :, :2], ref[:, :, :2], atol=0)


def test_causal_rows_ignore_later_keys():
    q, k, v, lam = _case(5)
    out = v2_prefill_fwd(q, k, v, lam)
    k2, v2 = k.copy(), v.copy()
    k2[:, 5:] += 3.0
    v2[:, 5:] -= 2.0
    out2 = v2_prefill_fwd(q, k2, v2, lam)
    np.testing.assert_allclose(out2[:, :5], out[:, :5], atol=0)
    assert np.abs(out2[:, 5:] - out[:, 5:]).max() > 1e-3


def test_lambda_is_per_token():
    """Changing lambda of one token changes only that token's row."""
    q, k, v, lam = _case(6)
    lam2 = lam.copy()
    lam2[:, 3] += 1.0
    out, out2 = v2_prefill_fwd(q, k, v, lam), v2_prefill_fwd(q, k, v, lam2)
    np.testing.assert_allclose(np.delete(out2, 3, axis=1), np.delete(out, 3, axis=1), atol=0)
    assert np.abs(out2[:, 3] - out[:, 3]).max() > 1e-3


def test_last_row_matches_the_decode_step():
    """The causal prefill's last token sees every key: the same as one decode
    step whose cache holds the whole sequence."""
    q, k, v, lam = _case(7)
    pre = v2_prefill_fwd(q, k, v, lam)[:, -1]
    dec = v2_decode(q[:, -1], k, v, lam[:, -1])
    np.testing.assert_allclose(pre, dec, atol=1e-12)


def test_sampled_rows_match_full():
    q, k, v, lam = _case(8)
    rows = np.array([0, 4, 8])
    np.testing.assert_allclose(v2_prefill_fwd(q, k, v, lam, rows=rows), v2_prefill_fwd(q, k, v, lam)[:, rows],
                               atol=0)
