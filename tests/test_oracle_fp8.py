"""Pins of the oracle's fp8 e4m3 logit quantisation (CPU only): the encoder
against torch's float8_e4m3fn cast (an independent implementation, round to
nearest even), the power-of-two absmax rule, the error bound, and the fp8-logit
forward reducing to the ordinary forward when the inputs are already
representable."""
import numpy as np
import torch

from oracle import diff_attn_fwd, diff_attn_fwd_fp8_logits, fp8_decode, fp8_quantize_rows, lambda_init


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_codes_match_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal((64, 64)) * s for s in (1e-3, 0.1, 1.0, 30.0)])
    x = x.astype(np.float32).astype(np.float64)
    codes, e = fp8_quantize_rows(x)
    scaled = (x * 2.0 ** -e[:, None].astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(codes, _torch_codes(scaled))


def test_ties_and_subnormals_round_to_even():
    # one row whose absmax is exactly 448 (scale exponent 0) plus tie cases
    vals = np.array([448.0, 8.5, 9.5, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9 * 2.5, -17.0, 0.0])
    codes, e = fp8_quantize_rows(vals[None])
    assert e[0] == 0
    np.testing.assert_array_equal(codes[0], _torch_codes(vals))
    np.testing.assert_array_equal(fp8_decode(codes[0]), [448.0, 8.0, 10.0, 0.0, 2.0 ** -8, 2.0 ** -8, -16.0, 0.0])


def test_signed_zero():
    """Negative values that round to zero keep the sign bit (e4m3 has -0,
    code 0x80), as torch's cast does."""
    row = np.array([[448.0, -2.0 ** -11, 2.0 ** -11, -0.0, 0.0, -2.0 ** -10]])
    codes, _ = fp8_quantize_rows(row)
    np.testing.assert_array_equal(codes[0], _torch_codes(row[0]))
    np.testing.assert_array_equal(codes[0, 1:], [0x80, 0x00, 0x80, 0x00, 0x80])


def test_absmax_rule_and_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((500, 64)) * np.exp(rng.uniform(-8, 8, (500, 1)))
    codes, e = fp8_quantize_rows(x)
    amax = np.abs(x).max(axis=1)
    scaled = amax * 2.0 ** -e
    assert np.all(scaled <= 448.0) and np.all(scaled > 224.0)
    deq = fp8_decode(codes) * 2.0 ** e[:, None]
    big = np.abs(x) >= 2.0 ** -6 * 2.0 ** e[:, None]          # normal-range elements
    assert np.all(np.abs(deq - x)[big] <= np.abs(x)[big] * 2.0 ** -4)
    assert np.all(np.abs(deq - x)[~big] <= 2.0 ** -10 * 2.0 ** e[:, None].repeat(64, 1)[~big])
    z, ez = fp8_quantize_rows(np.zeros((2, 64)))
    assert np.all(z == 0) and np.all(ez == 0)


def test_representable_inputs_are_unchanged():
    """Inputs that are already fp8 values times a power of two per row make the
    fp8-logit forward equal to the ordinary forward."""
    rng = np.random.default_rng(2)
    B, S, H, d = 1, 20, 2, 16
    parts = []
    for _ in range(4):
        c = rng.integers(0, 126, (B, S, H, d)).astype(np.uint8) | (rng.integers(0, 2, (B, S, H, d)) * 128).astype(np.uint8)
        c[..., 0] = 0x7E   # 448 in every row: the scale exponent is exactly the row's power of two
        parts.append(fp8_decode(c) * 2.0 ** rng.integers(-12, -6, (B, S, H, 1)))
    v = rng.standard_normal((B, S, H, 2 * d))
    li = lambda_init(3)
    np.testing.assert_allclose(diff_attn_fwd_fp8_logits(*parts, v, 0.6, li), diff_attn_fwd(*parts, v, 0.6, li),
                               atol=1e-13)
