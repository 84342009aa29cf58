"""Pins of the oracle's block-sparse DIFF V2 forward (CPU only): all blocks
selected is the dense forward; a selection is the same as masking the keys of
unselected blocks by hand in a torch attention call; both heads of a pair use
the pair's selection; rows with no selected key give zeros."""
import numpy as np
import torch

from oracle import sigmoid, v2_prefill_fwd, v2_prefill_fwd_block_sparse


def _case(seed, B=1, S=40, Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, S, Hkv, D)),
            rng.standard_normal((B, S, Hkv, D)), rng.standard_normal((B, S, Hq // 2)))


def test_all_blocks_is_dense():
    q, k, v, lam = _case(0)
    for causal in (True, False):
        mask = np.ones((1, 2, 3, 5), dtype=bool)   # q blocks of 16, k blocks of 8
        np.testing.assert_allclose(
            v2_prefill_fwd_block_sparse(q, k, v, lam, mask, q_block=16, k_block=8, causal=causal),
            v2_prefill_fwd(q, k, v, lam, causal=causal), atol=1e-12)


def test_selection_equals_masked_torch_attention():
    q, k, v, lam = _case(1)
    rng = np.random.default_rng(5)
    mask = rng.random((1, 2, 3, 5)) < 0.5
    mask[..., 0] = True     # every query block keeps key block 0, so no row is empty
    out = v2_prefill_fwd_block_sparse(q, k, v, lam, mask, q_block=16, k_block=8)
    S = 40
    i, j = np.arange(S)[:, None], np.arange(S)[None, :]
    for p in range(2):
        allowed = mask[0, p][i // 16, j // 8] & (j <= i)
        att = []
        for t in (2 * p, 2 * p + 1):
            a = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[0, :, t])[None], torch.from_numpy(k[0, :, t // 2])[None],
                torch.from_numpy(v[0, :, t // 2])[None], attn_mask=torch.from_numpy(allowed)[None])[0].numpy()
            att.append(a)
        want = att[0] - sigmoid(lam[0, :, p])[:, None] * att[1]
        np.testing.assert_allclose(out[0, :, p], want, atol=1e-12)


def test_empty_rows_are_zero():
    q, k, v, lam = _case(2)
    mask = np.zeros((1, 2, 3, 5), dtype=bool)
    mask[0, 0, 1, 4] = True   # pair 0, query block 1 (rows 16..31) sees only keys 32..39: all in its future
    out = v2_prefill_fwd_block_sparse(q, k, v, lam, mask, q_block=16, k_block=8)
    assert np.all(out == 0.0)


def test_row_selection_matches_full_evaluation():
    """rows= evaluates the chosen query rows only; they equal those rows of
    the full evaluation (used at 65,536 tokens, where the full maps do not fit)."""
    q, k, v, lam = _case(3)
    rng = np.random.default_rng(9)
    mask = rng.random((1, 2, 3, 5)) < 0.6
    rows = np.array([0, 5, 16, 31, 39])
    for causal in (True, False):
        full = v2_prefill_fwd_block_sparse(q, k, v, lam, mask, q_block=16, k_block=8, causal=causal)
        part = v2_prefill_fwd_block_sparse(q, k, v, lam, mask, q_block=16, k_block=8, causal=causal, rows=rows)
        np.testing.assert_array_equal(part, full[:, rows])
