"""GPU parity of diffattn_fwd_fp8 (the forward with fp8 e4m3 attention logits,
through the C ABI) against the float64 oracle: the quantised codes and scale
exponents bit for bit (integer work), the forward within the bf16 bar on
small ragged cases (causal and not, with and without the norm, peaked maps),
and sampled rows of the full 4 x 4096-token workload."""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_02_amd import binding as B
from differential_attention_02_amd import workloads
from tests.parity import as_f64, assert_bf16_rows

pytestmark = pytest.mark.gpu

NAMES = ("q1", "k1", "q2", "k2", "v")


def _note(msg):
    print(f"[gpu] {msg}", flush=True)


def _run(inp, causal=True, norm=True, eps=1e-5, ws=False):
    x = [inp[k].cuda() for k in NAMES]
    vecs = [t.cuda() for t in inp["lambda_vecs"]]
    r = B.fwd_fp8(*x, lambda_init=B.lambda_init(inp["cfg"].layer), lambda_vecs=vecs, causal=causal, norm=norm,
                  eps=eps, return_workspace=ws)
    torch.cuda.synchronize()
    return r


def _ref(inp, causal=True, norm=True, eps=1e-5, rows=None):
    li = oracle.lambda_init(inp["cfg"].layer)
    lam = oracle.lambda_value(*[t.double().numpy() for t in inp["lambda_vecs"]], li)
    x = [as_f64(inp[k]) for k in NAMES]
    return oracle.diff_attn_fwd_fp8_logits(*x, lam, li, causal=causal, norm=norm, eps=eps, rows=rows)


def test_codes_and_exponents_bit_exact():
    _note("fp8 codes")
    inp = workloads.make_attn_inputs("prefill_4k", seed=3, batch=2, seqlen=150, heads=3)
    inp["q2"][0, 5, 1] *= 1e4      # one row with a large exponent
    inp["k1"][1, 7, 2] *= 1e-6     # and one with a small one
    inp["k2"][0, 9, 0] = 0.0       # and an all-zero row
    _, ws = _run(inp, ws=True)
    B_, S, H, d = inp["q1"].shape
    rows = B_ * H * S
    codes = ws[:4 * rows * d].cpu().numpy().reshape(4, B_, H, S, d)
    off = (4 * rows * d + 255) // 256 * 256
    exps = ws[off:off + 4 * rows * 4].cpu().numpy().view(np.int32).reshape(4, B_, H, S)
    for t, name in enumerate(("q1", "k1", "q2", "k2")):
        c, e = oracle.fp8_quantize_rows(as_f64(inp[name]).transpose(0, 2, 1, 3))   # [B, H, S, d]
        np.testing.assert_array_equal(exps[t], e, err_msg=name)
        np.testing.assert_array_equal(codes[t], c, err_msg=name)


@pytest.mark.parametrize("S,causal,norm", [(1, True, True), (65, True, True), (300, True, False),
                                           (200, False, True), (129, True, True)])
def test_forward_small(S, causal, norm):
    _note(f"fp8 forward S={S} causal={causal} norm={norm}")
    inp = workloads.make_attn_inputs("prefill_4k", seed=S, batch=2, seqlen=S, heads=2)
    assert_bf16_rows(_run(inp, causal, norm), _ref(inp, causal, norm), f"fp8 forward S={S}")


def test_forward_peaked_maps():
    """Unit-scale inputs: logits of tens, where the fp8 rounding of Q and K
    moves the scores the most."""
    _note("fp8 forward peaked")
    inp = workloads.make_attn_inputs("prefill_4k", seed=9, batch=1, seqlen=257, heads=2)
    for k in ("q1", "k1", "q2", "k2"):
        inp[k] = (inp[k].float() * 8.0).to(torch.bfloat16)
    assert_bf16_rows(_run(inp, eps=1e-8), _ref(inp, eps=1e-8), "fp8 forward peaked")


def test_full_workload_sampled_rows():
    _note("fp8 forward full 4K workload")
    inp = workloads.make_attn_inputs("prefill_4k", seed=11)
    out = _run(inp, eps=1e-8)
    rows = np.array([0, 1, 63, 64, 127, 128, 1000, 2047, 3001, 4095])
    ref = _ref(inp, eps=1e-8, rows=rows)
    assert_bf16_rows(out[:, torch.as_tensor(rows, device=out.device)], ref, "fp8 forward full workload sampled")


def test_forward_strided_views():
    """Q1, K1, Q2, K2, V as views into one packed per-token projection
    [B, S, H, 4 d + dv]: the quantisation and the forward follow the strides."""
    _note("fp8 strided views")
    inp = workloads.make_attn_inputs("prefill_4k", seed=9, batch=2, seqlen=333, heads=3)
    Bn, S, H, d = inp["q1"].shape
    packed = torch.cat([inp[k] for k in NAMES], dim=-1).cuda()
    offs = [0, d, 2 * d, 3 * d, 4 * d, packed.shape[-1]]
    x = [packed[..., offs[i]:offs[i + 1]] for i in range(5)]
    assert not any(t.is_contiguous() for t in x)
    vecs = [t.cuda() for t in inp["lambda_vecs"]]
    y = B.fwd_fp8(*x, lambda_init=B.lambda_init(inp["cfg"].layer), lambda_vecs=vecs, causal=True, norm=True,
                  eps=1e-5)
    torch.cuda.synchronize()
    assert_bf16_rows(y, _ref(inp), "fp8 strided views")
