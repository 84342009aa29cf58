"""GPU parity at the edges of bf16's range.  The matrix-core kernels feed V
(and, in the backward, Q, K, V and the upstream gradient) to fp16 products,
whose normal range is [2^-14, 65504] where bf16 reaches 2^-126 .. 3.4e38;
each kernel scales its fp16 copies by powers of two chosen from the data, so
inputs far outside fp16's range must still meet the bf16 bar against the
float64 oracle.  Inputs are the workload recipes with V (or Q and K) scaled
by exact powers of two: 2^16 pushes V past 65504, 2^-20 below fp16's normal
range; one case mixes heads scaled both ways."""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_02_amd import binding as B
from differential_attention_02_amd import workloads
from tests.parity import as_f64, assert_bf16_grad, assert_bf16_rows

pytestmark = pytest.mark.gpu

X = ("q1", "k1", "q2", "k2", "v")
SCALES = [2.0 ** 16, 2.0 ** -20]


def _note(msg):
    print(f"[gpu] {msg}", flush=True)


def _scaled(inp, names, factor, heads=None):
    out = dict(inp)
    for n in names:
        t = inp[n].float().clone()
        if heads is None:
            t *= factor
        else:
            t[:, :, heads] *= factor
        out[n] = t.to(inp[n].dtype)
    return out


def _v1_fwd(inp, *, causal=True, save=False):
    x = [inp[k].cuda() for k in X]
    vecs = [t.cuda() for t in inp["lambda_vecs"]]
    r = B.fwd(*x, lambda_init=B.lambda_init(12), lambda_vecs=vecs, causal=causal, norm=True, eps=1e-8, save=save)
    torch.cuda.synchronize()
    return r


def _v1_ref(inp, *, causal=True, aux=False):
    li = oracle.lambda_init(12)
    lam = oracle.lambda_value(*[as_f64(t) for t in inp["lambda_vecs"]], li)
    return oracle.diff_attn_fwd(*[as_f64(inp[k]) for k in X], lam, li, causal=causal, norm=True, eps=1e-8,
                                return_aux=aux)


@pytest.mark.parametrize("factor", SCALES, ids=["v_x2^16", "v_x2^-20"])
@pytest.mark.parametrize("causal", [True, False])
def test_v1_forward_v_outside_fp16(factor, causal):
    _note(f"range: V1 forward, V x {factor}, causal={causal}")
    inp = _scaled(workloads.make_attn_inputs("prefill_4k", seed=40, batch=2, seqlen=300, heads=2), ["v"], factor)
    assert_bf16_rows(_v1_fwd(inp, causal=causal), _v1_ref(inp, causal=causal), f"V1 fwd V x {factor}")


def test_v1_forward_mixed_heads():
    """Head 0's V scaled by 2^16 and head 1's by 2^-20 in one call (each
    (batch, head) slice is scaled on its own)."""
    _note("range: V1 forward, mixed heads")
    inp = workloads.make_attn_inputs("prefill_4k", seed=41, batch=1, seqlen=700, heads=2)
    inp = _scaled(_scaled(inp, ["v"], 2.0 ** 16, heads=[0]), ["v"], 2.0 ** -20, heads=[1])
    assert_bf16_rows(_v1_fwd(inp), _v1_ref(inp), "V1 fwd mixed heads")


@pytest.mark.parametrize("factor", SCALES, ids=["v_x2^16", "v_x2^-20"])
def test_v1_training_saves_v_outside_fp16(factor):
    _note(f"range: V1 training forward, V x {factor}")
    inp = _scaled(workloads.make_attn_inputs("train_8k", seed=42, batch=1, seqlen=260, heads=2), ["v"], factor)
    y, sv = _v1_fwd(inp, save=True)
    ref, aux = _v1_ref(inp, aux=True)
    assert_bf16_rows(y, ref, f"V1 train fwd out V x {factor}")
    assert_bf16_rows(sv["o_pre"], aux["O"], f"V1 train fwd o_pre V x {factor}")
    assert_bf16_rows(sv["a2"], aux["A2"], f"V1 train fwd a2 V x {factor}")


@pytest.mark.parametrize("factor", SCALES, ids=["v_x2^16", "v_x2^-20"])
def test_fp8_logit_forward_v_outside_fp16(factor):
    _note(f"range: fp8-logit forward, V x {factor}")
    inp = _scaled(workloads.make_attn_inputs("prefill_4k", seed=43, batch=1, seqlen=333, heads=2), ["v"], factor)
    x = [inp[k].cuda() for k in X]
    vecs = [t.cuda() for t in inp["lambda_vecs"]]
    y = B.fwd_fp8(*x, lambda_init=B.lambda_init(12), lambda_vecs=vecs, causal=True, norm=True, eps=1e-8)
    torch.cuda.synchronize()
    li = oracle.lambda_init(12)
    lam = oracle.lambda_value(*[as_f64(t) for t in inp["lambda_vecs"]], li)
    ref = oracle.diff_attn_fwd_fp8_logits(*[as_f64(inp[k]) for k in X], lam, li, causal=True, norm=True, eps=1e-8)
    assert_bf16_rows(y, ref, f"fp8 fwd V x {factor}")


def _v2_inputs(seed, factor):
    inp = workloads.make_v2_prefill_inputs("v2_prefill_4k", seed=seed, batch=2, seqlen=280, q_heads=4, kv_heads=2)
    return _scaled(inp, ["v"], factor)


@pytest.mark.parametrize("factor", SCALES, ids=["v_x2^16", "v_x2^-20"])
def test_v2_forward_v_outside_fp16(factor):
    _note(f"range: V2 forward, V x {factor}")
    inp = _v2_inputs(44, factor)
    q, k, v, lam = (inp[n].cuda() for n in ("q", "k", "v", "lam"))
    out, sv = B.v2_fwd(q, k, v, lam, save=True)
    torch.cuda.synchronize()
    q64, k64, v64, lam64 = (as_f64(inp[n]) for n in ("q", "k", "v", "lam"))
    assert_bf16_rows(out, oracle.v2_prefill_fwd(q64, k64, v64, lam64), f"V2 fwd V x {factor}")
    # each head's own output: the odd term switched off (sigmoid(-800) = 0)
    off = np.full_like(lam64, -800.0)
    assert_bf16_rows(sv["a_even"], oracle.v2_prefill_fwd(q64, k64, v64, off), f"V2 fwd a_even V x {factor}")
    qs = q64.copy()
    qs[:, :, 0::2] = q64[:, :, 1::2]
    assert_bf16_rows(sv["a_odd"], oracle.v2_prefill_fwd(qs, k64, v64, off), f"V2 fwd a_odd V x {factor}")


@pytest.mark.parametrize("factor", SCALES, ids=["v_x2^16", "v_x2^-20"])
def test_v2_sparse_forward_v_outside_fp16(factor):
    _note(f"range: V2 block-sparse forward, V x {factor}")
    inp = _v2_inputs(45, factor)
    Bn, S, Hq, _ = inp["q"].shape
    m = workloads.make_block_selection(Bn, Hq // 2, S, budget=2, sink=1, local=1, seed=3)
    q, k, v, lam = (inp[n].cuda() for n in ("q", "k", "v", "lam"))
    idx, cnt = B.v2_block_lists(m.cuda())
    out = B.v2_fwd_sparse(q, k, v, lam, idx, cnt)
    torch.cuda.synchronize()
    ref = oracle.v2_prefill_fwd_block_sparse(*[as_f64(inp[n]) for n in ("q", "k", "v", "lam")], m.numpy())
    assert_bf16_rows(out, ref, f"V2 sparse fwd V x {factor}")


# Backward: every fp16 operand is scaled per (batch, head) or (batch, KV
# head).  "qk" scales Q by the factor and K by its inverse, so the logits and
# maps stay those of the recipe while Q and K leave fp16's range; "v" scales V;
# "dy" scales the upstream gradient.
BWD_CASES = [("v", 2.0 ** 16), ("v", 2.0 ** -20), ("qk", 2.0 ** 16), ("qk", 2.0 ** -20), ("dy", 2.0 ** -24)]
BWD_IDS = ["v_x2^16", "v_x2^-20", "q_x2^16", "q_x2^-20", "dy_x2^-24"]


def _scale_bwd_v1(inp, kind, f):
    if kind == "v":
        return _scaled(inp, ["v"], f)
    if kind == "qk":
        return _scaled(_scaled(inp, ["q1", "q2"], f), ["k1", "k2"], 1.0 / f)
    return _scaled(inp, ["dy"], f)


@pytest.mark.parametrize("kind,factor", BWD_CASES, ids=BWD_IDS)
def test_v1_backward_outside_fp16(kind, factor):
    _note(f"range: V1 backward, {kind} x {factor}")
    inp = _scale_bwd_v1(workloads.make_attn_inputs("train_8k", seed=46, batch=2, seqlen=270, heads=2), kind, factor)
    x = {k: inp[k].cuda() for k in X}
    vecs = [t.cuda() for t in inp["lambda_vecs"]]
    li = B.lambda_init(12)
    _, saves = B.fwd(*(x[k] for k in X), lambda_init=li, lambda_vecs=vecs, causal=True, norm=True, eps=1e-8,
                     save=True)
    g = B.bwd(*(x[k] for k in X), inp["dy"].cuda(), saves, lambda_init=li, lambda_vecs=vecs, causal=True,
              norm=True)
    torch.cuda.synchronize()
    ref = oracle.diff_attn_bwd(*[as_f64(inp[k]) for k in X], as_f64(inp["dy"]), lam_init=oracle.lambda_init(12),
                               lam_vectors=[as_f64(t) for t in inp["lambda_vecs"]], causal=True, norm=True,
                               eps=1e-8)
    for k in ("dq1", "dk1", "dq2", "dk2", "dv"):
        got = g[k].float().cpu().numpy()
        assert np.isfinite(got).all(), k
        assert_bf16_grad(got, ref[k], f"V1 bwd {kind} x {factor} {k}")
    assert_bf16_rows(g["dlambda"].cpu().numpy()[None, :], np.array([[ref["dlambda"]]]),
                     f"V1 bwd {kind} x {factor} dlambda")


@pytest.mark.parametrize("kind,factor", BWD_CASES, ids=BWD_IDS)
def test_v2_backward_outside_fp16(kind, factor):
    _note(f"range: V2 backward, {kind} x {factor}")
    inp = workloads.make_v2_prefill_inputs("v2_prefill_4k", seed=47, batch=2, seqlen=260, q_heads=4, kv_heads=2)
    gen = torch.Generator().manual_seed(48)
    Bn, S, Hq, D = inp["q"].shape
    inp["dout"] = torch.randn((Bn, S, Hq // 2, D), generator=gen).to(torch.bfloat16)
    if kind == "v":
        inp = _scaled(inp, ["v"], factor)
    elif kind == "qk":
        inp = _scaled(_scaled(inp, ["q"], factor), ["k"], 1.0 / factor)
    else:
        inp = _scaled(inp, ["dout"], factor)
    q, k, v, lam, dout = (inp[n].cuda() for n in ("q", "k", "v", "lam", "dout"))
    _, saves = B.v2_fwd(q, k, v, lam, save=True)
    g = B.v2_bwd(q, k, v, lam, dout, saves)
    torch.cuda.synchronize()
    ref = oracle.v2_prefill_bwd(*[as_f64(inp[n]) for n in ("q", "k", "v", "lam", "dout")], causal=True)
    for n in ("dq", "dk", "dv"):
        got = as_f64(g[n])
        assert np.isfinite(got).all(), n
        assert_bf16_grad(got, ref[n], f"V2 bwd {kind} x {factor} {n}")
    got = as_f64(g["dlam"])
    assert_bf16_grad(got.reshape(-1, got.shape[-1]), ref["dlam"].reshape(-1, ref["dlam"].shape[-1]),
                     f"V2 bwd {kind} x {factor} dlam")
