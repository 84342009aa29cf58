"""GPU parity of diffattn_v1_decode (DIFF V1 decode over a K1/K2/V cache,
through the C ABI) against the float64 oracle: float32 and bf16, ragged
sequence lengths (empty and one-key sequences included), fixed lambda and
lambda vectors, with and without the per-head norm, split invariance, strided
views, and sampled sequences of the full 64 x 8192-token workload."""
import numpy as np
import pytest
import torch

import oracle
from differential_attention_02_amd import binding as B
from differential_attention_02_amd import workloads
from tests.parity import as_f64, assert_bf16_rows, assert_f32

pytestmark = pytest.mark.gpu

NAMES = ("q1", "q2", "k1_cache", "k2_cache", "v_cache")


def _note(msg):
    print(f"[gpu] {msg}", flush=True)


def _inputs(seed, dtype=torch.bfloat16, **kw):
    cfg = workloads.CONFIGS["v1_decode"]
    if dtype != cfg.dtype:
        cfg = workloads.V1DecodeConfig("t", cfg.batch, cfg.heads, cfg.head_dim, cfg.v_dim, cfg.kv_len, dtype,
                                       cfg.input_scale, cfg.layer)
    return workloads.make_v1_decode_inputs(cfg, seed=seed, **kw)


def _lam(inp):
    li = oracle.lambda_init(inp["cfg"].layer)
    return oracle.lambda_value(*[t.double().numpy() for t in inp["lambda_vecs"]], li), li


def _run(inp, seqlens=None, num_splits=0, norm=True, vectors=True, lam_fixed=0.8):
    x = [inp[n].cuda() for n in NAMES]
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    vecs = [t.cuda() for t in inp["lambda_vecs"]] if vectors else None
    out = B.v1_decode(*x, lambda_init=B.lambda_init(inp["cfg"].layer), lambda_vecs=vecs, lambda_fixed=lam_fixed,
                      norm=norm, eps=inp["cfg"].eps, seqlens=sl, num_splits=num_splits)
    torch.cuda.synchronize()
    return out


def _ref(inp, seqlens=None, norm=True, vectors=True, lam_fixed=0.8, batch=None):
    lam, li = _lam(inp)
    if not vectors:
        lam = lam_fixed
    xs = [as_f64(inp[n]) for n in NAMES]
    if batch is not None:
        xs = [x[batch] for x in xs]
    return oracle.v1_decode(*xs, lam, li, seqlens, norm=norm, eps=inp["cfg"].eps)


@pytest.mark.parametrize("norm", [True, False])
def test_small_f32(norm):
    _note(f"v1 decode f32 norm={norm}")
    inp = _inputs(0, torch.float32, batch=3, kv_len=1000, heads=4)
    lens = [1000, 513, 0]
    out = _run(inp, lens, norm=norm)
    assert_f32(out, _ref(inp, lens, norm=norm), f"v1 decode f32 norm={norm}")
    assert np.all(out[2].cpu().numpy() == 0.0)


def test_small_bf16_ragged():
    _note("v1 decode bf16 ragged")
    inp = _inputs(1, batch=5, kv_len=777, heads=3)
    lens = [777, 1, 300, 64, 0]
    out = _run(inp, lens)
    ref = _ref(inp, lens)
    assert_bf16_rows(out[:4], ref[:4], "v1 decode bf16 ragged")
    assert np.all(out[4].float().cpu().numpy() == 0.0)


def test_fixed_lambda_no_norm():
    _note("v1 decode fixed lambda")
    inp = _inputs(2, batch=2, kv_len=600, heads=2)
    out = _run(inp, vectors=False, lam_fixed=0.95, norm=False)
    assert_bf16_rows(out, _ref(inp, vectors=False, lam_fixed=0.95, norm=False), "v1 decode lambda 0.95")


def test_split_invariance():
    """The answer does not depend on how many key chunks the cache is split
    into (float32, up to accumulation order)."""
    _note("v1 decode split invariance")
    inp = _inputs(3, torch.float32, batch=2, kv_len=3000, heads=2)
    outs = [_run(inp, num_splits=s).cpu().numpy() for s in (2, 3, 7, 12)]
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=1e-5, atol=1e-6)
    assert_f32(outs[0], _ref(inp), "v1 decode f32 splits")


def test_strided_views():
    """Queries and caches as views into packed tensors."""
    _note("v1 decode strided")
    inp = _inputs(4, batch=2, kv_len=300, heads=2)
    q = torch.cat([inp["q1"], inp["q2"]], dim=2).cuda()          # [B, H, 2d]
    kc = torch.cat([inp["k1_cache"], inp["k2_cache"]], dim=3).cuda()  # [B, L, H, 2d]
    vv = torch.zeros((2, 300, 3, 128), dtype=torch.bfloat16, device="cuda")
    vv[:, :, 1] = inp["v_cache"][:, :, 0].cuda()
    vv[:, :, 2] = inp["v_cache"][:, :, 1].cuda()
    vecs = [t.cuda() for t in inp["lambda_vecs"]]
    out = B.v1_decode(q[:, :, :64], q[:, :, 64:], kc[..., :64], kc[..., 64:], vv[:, :, 1:],
                      lambda_init=B.lambda_init(inp["cfg"].layer), lambda_vecs=vecs, eps=inp["cfg"].eps)
    torch.cuda.synchronize()
    assert_bf16_rows(out, _ref(inp), "v1 decode strided")


def test_full_workload_sampled_sequences():
    cfg = workloads.CONFIGS["v1_decode"]
    _note(f"v1 decode full workload {cfg}")
    inp = _inputs(5)
    out = _run(inp)
    pick = np.array([0, 17, 40, 63])
    assert_bf16_rows(out[torch.as_tensor(pick, device=out.device)], _ref(inp, batch=pick),
                     "v1 decode full workload sampled")
    assert torch.isfinite(out.float()).all()
