"""GPU test of diffattn_v2_decode_noalloc (the decode step that allocates
nothing and keeps its split partials in the library's fixed per-GPU scratch)
through the C ABI: two calls in a row, the second with a smaller input, each
compared with diffattn_v2_decode on the same inputs (same kernels, so the
results must agree bit for bit), and one with the oracle; a call needing more
scratch than the fixed array holds is rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from differential_attention_02_amd import binding as B
from differential_attention_02_amd import workloads
from tests.parity import as_f64, assert_bf16_rows

pytestmark = pytest.mark.gpu


def _inputs(seed, Bn, Hq, Hkv, D, L):
    cfg = workloads.DecodeConfig("t", Bn, Hq, Hkv, D, L, torch.bfloat16, D ** -0.5, lam_shape="per_head")
    return workloads.make_decode_inputs(cfg, seed=seed)


def _both(inp, seqlens):
    q, k, v, lam = (inp[n].cuda() for n in ("q", "k_cache", "v_cache", "lam"))
    Bn, Hq, D = q.shape
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    out_ws = torch.empty((Bn, Hq // 2, D), dtype=q.dtype, device="cuda")
    out_na = torch.full_like(out_ws, float("nan"))
    a = B.decode_args(q, k, v, lam, out_ws, seqlens=sl)
    nbytes = B.decode_workspace_size(a)
    assert 0 < nbytes <= B.DECODE_SCRATCH_BYTES
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes
    B.decode_launch(a)
    b = B.decode_args(q, k, v, lam, out_na, seqlens=sl)   # no workspace given
    B.decode_noalloc_launch(b)
    torch.cuda.synchronize()
    return out_ws.cpu(), out_na.cpu()


def test_noalloc_matches_workspace_entry_point_twice():
    print("[gpu] noalloc decode: call 1 (B 16, 32 q heads over 16 KV heads, D 128, 8192 keys)", flush=True)
    big = _inputs(5, 16, 32, 16, 128, 8192)
    lens = [8192, 1, 5000, 0] * 4
    ws1, na1 = _both(big, lens)
    assert torch.equal(ws1, na1)
    ref = oracle.v2_decode(as_f64(big["q"]), as_f64(big["k_cache"]), as_f64(big["v_cache"]), as_f64(big["lam"]),
                           lens)
    assert_bf16_rows(na1[[0, 1, 2, 4]], ref[[0, 1, 2, 4]], "noalloc decode call 1")
    assert np.all(na1[3].float().numpy() == 0.0)
    print("[gpu] noalloc decode: call 2 (smaller: B 3, 8 q heads over 4 KV heads, D 64, 700 keys)", flush=True)
    small = _inputs(6, 3, 8, 4, 64, 700)
    ws2, na2 = _both(small, [700, 333, 1])
    assert torch.equal(ws2, na2)


def test_noalloc_rejects_more_than_the_fixed_scratch():
    """20000 one-key splits of 4 x 4 heads need ~166 MB of partials: rejected
    on the host, nothing launched."""
    q = torch.empty((4, 4, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((4, 20000, 2, 128), dtype=torch.bfloat16, device="cuda")
    lam = torch.zeros(2, dtype=torch.float32, device="cuda")
    out = torch.empty((4, 2, 128), dtype=torch.bfloat16, device="cuda")
    a = B.decode_args(q, kv, kv, lam, out, num_splits=20000)
    assert B.decode_workspace_size(a) > B.DECODE_SCRATCH_BYTES
    rc = B.lib().diffattn_v2_decode_noalloc(ctypes.byref(a), None)
    assert rc == -3, rc
    assert b"scratch" in B.lib().diffattn_last_error()
