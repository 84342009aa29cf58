"""ctypes binding of libdiffattn.so (C ABI in include/diffattn.h).

Argument marshalling only: torch tensors supply device pointers, strides and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  The binding allocates outputs and workspaces with torch (device
memory plumbing) and raises RuntimeError on any non-zero status.  There is no
fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdiffattn.so")

F32, BF16 = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
c_fp = ctypes.c_void_p  # float* passed as raw address


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32), ("seqlen", c_i32), ("heads", c_i32), ("head_dim", c_i32), ("v_dim", c_i32),
        ("dtype", c_i32), ("causal", c_i32), ("norm", c_i32),
        ("q1", c_vp), ("k1", c_vp), ("q2", c_vp), ("k2", c_vp), ("v", c_vp),
        ("q_stride", c_i64 * 3), ("k_stride", c_i64 * 3), ("v_stride", c_i64 * 3), ("o_stride", c_i64 * 3),
        ("lq1", c_fp), ("lk1", c_fp), ("lq2", c_fp), ("lk2", c_fp),
        ("lambda_dim", c_i32), ("lambda_fixed", c_f32), ("lambda_init", c_f32),
        ("softmax_scale", c_f32), ("eps", c_f32),
        ("out", c_vp), ("lambda_out", c_fp),
        ("lse1", c_fp), ("lse2", c_fp), ("rstd", c_fp), ("o_pre", c_fp), ("a2", c_fp),
        ("workspace", c_vp), ("workspace_bytes", c_sz),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32), ("seqlen", c_i32), ("heads", c_i32), ("head_dim", c_i32), ("v_dim", c_i32),
        ("dtype", c_i32), ("causal", c_i32), ("norm", c_i32),
        ("q1", c_vp), ("k1", c_vp), ("q2", c_vp), ("k2", c_vp), ("v", c_vp),
        ("q_stride", c_i64 * 3), ("k_stride", c_i64 * 3), ("v_stride", c_i64 * 3),
        ("dout", c_vp), ("do_stride", c_i64 * 3),
        ("lq1", c_fp), ("lk1", c_fp), ("lq2", c_fp), ("lk2", c_fp),
        ("lambda_dim", c_i32), ("lambda_fixed", c_f32), ("lambda_init", c_f32), ("softmax_scale", c_f32),
        ("lse1", c_fp), ("lse2", c_fp), ("rstd", c_fp), ("o_pre", c_fp), ("a2", c_fp),
        ("dq1", c_vp), ("dk1", c_vp), ("dq2", c_vp), ("dk2", c_vp), ("dv", c_vp),
        ("dq_stride", c_i64 * 3), ("dk_stride", c_i64 * 3), ("dv_stride", c_i64 * 3),
        ("dlq1", c_fp), ("dlk1", c_fp), ("dlq2", c_fp), ("dlk2", c_fp), ("dlambda", c_fp),
        ("workspace", c_vp), ("workspace_bytes", c_sz),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32), ("q_heads", c_i32), ("kv_heads", c_i32), ("head_dim", c_i32), ("kv_len", c_i32),
        ("dtype", c_i32),
        ("q", c_vp), ("q_stride", c_i64 * 2),
        ("k_cache", c_vp), ("v_cache", c_vp), ("kv_stride", c_i64 * 3),
        ("seqlens", c_vp),
        ("lam", c_fp), ("lam_stride_b", c_i64),
        ("softmax_scale", c_f32),
        ("out", c_vp), ("o_stride", c_i64 * 2),
        ("num_splits", c_i32),
        ("workspace", c_vp), ("workspace_bytes", c_sz),
    ]


class V1DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32), ("heads", c_i32), ("head_dim", c_i32), ("v_dim", c_i32), ("kv_len", c_i32),
        ("dtype", c_i32), ("norm", c_i32),
        ("q1", c_vp), ("q2", c_vp), ("q_stride", c_i64 * 2),
        ("k1_cache", c_vp), ("k2_cache", c_vp), ("k_stride", c_i64 * 3),
        ("v_cache", c_vp), ("v_stride", c_i64 * 3),
        ("seqlens", c_vp),
        ("lq1", c_fp), ("lk1", c_fp), ("lq2", c_fp), ("lk2", c_fp),
        ("lambda_dim", c_i32), ("lambda_fixed", c_f32), ("lambda_init", c_f32),
        ("softmax_scale", c_f32), ("eps", c_f32),
        ("out", c_vp), ("o_stride", c_i64 * 2),
        ("num_splits", c_i32),
        ("workspace", c_vp), ("workspace_bytes", c_sz),
    ]


class V2FwdArgs(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32), ("seqlen", c_i32), ("q_heads", c_i32), ("kv_heads", c_i32), ("head_dim", c_i32),
        ("dtype", c_i32), ("causal", c_i32),
        ("q", c_vp), ("k", c_vp), ("v", c_vp),
        ("q_stride", c_i64 * 3), ("kv_stride", c_i64 * 3),
        ("lam", c_fp), ("lam_stride", c_i64 * 3),
        ("softmax_scale", c_f32),
        ("out", c_vp), ("o_stride", c_i64 * 3),
        ("lse", c_fp), ("a_even", c_fp), ("a_odd", c_fp),
        ("workspace", c_vp), ("workspace_bytes", c_sz),
    ]


class V2BwdArgs(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32), ("seqlen", c_i32), ("q_heads", c_i32), ("kv_heads", c_i32), ("head_dim", c_i32),
        ("dtype", c_i32), ("causal", c_i32),
        ("q", c_vp), ("k", c_vp), ("v", c_vp),
        ("q_stride", c_i64 * 3), ("kv_stride", c_i64 * 3),
        ("lam", c_fp), ("lam_stride", c_i64 * 3),
        ("softmax_scale", c_f32),
        ("dout", c_vp), ("do_stride", c_i64 * 3),
        ("lse", c_fp), ("a_even", c_fp), ("a_odd", c_fp),
        ("dq", c_vp), ("dq_stride", c_i64 * 3),
        ("dk", c_vp), ("dv", c_vp), ("dkv_stride", c_i64 * 3),
        ("dlam", c_fp),
        ("workspace", c_vp), ("workspace_bytes", c_sz),
    ]


# Every symbol include/diffattn.h declares, with its ctypes signature.
SIGNATURES = {
    "diffattn_fwd": (ctypes.c_int, [ctypes.POINTER(FwdArgs), c_vp]),
    "diffattn_bwd": (ctypes.c_int, [ctypes.POINTER(BwdArgs), c_vp]),
    "diffattn_fwd_fp8": (ctypes.c_int, [ctypes.POINTER(FwdArgs), c_vp, c_sz, c_vp]),
    "diffattn_fwd_fp8_workspace_size": (c_sz, [ctypes.POINTER(FwdArgs)]),
    "diffattn_fwd_workspace_size": (c_sz, [ctypes.POINTER(FwdArgs)]),
    "diffattn_v2_fwd_workspace_size": (c_sz, [ctypes.POINTER(V2FwdArgs)]),
    "diffattn_bwd_workspace_size": (c_sz, [ctypes.POINTER(BwdArgs)]),
    "diffattn_v2_decode": (ctypes.c_int, [ctypes.POINTER(DecodeArgs), c_vp]),
    "diffattn_v2_decode_workspace_size": (c_sz, [ctypes.POINTER(DecodeArgs)]),
    "diffattn_v2_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(DecodeArgs), c_vp]),
    "diffattn_v1_decode": (ctypes.c_int, [ctypes.POINTER(V1DecodeArgs), c_vp]),
    "diffattn_v1_decode_workspace_size": (c_sz, [ctypes.POINTER(V1DecodeArgs)]),
    "diffattn_v2_fwd": (ctypes.c_int, [ctypes.POINTER(V2FwdArgs), c_vp]),
    "diffattn_v2_bwd": (ctypes.c_int, [ctypes.POINTER(V2BwdArgs), c_vp]),
    "diffattn_v2_fwd_sparse": (ctypes.c_int, [ctypes.POINTER(V2FwdArgs), c_vp, c_vp, c_i32, c_vp]),
    "diffattn_v2_bwd_workspace_size": (c_sz, [ctypes.POINTER(V2BwdArgs)]),
    "diffattn_lambda_init": (c_f32, [ctypes.c_int]),
    "diffattn_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "diffattn_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libdiffattn.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m differential_attention_02_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise RuntimeError(f"{what} failed: {L.diffattn_status_str(status).decode()}: "
                           f"{L.diffattn_last_error().decode()}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _strides3(t):
    s = t.stride()
    return (c_i64 * 3)(s[0], s[1], s[2])


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_dev(named, dtype=None, device=None):
    """Every tensor on one GPU, channel dim contiguous, optional dtype."""
    for name, t in named:
        if t is None:
            continue
        _require(isinstance(t, torch.Tensor) and t.is_cuda, f"{name} must be a GPU tensor")
        _require(t.dim() == 0 or t.stride(-1) == 1 or t.shape[-1] == 1, f"{name}: last dim must be contiguous")
        if dtype is not None:
            _require(t.dtype == dtype, f"{name}: expected {dtype}, got {t.dtype}")
        if device is not None:
            _require(t.device == device, f"{name} is on {t.device}, expected {device}")


def _check_attn(q1, k1, q2, k2, v, out, lambda_vecs):
    _require(q1.dim() == 4, "q1 must be [B, S, H, d]")
    B, S, H, d = q1.shape
    for name, t in (("k1", k1), ("q2", q2), ("k2", k2)):
        _require(tuple(t.shape) == (B, S, H, d), f"{name} shape {tuple(t.shape)} != {(B, S, H, d)}")
    _require(v.dim() == 4 and tuple(v.shape[:3]) == (B, S, H), "v must be [B, S, H, dv]")
    if out is not None:
        _require(tuple(out.shape) == tuple(v.shape), "out must have v's shape")
    _check_dev((("q1", q1), ("k1", k1), ("q2", q2), ("k2", k2), ("v", v), ("out", out)),
               dtype=q1.dtype, device=q1.device)
    if lambda_vecs is not None:
        _require(len(lambda_vecs) == 4, "lambda_vecs must hold lq1, lk1, lq2, lk2")
        n = lambda_vecs[0].numel()
        for i, t in enumerate(lambda_vecs):
            _require(t.is_contiguous() and t.numel() == n and t.dim() == 1, "lambda vectors: 1-D, contiguous, equal length")
        _check_dev((("lambda_vec%d" % i, t) for i, t in enumerate(lambda_vecs)), dtype=torch.float32,
                   device=q1.device)


def _attach_workspace(a, size_fn, device):
    """Allocates the workspace size_fn(args) asks for (if any) and attaches it;
    the tensor is kept on the args object so it lives as long as they do."""
    nbytes = int(size_fn(ctypes.byref(a)))
    if nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        a.workspace, a.workspace_bytes = _ptr(ws), nbytes
        a._workspace = ws
    return a


def lambda_init(layer: int) -> float:
    """lambda_init for layer l >= 1 as the library computes it."""
    return float(lib().diffattn_lambda_init(int(layer)))


def _lambda_fields(a, lambda_vecs, lambda_fixed):
    if lambda_vecs is not None:
        lq1, lk1, lq2, lk2 = lambda_vecs
        a.lq1, a.lk1, a.lq2, a.lk2 = (_ptr(t) for t in (lq1, lk1, lq2, lk2))
        a.lambda_dim = lq1.numel()
    else:
        a.lambda_dim = 0
    a.lambda_fixed = float(lambda_fixed)


def fwd(q1, k1, q2, k2, v, *, lambda_init: float, lambda_vecs=None, lambda_fixed: float = 0.8,
        causal: bool = True, norm: bool = True, eps: float = 1e-5, softmax_scale: float = 0.0,
        out=None, save: bool = False, lambda_out=None):
    """Differential attention forward through diffattn_fwd.

    q1, k1, q2, k2: [B, S, H, d]; v: [B, S, H, dv] (device tensors, channel
    dim contiguous).  lambda_vecs: four float32 device vectors, or None to use
    lambda_fixed.  Returns out [B, S, H, dv]; with save=True returns
    (out, saves) where saves holds lse1, lse2, rstd, o_pre, a2 and lambda.
    lambda_out: optional float32 device tensor of one element that receives
    the lambda the kernel used.
    """
    _check_attn(q1, k1, q2, k2, v, out, lambda_vecs)
    B, S, H, d = q1.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, S, H, dv), dtype=v.dtype, device=v.device)
    if lambda_out is not None:
        _check_dev((("lambda_out", lambda_out),), dtype=torch.float32, device=v.device)
        _require(lambda_out.numel() >= 1, "lambda_out needs one element")
    a = FwdArgs()
    a.batch, a.seqlen, a.heads, a.head_dim, a.v_dim = B, S, H, d, dv
    a.dtype, a.causal, a.norm = _dtype_code(q1), int(causal), int(norm)
    a.q1, a.k1, a.q2, a.k2, a.v = (_ptr(t) for t in (q1, k1, q2, k2, v))
    a.q_stride, a.k_stride, a.v_stride, a.o_stride = (_strides3(t) for t in (q1, k1, v, out))
    _lambda_fields(a, lambda_vecs, lambda_fixed)
    a.lambda_init, a.softmax_scale, a.eps = float(lambda_init), float(softmax_scale), float(eps)
    a.out = _ptr(out)
    lam = lambda_out if lambda_out is not None else torch.empty(1, dtype=torch.float32, device=v.device)
    a.lambda_out = _ptr(lam)
    saves = None
    if save:
        f32 = dict(dtype=torch.float32, device=v.device)
        saves = {"lse1": torch.empty((B, H, S), **f32), "lse2": torch.empty((B, H, S), **f32),
                 "rstd": torch.empty((B, H, S), **f32), "o_pre": torch.empty((B, S, H, dv), **f32),
                 "a2": torch.empty((B, S, H, dv), **f32), "lambda": lam}
        a.lse1, a.lse2, a.rstd, a.o_pre, a.a2 = (_ptr(saves[k]) for k in ("lse1", "lse2", "rstd", "o_pre", "a2"))
    _attach_workspace(a, lib().diffattn_fwd_workspace_size, v.device)
    _check(lib().diffattn_fwd(ctypes.byref(a), _stream()), "diffattn_fwd")
    return (out, saves) if save else out


def fwd_args(q1, k1, q2, k2, v, out, *, lambda_init, lambda_vecs=None, lambda_fixed=0.8,
             causal=True, norm=True, eps=1e-5, softmax_scale=0.0, saves=None):
    """Prebuilt FwdArgs for repeated launches (benchmarks): call
    fwd_launch(args) to run it on the current stream.  saves: optional dict of
    the five float32 training-save tensors (see fwd)."""
    _check_attn(q1, k1, q2, k2, v, out, lambda_vecs)
    B, S, H, d = q1.shape
    a = FwdArgs()
    a.batch, a.seqlen, a.heads, a.head_dim, a.v_dim = B, S, H, d, v.shape[-1]
    a.dtype, a.causal, a.norm = _dtype_code(q1), int(causal), int(norm)
    a.q1, a.k1, a.q2, a.k2, a.v = (_ptr(t) for t in (q1, k1, q2, k2, v))
    a.q_stride, a.k_stride, a.v_stride, a.o_stride = (_strides3(t) for t in (q1, k1, v, out))
    _lambda_fields(a, lambda_vecs, lambda_fixed)
    a.lambda_init, a.softmax_scale, a.eps = float(lambda_init), float(softmax_scale), float(eps)
    a.out = _ptr(out)
    if saves is not None:
        dv = v.shape[-1]
        for k, shape in (("lse1", (B, H, S)), ("lse2", (B, H, S)), ("rstd", (B, H, S)),
                         ("o_pre", (B, S, H, dv)), ("a2", (B, S, H, dv))):
            t = saves[k]
            _require(tuple(t.shape) == shape and t.is_contiguous(), f"saved {k} must be contiguous {shape}")
            _check_dev(((k, t),), dtype=torch.float32, device=q1.device)
        a.lse1, a.lse2, a.rstd, a.o_pre, a.a2 = (_ptr(saves[k]) for k in ("lse1", "lse2", "rstd", "o_pre", "a2"))
    return _attach_workspace(a, lib().diffattn_fwd_workspace_size, q1.device)


def fwd_launch(args: FwdArgs) -> None:
    _check(lib().diffattn_fwd(ctypes.byref(args), _stream()), "diffattn_fwd")


def fwd_fp8_workspace(args: FwdArgs, device) -> torch.Tensor:
    """Workspace tensor for diffattn_fwd_fp8 with these arguments."""
    nbytes = int(lib().diffattn_fwd_fp8_workspace_size(ctypes.byref(args)))
    _require(nbytes > 0, "invalid arguments for the fp8-logit forward: " + lib().diffattn_last_error().decode())
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def fwd_fp8_launch(args: FwdArgs, ws: torch.Tensor) -> None:
    _check(lib().diffattn_fwd_fp8(ctypes.byref(args), _ptr(ws), ws.numel(), _stream()), "diffattn_fwd_fp8")


def fwd_fp8(q1, k1, q2, k2, v, *, lambda_init: float, lambda_vecs=None, lambda_fixed: float = 0.8,
            causal: bool = True, norm: bool = True, eps: float = 1e-5, softmax_scale: float = 0.0, out=None,
            return_workspace: bool = False):
    """Forward with fp8 e4m3 attention logits through diffattn_fwd_fp8 (per-row
    power-of-two absmax quantisation of Q1, K1, Q2, K2).  Returns out, or
    (out, workspace) with return_workspace=True: the workspace then holds the
    codes (uint8 [4, B, H, S, d]: Q1, K1, Q2, K2) followed, at the next
    256-byte boundary, by the exponents (int32 [4, B, H, S])."""
    B, S, H, d = q1.shape
    if out is None:
        out = torch.empty((B, S, H, v.shape[-1]), dtype=v.dtype, device=v.device)
    a = fwd_args(q1, k1, q2, k2, v, out, lambda_init=lambda_init, lambda_vecs=lambda_vecs,
                 lambda_fixed=lambda_fixed, causal=causal, norm=norm, eps=eps, softmax_scale=softmax_scale)
    ws = fwd_fp8_workspace(a, v.device)
    fwd_fp8_launch(a, ws)
    return (out, ws) if return_workspace else out


def bwd_args(q1, k1, q2, k2, v, dout, saves, *, lambda_init: float, lambda_vecs=None,
             lambda_fixed: float = 0.8, causal: bool = True, norm: bool = True, softmax_scale: float = 0.0):
    """Prebuilt BwdArgs with its outputs and workspace allocated: returns
    (args, grads, workspace); bwd_launch(args) runs it on the current stream."""
    _check_attn(q1, k1, q2, k2, v, dout, lambda_vecs)
    B, S, H, d = q1.shape
    dv_w0 = v.shape[-1]
    for k, shape in (("lse1", (B, H, S)), ("lse2", (B, H, S)), ("rstd", (B, H, S)),
                     ("o_pre", (B, S, H, dv_w0)), ("a2", (B, S, H, dv_w0))):
        t = saves[k]
        _require(tuple(t.shape) == shape and t.is_contiguous(), f"saved {k} must be contiguous {shape}")
        _check_dev(((k, t),), dtype=torch.float32, device=q1.device)
    dv_w = v.shape[-1]
    g = {k: torch.empty_like(t) for k, t in (("dq1", q1), ("dk1", k1), ("dq2", q2), ("dk2", k2), ("dv", v))}
    a = BwdArgs()
    a.batch, a.seqlen, a.heads, a.head_dim, a.v_dim = B, S, H, d, dv_w
    a.dtype, a.causal, a.norm = _dtype_code(q1), int(causal), int(norm)
    a.q1, a.k1, a.q2, a.k2, a.v = (_ptr(t) for t in (q1, k1, q2, k2, v))
    a.q_stride, a.k_stride, a.v_stride = (_strides3(t) for t in (q1, k1, v))
    a.dout, a.do_stride = _ptr(dout), _strides3(dout)
    _lambda_fields(a, lambda_vecs, lambda_fixed)
    a.lambda_init, a.softmax_scale = float(lambda_init), float(softmax_scale)
    a.lse1, a.lse2, a.rstd, a.o_pre, a.a2 = (_ptr(saves[k]) for k in ("lse1", "lse2", "rstd", "o_pre", "a2"))
    a.dq1, a.dk1, a.dq2, a.dk2, a.dv = (_ptr(g[k]) for k in ("dq1", "dk1", "dq2", "dk2", "dv"))
    a.dq_stride, a.dk_stride, a.dv_stride = (_strides3(g[k]) for k in ("dq1", "dk1", "dv"))
    g["dlambda"] = torch.empty(1, dtype=torch.float32, device=v.device)
    a.dlambda = _ptr(g["dlambda"])
    if lambda_vecs is not None:
        for name, vec in zip(("dlq1", "dlk1", "dlq2", "dlk2"), lambda_vecs):
            g[name] = torch.empty_like(vec)
        a.dlq1, a.dlk1, a.dlq2, a.dlk2 = (_ptr(g[k]) for k in ("dlq1", "dlk1", "dlq2", "dlk2"))
    nbytes = lib().diffattn_bwd_workspace_size(ctypes.byref(a))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=v.device)
    a.workspace, a.workspace_bytes = _ptr(ws), nbytes
    return a, g, ws


def bwd_launch(args: BwdArgs) -> None:
    _check(lib().diffattn_bwd(ctypes.byref(args), _stream()), "diffattn_bwd")


def bwd(q1, k1, q2, k2, v, dout, saves, *, lambda_init: float, lambda_vecs=None,
        lambda_fixed: float = 0.8, causal: bool = True, norm: bool = True,
        softmax_scale: float = 0.0):
    """Gradients through diffattn_bwd for the forward run with save=True.

    Returns a dict: dq1, dk1, dq2, dk2, dv (activation dtype), dlambda
    (float32 [1]) and, with lambda_vecs, dlq1, dlk1, dlq2, dlk2."""
    a, g, ws = bwd_args(q1, k1, q2, k2, v, dout, saves, lambda_init=lambda_init, lambda_vecs=lambda_vecs,
                        lambda_fixed=lambda_fixed, causal=causal, norm=norm, softmax_scale=softmax_scale)
    bwd_launch(a)
    del ws  # the stream-ordered caching allocator keeps it alive until the kernels have run
    return g


def decode_args(q, k_cache, v_cache, lam, out, *, seqlens=None, softmax_scale=0.0, num_splits=0):
    """DecodeArgs for q [B,Hq,D], caches [B,S_kv,Hkv,D], lam [Hq/2] or [B,Hq/2],
    out [B,Hq/2,D] (workspace not yet attached)."""
    _require(q.dim() == 3 and k_cache.dim() == 4, "q must be [B, Hq, D], caches [B, S_kv, Hkv, D]")
    B, Hq, D = q.shape
    _require(k_cache.shape[0] == B and k_cache.shape[3] == D, "cache shape does not match q")
    _require(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache shapes differ")
    _require(tuple(out.shape) == (B, Hq // 2, D), "out must be [B, Hq/2, D]")
    _check_dev((("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("out", out)), dtype=q.dtype,
               device=q.device)
    _require(lam.dtype == torch.float32 and lam.is_cuda and lam.device == q.device, "lam: float32 on q's GPU")
    _require(tuple(lam.shape) in ((Hq // 2,), (B, Hq // 2)) and lam.stride(-1) == 1, "lam must be [Hq/2] or [B, Hq/2]")
    if seqlens is not None:
        _require(seqlens.dtype == torch.int32 and seqlens.is_cuda and seqlens.device == q.device
                 and tuple(seqlens.shape) == (B,) and seqlens.is_contiguous(), "seqlens: int32 [B] on q's GPU")
    a = DecodeArgs()
    a.batch, a.q_heads, a.kv_heads, a.head_dim, a.kv_len = B, Hq, k_cache.shape[2], D, k_cache.shape[1]
    a.dtype = _dtype_code(q)
    a.q, a.q_stride = _ptr(q), (c_i64 * 2)(q.stride(0), q.stride(1))
    if k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    a.k_cache, a.v_cache, a.kv_stride = _ptr(k_cache), _ptr(v_cache), _strides3(k_cache)
    a.seqlens = _ptr(seqlens)
    a.lam = _ptr(lam)
    a.lam_stride_b = 0 if lam.dim() == 1 else lam.stride(0)
    a.softmax_scale = float(softmax_scale)
    a.out, a.o_stride = _ptr(out), (c_i64 * 2)(out.stride(0), out.stride(1))
    a.num_splits = int(num_splits)
    return a


def decode_workspace_size(args: DecodeArgs) -> int:
    return int(lib().diffattn_v2_decode_workspace_size(ctypes.byref(args)))


def decode_launch(args: DecodeArgs) -> None:
    _check(lib().diffattn_v2_decode(ctypes.byref(args), _stream()), "diffattn_v2_decode")


DECODE_SCRATCH_BYTES = 32 << 20   # DIFFATTN_DECODE_SCRATCH_BYTES


def decode_noalloc_launch(args: DecodeArgs) -> None:
    """diffattn_v2_decode_noalloc: the split partials go to the library's fixed
    per-GPU scratch (args.workspace is ignored)."""
    _check(lib().diffattn_v2_decode_noalloc(ctypes.byref(args), _stream()), "diffattn_v2_decode_noalloc")


def v2_decode(q, k_cache, v_cache, lam, *, seqlens=None, softmax_scale: float = 0.0,
              num_splits: int = 0, out=None):
    """DIFF V2 decode through diffattn_v2_decode; returns out [B, Hq/2, D]."""
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq // 2, D), dtype=q.dtype, device=q.device)
    a = decode_args(q, k_cache, v_cache, lam, out, seqlens=seqlens, softmax_scale=softmax_scale,
                    num_splits=num_splits)
    nbytes = decode_workspace_size(a)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    a.workspace, a.workspace_bytes = _ptr(ws), nbytes
    decode_launch(a)
    return out


def _lam_strides(lam, B, S, P):
    shapes = {1: (P,), 2: (S, P), 3: (B, S, P)}
    _require(lam.dim() in shapes and tuple(lam.shape) == shapes[lam.dim()],
             "lam must be [Hq/2], [S, Hq/2] or [B, S, Hq/2]")
    return (c_i64 * 3)(*((0,) * (3 - lam.dim()) + tuple(lam.stride())))


def v2_fwd_args(q, k, v, lam, out, *, causal=True, softmax_scale=0.0, saves=None):
    """V2FwdArgs for q [B,S,Hq,D], k, v [B,S,Hkv,D], out [B,S,Hq/2,D] and lam
    [Hq/2], [S, Hq/2] or [B, S, Hq/2] (float32; missing leading axes
    broadcast).  saves: optional dict of float32 training-save tensors lse
    [B,Hq,S], a_even and a_odd [B,S,Hq/2,D] (contiguous)."""
    _require(q.dim() == 4 and k.dim() == 4, "q must be [B, S, Hq, D], k and v [B, S, Hkv, D]")
    B, S, Hq, D = q.shape
    _require(k.shape[0] == B and k.shape[1] == S and k.shape[3] == D, "k shape does not match q")
    _require(tuple(v.shape) == tuple(k.shape), "k and v shapes differ")
    _require(tuple(out.shape) == (B, S, Hq // 2, D), "out must be [B, S, Hq/2, D]")
    _check_dev((("q", q), ("k", k), ("v", v), ("out", out)), dtype=q.dtype, device=q.device)
    _require(lam.dtype == torch.float32 and lam.is_cuda and lam.device == q.device, "lam: float32 on q's GPU")
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    a = V2FwdArgs()
    a.batch, a.seqlen, a.q_heads, a.kv_heads, a.head_dim = B, S, Hq, k.shape[2], D
    a.dtype, a.causal = _dtype_code(q), int(bool(causal))
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.q_stride, a.kv_stride = _strides3(q), _strides3(k)
    a.lam, a.lam_stride = _ptr(lam), _lam_strides(lam, B, S, Hq // 2)
    a.softmax_scale = float(softmax_scale)
    a.out, a.o_stride = _ptr(out), _strides3(out)
    if saves is not None:
        for name, shape in (("lse", (B, Hq, S)), ("a_even", (B, S, Hq // 2, D)), ("a_odd", (B, S, Hq // 2, D))):
            t = saves[name]
            _require(t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shape
                     and t.device == q.device, f"{name}: contiguous float32 {shape} on q's GPU")
        a.lse, a.a_even, a.a_odd = _ptr(saves["lse"]), _ptr(saves["a_even"]), _ptr(saves["a_odd"])
    return _attach_workspace(a, lib().diffattn_v2_fwd_workspace_size, q.device)


def v2_fwd_launch(args: V2FwdArgs) -> None:
    _check(lib().diffattn_v2_fwd(ctypes.byref(args), _stream()), "diffattn_v2_fwd")


def v2_fwd(q, k, v, lam, *, causal: bool = True, softmax_scale: float = 0.0, out=None, save: bool = False):
    """DIFF V2 prefill forward through diffattn_v2_fwd; returns out [B, S, Hq/2, D],
    or (out, saves) with save=True (the backward's inputs)."""
    B, S, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, S, Hq // 2, D), dtype=q.dtype, device=q.device)
    saves = None
    if save:
        f32 = dict(dtype=torch.float32, device=q.device)
        saves = {"lse": torch.empty((B, Hq, S), **f32), "a_even": torch.empty((B, S, Hq // 2, D), **f32),
                 "a_odd": torch.empty((B, S, Hq // 2, D), **f32)}
    v2_fwd_launch(v2_fwd_args(q, k, v, lam, out, causal=causal, softmax_scale=softmax_scale, saves=saves))
    return (out, saves) if save else out


def v2_bwd_args(q, k, v, lam, dout, saves, dq, dk, dv, dlam, *, causal=True, softmax_scale=0.0):
    """V2BwdArgs (workspace not yet attached); dlam is float32 [B, S, Hq/2]
    contiguous (the per-(batch, token, pair) gradient)."""
    a = V2BwdArgs()
    fa = v2_fwd_args(q, k, v, lam, dout, causal=causal, softmax_scale=softmax_scale, saves=saves)
    B, S, Hq, D = q.shape
    _require(tuple(dq.shape) == tuple(q.shape) and tuple(dk.shape) == tuple(k.shape)
             and tuple(dv.shape) == tuple(v.shape), "dq, dk, dv must match q, k, v")
    _check_dev((("dq", dq), ("dk", dk), ("dv", dv)), dtype=q.dtype, device=q.device)
    if dk.stride() != dv.stride():
        raise ValueError("dk and dv must share strides")
    _require(dlam.dtype == torch.float32 and dlam.is_contiguous() and tuple(dlam.shape) == (B, S, Hq // 2)
             and dlam.device == q.device, "dlam: contiguous float32 [B, S, Hq/2] on q's GPU")
    for name, _ in V2FwdArgs._fields_:
        if hasattr(a, name) and name not in ("out", "o_stride"):
            setattr(a, name, getattr(fa, name))
    a.dout, a.do_stride = _ptr(dout), _strides3(dout)
    a.dq, a.dq_stride = _ptr(dq), _strides3(dq)
    a.dk, a.dv, a.dkv_stride = _ptr(dk), _ptr(dv), _strides3(dk)
    a.dlam = _ptr(dlam)
    return a


def v2_bwd_workspace_size(args: V2BwdArgs) -> int:
    return int(lib().diffattn_v2_bwd_workspace_size(ctypes.byref(args)))


def v2_bwd_launch(args: V2BwdArgs) -> None:
    _check(lib().diffattn_v2_bwd(ctypes.byref(args), _stream()), "diffattn_v2_bwd")


def v2_bwd(q, k, v, lam, dout, saves, *, causal: bool = True, softmax_scale: float = 0.0):
    """DIFF V2 prefill backward through diffattn_v2_bwd.  Returns dq, dk, dv and
    dlam, the latter summed over the axes lam broadcast over (lam's shape)."""
    B, S, Hq, D = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dlam = torch.empty((B, S, Hq // 2), dtype=torch.float32, device=q.device)
    a = v2_bwd_args(q, k, v, lam, dout, saves, dq, dk, dv, dlam, causal=causal, softmax_scale=softmax_scale)
    nbytes = v2_bwd_workspace_size(a)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    a.workspace, a.workspace_bytes = _ptr(ws), nbytes
    v2_bwd_launch(a)
    dl = dlam
    if lam.dim() < 3:
        dl = dlam.sum(dim=tuple(range(3 - lam.dim())))
    return {"dq": dq, "dk": dk, "dv": dv, "dlam": dl}


def v1_decode_args(q1, q2, k1_cache, k2_cache, v_cache, out, *, lambda_init: float, lambda_vecs=None,
                   lambda_fixed: float = 0.8, norm: bool = True, eps: float = 1e-5, seqlens=None,
                   softmax_scale: float = 0.0, num_splits: int = 0):
    """V1DecodeArgs for q1, q2 [B,H,d], k1_cache, k2_cache [B,S_kv,H,d],
    v_cache [B,S_kv,H,dv], out [B,H,dv] (workspace not yet attached)."""
    _require(q1.dim() == 3 and k1_cache.dim() == 4 and v_cache.dim() == 4,
             "q must be [B, H, d], caches [B, S_kv, H, c]")
    B, H, d = q1.shape
    _require(tuple(q2.shape) == (B, H, d) and q2.stride() == q1.stride(), "q1 and q2 must share shape and strides")
    _require(k1_cache.shape[0] == B and k1_cache.shape[2] == H and k1_cache.shape[3] == d,
             "k cache shape does not match q")
    _require(tuple(k2_cache.shape) == tuple(k1_cache.shape) and k2_cache.stride() == k1_cache.stride(),
             "k1_cache and k2_cache must share shape and strides")
    _require(tuple(v_cache.shape[:3]) == tuple(k1_cache.shape[:3]), "v_cache must be [B, S_kv, H, dv]")
    dv = v_cache.shape[3]
    _require(tuple(out.shape) == (B, H, dv), "out must be [B, H, dv]")
    _check_dev((("q1", q1), ("q2", q2), ("k1_cache", k1_cache), ("k2_cache", k2_cache), ("v_cache", v_cache),
                ("out", out)), dtype=q1.dtype, device=q1.device)
    if seqlens is not None:
        _require(seqlens.dtype == torch.int32 and seqlens.is_cuda and seqlens.device == q1.device
                 and tuple(seqlens.shape) == (B,) and seqlens.is_contiguous(), "seqlens: int32 [B] on q's GPU")
    a = V1DecodeArgs()
    a.batch, a.heads, a.head_dim, a.v_dim, a.kv_len = B, H, d, dv, k1_cache.shape[1]
    a.dtype, a.norm = _dtype_code(q1), int(bool(norm))
    a.q1, a.q2, a.q_stride = _ptr(q1), _ptr(q2), (c_i64 * 2)(q1.stride(0), q1.stride(1))
    a.k1_cache, a.k2_cache, a.k_stride = _ptr(k1_cache), _ptr(k2_cache), _strides3(k1_cache)
    a.v_cache, a.v_stride = _ptr(v_cache), _strides3(v_cache)
    a.seqlens = _ptr(seqlens)
    if lambda_vecs is not None:
        _require(len(lambda_vecs) == 4, "lambda_vecs must hold lq1, lk1, lq2, lk2")
        n = lambda_vecs[0].numel()
        for t in lambda_vecs:
            _require(t.is_contiguous() and t.numel() == n and t.dim() == 1, "lambda vectors: 1-D, contiguous, equal length")
        _check_dev((("lambda_vec%d" % i, t) for i, t in enumerate(lambda_vecs)), dtype=torch.float32, device=q1.device)
        a.lq1, a.lk1, a.lq2, a.lk2 = (_ptr(t) for t in lambda_vecs)
        a.lambda_dim = n
    a.lambda_fixed, a.lambda_init = float(lambda_fixed), float(lambda_init)
    a.softmax_scale, a.eps = float(softmax_scale), float(eps)
    a.out, a.o_stride = _ptr(out), (c_i64 * 2)(out.stride(0), out.stride(1))
    a.num_splits = int(num_splits)
    return a


def v1_decode_workspace_size(args: V1DecodeArgs) -> int:
    return int(lib().diffattn_v1_decode_workspace_size(ctypes.byref(args)))


def v1_decode_launch(args: V1DecodeArgs) -> None:
    _check(lib().diffattn_v1_decode(ctypes.byref(args), _stream()), "diffattn_v1_decode")


def v1_decode(q1, q2, k1_cache, k2_cache, v_cache, *, lambda_init: float, lambda_vecs=None,
              lambda_fixed: float = 0.8, norm: bool = True, eps: float = 1e-5, seqlens=None,
              softmax_scale: float = 0.0, num_splits: int = 0, out=None):
    """DIFF V1 decode step through diffattn_v1_decode; returns out [B, H, dv]."""
    B, H, _ = q1.shape
    if out is None:
        out = torch.empty((B, H, v_cache.shape[3]), dtype=q1.dtype, device=q1.device)
    a = v1_decode_args(q1, q2, k1_cache, k2_cache, v_cache, out, lambda_init=lambda_init, lambda_vecs=lambda_vecs,
                       lambda_fixed=lambda_fixed, norm=norm, eps=eps, seqlens=seqlens,
                       softmax_scale=softmax_scale, num_splits=num_splits)
    nbytes = v1_decode_workspace_size(a)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q1.device)
    a.workspace, a.workspace_bytes = _ptr(ws), nbytes
    v1_decode_launch(a)
    return out


def v2_block_lists(block_mask: torch.Tensor):
    """(block_idx, block_cnt) int32 device tensors from a bool block mask
    [B, Hq/2, ceil(S/128), ceil(S/64)] (host or device): the selected 64-key
    tiles of each (batch, pair, query tile), ascending."""
    m = block_mask.to(torch.bool)
    cnt = m.sum(dim=-1).to(torch.int32)
    max_blocks = max(int(cnt.max().item()), 1)
    n_kb = m.shape[-1]
    ar = torch.arange(n_kb, device=m.device).expand_as(m)
    key = torch.where(m, ar, ar + n_kb)                  # selected tiles first, in order
    idx = torch.sort(key, dim=-1).values[..., :max_blocks].to(torch.int32)
    idx = torch.where(idx < n_kb, idx, torch.full_like(idx, -1))
    return idx.contiguous(), cnt.contiguous()


def v2_fwd_sparse_launch(args: V2FwdArgs, block_idx, block_cnt) -> None:
    _check(lib().diffattn_v2_fwd_sparse(ctypes.byref(args), _ptr(block_idx), _ptr(block_cnt),
                                        int(block_idx.shape[-1]), _stream()), "diffattn_v2_fwd_sparse")


def v2_fwd_sparse(q, k, v, lam, block_idx, block_cnt, *, causal: bool = True, softmax_scale: float = 0.0, out=None):
    """Block-sparse DIFF V2 prefill forward through diffattn_v2_fwd_sparse;
    block_idx [B, Hq/2, ceil(S/128), max_blocks], block_cnt [B, Hq/2,
    ceil(S/128)] (int32 on q's GPU, e.g. from v2_block_lists)."""
    B, S, Hq, D = q.shape
    n_qt = (S + 127) // 128
    _require(block_idx.dtype == torch.int32 and block_cnt.dtype == torch.int32 and block_idx.is_cuda
             and block_cnt.is_cuda and block_idx.device == q.device and block_cnt.device == q.device,
             "block lists: int32 on q's GPU")
    _require(tuple(block_cnt.shape) == (B, Hq // 2, n_qt) and block_cnt.is_contiguous(),
             "block_cnt must be contiguous [B, Hq/2, ceil(S/128)]")
    _require(block_idx.dim() == 4 and tuple(block_idx.shape[:3]) == (B, Hq // 2, n_qt) and block_idx.is_contiguous(),
             "block_idx must be contiguous [B, Hq/2, ceil(S/128), max_blocks]")
    if out is None:
        out = torch.empty((B, S, Hq // 2, D), dtype=q.dtype, device=q.device)
    v2_fwd_sparse_launch(v2_fwd_args(q, k, v, lam, out, causal=causal, softmax_scale=softmax_scale), block_idx,
                         block_cnt)
    return out
