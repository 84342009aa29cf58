"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every function include/diffattn.h declares, and rejects bad arguments before
any launch.  The rejection checks hand the library stand-in addresses, so they
run only where no GPU is visible: there a call that wrongly passed
validation could not launch anything."""
import ctypes
import math
import os
import re

import pytest

from differential_attention_02_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "diffattn.h")
FAKE = 1 << 20  # 16-byte aligned non-NULL stand-in address; never dereferenced
host_only = pytest.mark.skipif(__import__("torch").cuda.is_available(),
                               reason="passes stand-in addresses; host-only")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(diffattn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = _declared_functions()
    assert len(names) == 19
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.SIGNATURES)


def test_struct_sizes_match_layout():
    # int32 x8 + 5 ptr + 4 x int64[3] + 4 ptr + int32 + 4 float + 7 ptr + workspace ptr and size
    assert ctypes.sizeof(B.FwdArgs) == 32 + 40 + 96 + 32 + 20 + 4 + 56 + 16
    assert ctypes.sizeof(B.DecodeArgs) % 8 == 0


def test_lambda_init_and_status_strings():
    lib = B.lib()
    assert lib.diffattn_lambda_init(1) == pytest.approx(0.2, abs=1e-7)
    assert lib.diffattn_lambda_init(12) == pytest.approx(0.8 - 0.6 * math.exp(-3.3), abs=1e-6)
    assert math.isnan(lib.diffattn_lambda_init(0))
    assert lib.diffattn_status_str(0) == b"ok"
    assert lib.diffattn_status_str(-3).startswith(b"workspace")


def _fwd_args(**kw):
    a = B.FwdArgs()
    a.batch, a.seqlen, a.heads, a.head_dim, a.v_dim = 1, 128, 2, 64, 128
    a.dtype, a.causal, a.norm = B.BF16, 1, 1
    a.q1 = a.k1 = a.q2 = a.k2 = a.v = a.out = FAKE
    for name in ("q_stride", "k_stride", "o_stride"):
        setattr(a, name, (ctypes.c_int64 * 3)(128 * 2 * 64, 2 * 64, 64))
    a.v_stride = (ctypes.c_int64 * 3)(128 * 2 * 128, 2 * 128, 128)
    a.o_stride = (ctypes.c_int64 * 3)(128 * 2 * 128, 2 * 128, 128)
    a.lambda_fixed, a.lambda_init, a.eps = 0.8, 0.2, 1e-5
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _fwd(a):
    return B.lib().diffattn_fwd(ctypes.byref(a), None)


def test_fwd_empty_problem_is_ok():
    """batch or seqlen 0: nothing to read or write, NULL pointers allowed."""
    a = B.FwdArgs()
    a.batch, a.seqlen, a.heads, a.head_dim, a.v_dim = 0, 128, 2, 64, 128
    assert _fwd(a) == 0
    a.batch, a.seqlen = 3, 0
    assert _fwd(a) == 0
    a.seqlen = -1
    assert _fwd(a) == -1


@host_only
@pytest.mark.parametrize("field,value,code", [
    ("heads", 0, -1), ("head_dim", 0, -1), ("dtype", 7, -1), ("q1", None, -1), ("v", None, -1),
    ("out", None, -1), ("eps", -1.0, -1), ("eps", float("nan"), -1), ("lambda_fixed", float("inf"), -1),
    ("lambda_init", float("nan"), -1), ("softmax_scale", float("nan"), -1),
    ("head_dim", 48, -2), ("v_dim", 64, -2), ("q1", FAKE + 2, -2),
    ("lq1", FAKE, -1), ("lse1", FAKE, -1),
])
def test_fwd_rejects(field, value, code):
    a = _fwd_args(**{field: value})
    assert _fwd(a) == code
    assert B.lib().diffattn_last_error() != b""


@host_only
def test_fwd_rejects_bad_strides():
    a = _fwd_args()
    a.k_stride = (ctypes.c_int64 * 3)(1, 0, 64)
    assert _fwd(a) == -1
    a = _fwd_args()
    a.k_stride = (ctypes.c_int64 * 3)(128 * 2 * 64, 2 * 64 + 4, 64)   # rows not 16-byte aligned
    assert _fwd(a) == -2


@host_only
@pytest.mark.parametrize("field,value,code", [
    ("dtype", B.F32, -2), ("head_dim", 32, -2), ("lse1", FAKE, -1), ("q1", FAKE + 4, -2), ("out", None, -1),
])
def test_fwd_fp8_rejects(field, value, code):
    a = _fwd_args(**{field: value})
    if field == "lse1":   # all five saves: a valid training request, which this entry point refuses
        a.lse2 = a.rstd = a.o_pre = a.a2 = FAKE
        code = -2
    assert B.lib().diffattn_fwd_fp8(ctypes.byref(a), FAKE, 1 << 40, None) == code
    assert B.lib().diffattn_last_error() != b""


def test_fwd_fp8_workspace_size():
    a = _fwd_args()
    n = B.lib().diffattn_fwd_fp8_workspace_size(ctypes.byref(a))
    rows = 1 * 2 * 128
    assert n >= 4 * rows * 64 + 4 * rows * 4


@host_only
def test_fwd_fp8_rejects_small_workspace():
    a = _fwd_args()
    n = B.lib().diffattn_fwd_fp8_workspace_size(ctypes.byref(a))
    assert B.lib().diffattn_fwd_fp8(ctypes.byref(a), FAKE, n - 1, None) == -3
    assert B.lib().diffattn_fwd_fp8(ctypes.byref(a), FAKE + 16, n, None) == -1


@host_only
def test_fwd_training_saves_need_fused_path():
    a = _fwd_args(dtype=B.F32, lse1=FAKE, lse2=FAKE, rstd=FAKE, o_pre=FAKE, a2=FAKE)
    assert _fwd(a) == -2


def _dec_args(**kw):
    a = B.DecodeArgs()
    a.batch, a.q_heads, a.kv_heads, a.head_dim, a.kv_len = 1, 32, 16, 128, 8192
    a.dtype = B.BF16
    a.q = a.k_cache = a.v_cache = a.out = a.lam = FAKE
    a.q_stride = (ctypes.c_int64 * 2)(32 * 128, 128)
    a.kv_stride = (ctypes.c_int64 * 3)(8192 * 16 * 128, 16 * 128, 128)
    a.o_stride = (ctypes.c_int64 * 2)(16 * 128, 128)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_decode_workspace_and_empty_call():
    lib = B.lib()
    a = _dec_args(batch=64)
    n = lib.diffattn_v2_decode_workspace_size(ctypes.byref(a))
    assert n > 0 and n % (64 * 32 * 130 * 4) == 0   # [B, Hq, splits, D + 2] float32
    a = B.DecodeArgs()
    a.batch = 0
    assert lib.diffattn_v2_decode(ctypes.byref(a), None) == 0


@host_only
def test_decode_noalloc_empty_and_oversized():
    """The allocation-free decode: an empty batch is OK, and a call whose split
    partials exceed the fixed scratch is rejected on the host (no launch)."""
    a = _dec_args(batch=0)
    assert B.lib().diffattn_v2_decode_noalloc(ctypes.byref(a), None) == 0
    a = _dec_args(batch=4, q_heads=4, kv_heads=2, kv_len=20000, num_splits=20000)
    a.q_stride = (ctypes.c_int64 * 2)(4 * 128, 128)
    a.kv_stride = (ctypes.c_int64 * 3)(20000 * 2 * 128, 2 * 128, 128)
    a.o_stride = (ctypes.c_int64 * 2)(2 * 128, 128)
    assert B.lib().diffattn_v2_decode_workspace_size(ctypes.byref(a)) > B.DECODE_SCRATCH_BYTES
    assert B.lib().diffattn_v2_decode_noalloc(ctypes.byref(a), None) == -3
    assert b"scratch" in B.lib().diffattn_last_error()


def test_decode_rejects_small_workspace():
    lib = B.lib()
    a = _dec_args(batch=64)
    n = lib.diffattn_v2_decode_workspace_size(ctypes.byref(a))
    a.workspace, a.workspace_bytes = None, n
    assert lib.diffattn_v2_decode(ctypes.byref(a), None) == -3
    a.workspace, a.workspace_bytes = FAKE, n - 1
    assert lib.diffattn_v2_decode(ctypes.byref(a), None) == -3


@host_only
@pytest.mark.parametrize("field,value,code", [
    ("q_heads", 24, -1),        # group of 24/16 is not an integer
    ("kv_heads", 32, -1),       # group of 1: a pair would straddle two KV heads
    ("head_dim", 96, -2), ("dtype", 3, -1), ("lam", None, -1), ("k_cache", None, -1),
    ("num_splits", -1, -1), ("num_splits", 2, -1),   # 4096 keys per split is above the chunk limit
    ("lam_stride_b", -1, -1),
])
def test_decode_rejects(field, value, code):
    a = _dec_args(**{field: value})
    a.workspace, a.workspace_bytes = FAKE, 1 << 40
    assert B.lib().diffattn_v2_decode(ctypes.byref(a), None) == code
    assert B.lib().diffattn_v2_decode_workspace_size(ctypes.byref(a)) == 0


def _v2_args(**kw):
    a = B.V2FwdArgs()
    a.batch, a.seqlen, a.q_heads, a.kv_heads, a.head_dim = 1, 256, 4, 2, 128
    a.dtype, a.causal = B.BF16, 1
    a.q = a.k = a.v = a.out = a.lam = FAKE
    a.q_stride = (ctypes.c_int64 * 3)(256 * 4 * 128, 4 * 128, 128)
    a.kv_stride = (ctypes.c_int64 * 3)(256 * 2 * 128, 2 * 128, 128)
    a.o_stride = (ctypes.c_int64 * 3)(256 * 2 * 128, 2 * 128, 128)
    a.lam_stride = (ctypes.c_int64 * 3)(0, 0, 1)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@host_only
@pytest.mark.parametrize("blk,cnt,maxb,code", [(None, FAKE, 4, -1), (FAKE, None, 4, -1), (FAKE, FAKE, 0, -1),
                                               (FAKE, FAKE, 1025, -1)])
def test_v2_fwd_sparse_rejects(blk, cnt, maxb, code):
    a = _v2_args()
    assert B.lib().diffattn_v2_fwd_sparse(ctypes.byref(a), blk, cnt, maxb, None) == code
    a = _v2_args(lse=FAKE, a_even=FAKE, a_odd=FAKE)
    assert B.lib().diffattn_v2_fwd_sparse(ctypes.byref(a), FAKE, FAKE, 4, None) == -2


def test_v2_fwd_empty_problem_is_ok():
    a = B.V2FwdArgs()
    a.batch, a.seqlen, a.q_heads, a.kv_heads, a.head_dim, a.dtype = 0, 64, 4, 2, 128, B.BF16
    assert B.lib().diffattn_v2_fwd(ctypes.byref(a), None) == 0
    a.batch, a.seqlen = 2, 0
    assert B.lib().diffattn_v2_fwd(ctypes.byref(a), None) == 0
    a.seqlen = -3
    assert B.lib().diffattn_v2_fwd(ctypes.byref(a), None) == -1


@host_only
@pytest.mark.parametrize("field,value,code", [
    ("q_heads", 3, -1),          # not a multiple of kv_heads
    ("kv_heads", 4, -1),         # group of 1: a pair would straddle two KV heads
    ("dtype", 5, -1), ("q", None, -1), ("lam", None, -1), ("out", None, -1),
    ("softmax_scale", float("nan"), -1),
    ("lam_stride", (ctypes.c_int64 * 3)(0, -1, 1), -1),
    ("kv_stride", (ctypes.c_int64 * 3)(1, 0, 128), -1),
    ("head_dim", 64, -2), ("dtype", B.F32, -2), ("k", FAKE + 4, -2),
    ("q_stride", (ctypes.c_int64 * 3)(256 * 4 * 128, 4 * 128 + 2, 128), -2),
    ("seqlen", 1 << 22, -2),     # 32-bit key-tile offsets would overflow
])
def test_v2_fwd_rejects(field, value, code):
    a = _v2_args(**{field: value})
    assert B.lib().diffattn_v2_fwd(ctypes.byref(a), None) == code
    assert B.lib().diffattn_last_error() != b""


@host_only
def test_v2_fwd_saves_all_or_none():
    a = _v2_args(lse=FAKE)
    assert B.lib().diffattn_v2_fwd(ctypes.byref(a), None) == -1


def _v2b_args(**kw):
    a = B.V2BwdArgs()
    f = _v2_args()
    for name, _ in B.V2BwdArgs._fields_:
        if hasattr(f, name):
            setattr(a, name, getattr(f, name))
    a.dout = a.dq = a.dk = a.dv = a.dlam = FAKE
    a.lse = a.a_even = a.a_odd = FAKE
    a.do_stride = (ctypes.c_int64 * 3)(256 * 2 * 128, 2 * 128, 128)
    a.dq_stride = (ctypes.c_int64 * 3)(256 * 4 * 128, 4 * 128, 128)
    a.dkv_stride = (ctypes.c_int64 * 3)(256 * 2 * 128, 2 * 128, 128)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_v2_bwd_workspace_and_empty_call():
    lib = B.lib()
    a = _v2b_args()
    n = lib.diffattn_v2_bwd_workspace_size(ctypes.byref(a))
    assert n >= 1 * 2 * 256 * 128 * 2 * 3   # fp16 g' and Q_e | Q_o rows
    a.batch = 0
    assert lib.diffattn_v2_bwd(ctypes.byref(a), None) == 0
    assert lib.diffattn_v2_bwd_workspace_size(ctypes.byref(a)) == 0


@host_only
@pytest.mark.parametrize("field,value,code", [
    ("lse", None, -1), ("a_odd", None, -1), ("dlam", None, -1), ("dout", None, -1), ("dk", None, -1),
    ("q_heads", 6, -1), ("head_dim", 64, -2), ("dq", FAKE + 8, -2),
    ("do_stride", (ctypes.c_int64 * 3)(1, 0, 128), -1),
])
def test_v2_bwd_rejects(field, value, code):
    a = _v2b_args(**{field: value})
    a.workspace, a.workspace_bytes = FAKE, 1 << 40
    assert B.lib().diffattn_v2_bwd(ctypes.byref(a), None) == code
    assert B.lib().diffattn_last_error() != b""


@host_only
def test_v2_bwd_rejects_small_workspace():
    lib = B.lib()
    a = _v2b_args()
    n = lib.diffattn_v2_bwd_workspace_size(ctypes.byref(a))
    a.workspace, a.workspace_bytes = FAKE, n - 1
    assert lib.diffattn_v2_bwd(ctypes.byref(a), None) == -3
    a.workspace, a.workspace_bytes = FAKE + 16, n
    assert lib.diffattn_v2_bwd(ctypes.byref(a), None) == -1


def _v1d_args(**kw):
    a = B.V1DecodeArgs()
    a.batch, a.heads, a.head_dim, a.v_dim, a.kv_len = 2, 16, 64, 128, 8192
    a.dtype, a.norm = B.BF16, 1
    a.q1 = a.q2 = a.k1_cache = a.k2_cache = a.v_cache = a.out = FAKE
    a.q_stride = (ctypes.c_int64 * 2)(16 * 64, 64)
    a.k_stride = (ctypes.c_int64 * 3)(8192 * 16 * 64, 16 * 64, 64)
    a.v_stride = (ctypes.c_int64 * 3)(8192 * 16 * 128, 16 * 128, 128)
    a.o_stride = (ctypes.c_int64 * 2)(16 * 128, 128)
    a.lambda_fixed, a.lambda_init, a.eps = 0.8, 0.2, 1e-5
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_v1_decode_workspace_and_empty_call():
    lib = B.lib()
    a = _v1d_args()
    n = lib.diffattn_v1_decode_workspace_size(ctypes.byref(a))
    assert n > 0 and n % (2 * 16 * 2 * 130 * 4) == 0   # [B, H, 2 maps, splits, dv + 2] float32
    a.batch = 0
    assert lib.diffattn_v1_decode(ctypes.byref(a), None) == 0


@host_only
@pytest.mark.parametrize("field,value,code", [
    ("heads", 0, -1), ("dtype", 4, -1), ("q2", None, -1), ("k2_cache", None, -1), ("out", None, -1),
    ("head_dim", 32, -2), ("v_dim", 64, -2), ("v_cache", FAKE + 8, -2),
    ("lq1", FAKE, -1), ("eps", -1.0, -1), ("num_splits", 2, -1), ("num_splits", -1, -1),
    ("k_stride", (ctypes.c_int64 * 3)(8192 * 16 * 64, 16 * 64 + 4, 64), -2),
])
def test_v1_decode_rejects(field, value, code):
    a = _v1d_args(**{field: value})
    a.workspace, a.workspace_bytes = FAKE, 1 << 40
    assert B.lib().diffattn_v1_decode(ctypes.byref(a), None) == code
    assert B.lib().diffattn_last_error() != b""


@host_only
def test_v1_decode_rejects_small_workspace():
    lib = B.lib()
    a = _v1d_args()
    n = lib.diffattn_v1_decode_workspace_size(ctypes.byref(a))
    a.workspace, a.workspace_bytes = FAKE, n - 1
    assert lib.diffattn_v1_decode(ctypes.byref(a), None) == -3


def test_bwd_rejects_without_saves():
    a = B.BwdArgs()
    a.batch, a.seqlen, a.heads, a.head_dim, a.v_dim = 1, 128, 2, 64, 128
    a.dtype, a.causal, a.norm = B.BF16, 1, 1
    a.q1 = a.k1 = a.q2 = a.k2 = a.v = a.dout = FAKE
    a.dq1 = a.dk1 = a.dq2 = a.dk2 = a.dv = FAKE
    for name in ("q_stride", "k_stride", "do_stride", "dq_stride", "dk_stride"):
        setattr(a, name, (ctypes.c_int64 * 3)(128 * 2 * 64, 2 * 64, 64))
    for name in ("v_stride", "dv_stride", "do_stride"):
        setattr(a, name, (ctypes.c_int64 * 3)(128 * 2 * 128, 2 * 128, 128))
    assert B.lib().diffattn_bwd(ctypes.byref(a), None) == -1
    a.lse1 = a.lse2 = a.rstd = a.o_pre = a.a2 = FAKE
    a.workspace, a.workspace_bytes = FAKE, 1 << 40
    a.lq1 = FAKE   # one vector without the other three
    assert B.lib().diffattn_bwd(ctypes.byref(a), None) == -1


def test_ctypes_layout_matches_c_compiler(tmp_path):
    """Compile a tiny C program against include/diffattn.h and compare struct
    sizes and field offsets with the ctypes mirrors."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    checks = {"diffattn_fwd_args": B.FwdArgs, "diffattn_bwd_args": B.BwdArgs,
              "diffattn_v2_decode_args": B.DecodeArgs, "diffattn_v2_fwd_args": B.V2FwdArgs,
              "diffattn_v2_bwd_args": B.V2BwdArgs, "diffattn_v1_decode_args": B.V1DecodeArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "diffattn.h"', "int main(void) {"]
    for cname, ct in checks.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in ct._fields_:
            lines.append(f'printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    for cname, ct in checks.items():
        assert int(out[cname]) == ctypes.sizeof(ct), cname
        for fname, _ in ct._fields_:
            assert int(out[f"{cname}.{fname}"]) == getattr(ct, fname).offset, (cname, fname)
