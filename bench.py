"""Benchmark of the differential-attention hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu-baseline]

Headline step: one forward pass (diffattn_fwd) over the 3B-class 4K workload
(batch 4, 4096 causal tokens, 12 heads, d 64, dv 128, bf16) with inputs
resident in HBM.  value = algorithmic TFLOP/s: 768 flop per unmasked
(query, key, head) pair (two QK^T products of width 64 and two PV products of
width 128, counted once however the kernel schedules them).
Also reported under "extra": the 64K-token forward, the 8K training step
(forward + backward) when the backward is built, and the DIFF V2 decode step
(GB/s of K/V cache + query + output bytes), and the DIFF V2 prefill forward
(batch 4, 4096 causal tokens, 24 query heads over 12 KV heads, D 128: 1024
flop per unmasked (query, key, pair of query heads), two QK^T and two PV
products of width 128), and its training step (forward with saves + backward,
2048 more flop per unmasked (query, key, pair): recomputed QK^T of both heads,
one shared dP, one merged dV, dQ and dK of both heads), and the DIFF V1 decode
over a K1/K2/V cache (GB/s of cache + query + output bytes), and the
block-sparse DIFF V2 forward over a seeded selection of 16 64-key tiles per
128-row query tile (1024 flop per selected (query, key, pair)).
Each timing: W untimed launches, then exactly K launches between two
synchronisations; HIP events on the launch stream give the average launch
duration used for the roofline.  "cpu_baseline" times the float64 oracle on a
bounded sample of the same workload on the host cores.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "diff-attn fwd TFLOP/s (bf16 causal, 4K seq) + V2 decode HBM GB/s, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
FLOP_PER_PAIR_FWD = 768
FLOP_PER_PAIR_BWD = 1280
FLOP_PER_PAIR_V2 = 8 * 128     # per (query, key, even/odd pair of query heads), D = 128
# V2 backward per (query, key, pair): recomputed Q K^T of both heads 512, shared dP 256, merged dV 256,
# dQ of both heads 512, dK of both heads 512.
FLOP_PER_PAIR_V2_BWD = 16 * 128
PROFILES = os.path.join(ROOT, "profiles")


def _kernel_digest(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def _traffic_from_profile(name, files):
    """HBM bytes per launch recorded by a committed counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    m = re.search(r"^traffic_json: (\{.*\})$", open(path).read(), flags=re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_digest") != _kernel_digest(files):
        return None
    return rec.get("hbm_bytes_per_launch")


_CSRC = "differential_attention_02_amd/csrc/"
# Sources of each timed kernel: a counter summary counts only while their digest matches.
FWD_SOURCES = [_CSRC + f for f in ("fwd_onepass.hip", "vrange.hip", "vrange.h", "attn_tile.h", "common.h")]
V2P_SOURCES = [_CSRC + f for f in ("fwd_v2.hip", "vrange.hip", "vrange.h", "attn_tile.h", "common.h")]
DEC_SOURCES = [_CSRC + f for f in ("decode.hip", "common.h")]
FP8_SOURCES = [_CSRC + f for f in ("fwd_fp8.hip", "vrange.hip", "vrange.h", "attn_tile.h", "common.h")]
BWD_SOURCES = [_CSRC + f for f in ("bwd.hip", "vrange.h", "common.h")]
V2B_SOURCES = [_CSRC + f for f in ("bwd_v2.hip", "vrange.h", "common.h")]
# fp8 leg: per pair, the two score products (256 flop) run at the fp8 peak and the PV products
# (512 flop) at the fp16 peak, so the mixed peak is 768 / (256 / 5000 + 512 / 2500) TFLOP/s.
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP8_MIXED_TFLOPS = FLOP_PER_PAIR_FWD / (256 / PEAK_FP8_TFLOPS + 512 / PEAK_BF16_TFLOPS)


def _time_launches(launch, steps, warmup, per_launch=None):
    """W untimed launches, then exactly K timed launches between two
    synchronisations.  Returns (wall seconds for the K launches, mean seconds per
    launch from HIP events on the launch stream).  With per_launch (a list), a
    second run of K launches records one event pair around each launch and
    appends the per-launch seconds (for median and min)."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if per_launch is not None:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            launch()
            b.record(stream)
        torch.cuda.synchronize()
        per_launch.extend(a.elapsed_time(b) / 1e3 for a, b in ev)
    return wall, e0.elapsed_time(e1) / 1e3 / steps   # seconds total, seconds per launch (events)


def _device_info():
    """CU count and peak clock read from the device (hipDeviceAttributeClockRate is
    5 in hip_runtime_api.h's enum)."""
    import ctypes
    import torch
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": props.gcnArchName, "compute_units": props.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:
            info["peak_clock_mhz"] = v.value / 1000.0
    except OSError:
        pass
    return info


def _gpu_attn(name, steps, warmup):
    import torch
    from differential_attention_02_amd import binding as B
    from differential_attention_02_amd import workloads
    cfg = workloads.CONFIGS[name]
    inp = workloads.make_attn_inputs(cfg)
    x = [inp[k].cuda() for k in ("q1", "k1", "q2", "k2", "v")]
    vecs = [t.cuda() for t in inp["lambda_vecs"]]
    out = torch.empty_like(x[4])
    args = B.fwd_args(*x, out, lambda_init=B.lambda_init(cfg.layer), lambda_vecs=vecs,
                      causal=cfg.causal, norm=True, eps=cfg.eps)
    each = []
    wall, per = _time_launches(lambda: B.fwd_launch(args), steps, warmup, each)
    flops = cfg.batch * cfg.heads * cfg.pairs * FLOP_PER_PAIR_FWD
    return {"cfg": cfg, "wall_s": wall, "event_s_per_launch": per, "flop_per_step": flops,
            "tflops": flops * steps / wall / 1e12, "event_tflops": flops / per / 1e12, "inputs": inp,
            "median_ms": statistics.median(each) * 1e3, "min_ms": min(each) * 1e3}


def _gpu_train(steps, warmup):
    import torch
    from differential_attention_02_amd import binding as B
    from differential_attention_02_amd import workloads
    cfg = workloads.CONFIGS["train_8k"]
    inp = workloads.make_attn_inputs(cfg)
    x = [inp[k].cuda() for k in ("q1", "k1", "q2", "k2", "v")]
    vecs = [t.cuda() for t in inp["lambda_vecs"]]
    dy = inp["dy"].cuda()
    li = B.lambda_init(cfg.layer)
    Bn, S, H, _ = x[0].shape
    dv = x[4].shape[-1]
    f32 = dict(dtype=torch.float32, device="cuda")
    saves = {"lse1": torch.empty((Bn, H, S), **f32), "lse2": torch.empty((Bn, H, S), **f32),
             "rstd": torch.empty((Bn, H, S), **f32), "o_pre": torch.empty((Bn, S, H, dv), **f32),
             "a2": torch.empty((Bn, S, H, dv), **f32)}
    out = torch.empty_like(x[4])
    fa = B.fwd_args(*x, out, lambda_init=li, lambda_vecs=vecs, causal=True, eps=cfg.eps, saves=saves)
    ba, _grads, _ws = B.bwd_args(*x, dy, saves, lambda_init=li, lambda_vecs=vecs, causal=True)

    def step():
        B.fwd_launch(fa)
        B.bwd_launch(ba)

    each = []
    wall, per = _time_launches(step, steps, warmup, each)
    pairs = cfg.batch * cfg.heads * cfg.pairs
    flops = pairs * (FLOP_PER_PAIR_FWD + FLOP_PER_PAIR_BWD)
    return {"tflops": flops * steps / wall / 1e12, "ms_per_step": wall / steps * 1e3,
            "event_tflops": flops / per / 1e12, "flop_per_step": flops, "inputs": inp,
            "median_ms": statistics.median(each) * 1e3, "min_ms": min(each) * 1e3}


def _gpu_decode(steps, warmup):
    import torch
    from differential_attention_02_amd import binding as B
    from differential_attention_02_amd import workloads
    cfg = workloads.CONFIGS["v2_decode"]
    inp = workloads.make_decode_inputs(cfg)
    q, k, v, lam = (inp[n].cuda() for n in ("q", "k_cache", "v_cache", "lam"))
    sample = {n: inp[n][:16].clone() for n in ("q", "k_cache", "v_cache")}
    sample["lam"] = inp["lam"]
    del inp
    out = torch.empty((cfg.batch, cfg.q_heads // 2, cfg.head_dim), dtype=q.dtype, device="cuda")
    args = B.decode_args(q, k, v, lam, out)
    nbytes = B.decode_workspace_size(args)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), nbytes
    each = []
    wall, per = _time_launches(lambda: B.decode_launch(args), steps, warmup, each)
    esz = 2
    moved = (2 * cfg.batch * cfg.kv_len * cfg.kv_heads * cfg.head_dim + cfg.batch * cfg.q_heads * cfg.head_dim
             + cfg.batch * cfg.q_heads // 2 * cfg.head_dim) * esz
    return {"cfg": cfg, "bytes_per_step": moved, "gbs": moved * steps / wall / 1e9,
            "event_gbs": moved / per / 1e9, "event_s_per_launch": per, "splits": args.num_splits,
            "sample": sample, "median_ms": statistics.median(each) * 1e3, "min_ms": min(each) * 1e3}


def _gpu_v2_prefill(steps, warmup):
    import torch
    from differential_attention_02_amd import binding as B
    from differential_attention_02_amd import workloads
    cfg = workloads.CONFIGS["v2_prefill_4k"]
    inp = workloads.make_v2_prefill_inputs(cfg)
    q, k, v, lam = (inp[n].cuda() for n in ("q", "k", "v", "lam"))
    out = torch.empty((cfg.batch, cfg.seqlen, cfg.q_heads // 2, cfg.head_dim), dtype=q.dtype, device="cuda")
    args = B.v2_fwd_args(q, k, v, lam, out, causal=cfg.causal)
    each = []
    wall, per = _time_launches(lambda: B.v2_fwd_launch(args), steps, warmup, each)
    flops = cfg.batch * (cfg.q_heads // 2) * cfg.pairs * FLOP_PER_PAIR_V2
    return {"cfg": cfg, "wall_s": wall, "event_s_per_launch": per, "flop_per_step": flops,
            "tflops": flops * steps / wall / 1e12, "event_tflops": flops / per / 1e12, "inputs": inp,
            "median_ms": statistics.median(each) * 1e3, "min_ms": min(each) * 1e3}


def _sparse_selection(cfg):
    """The block-sparse workload's seeded selection (seed 0): per (batch, pair,
    128-row query tile) 16 of the 64-key tiles: the first, the four ending at
    the tile's last row, and 11 drawn at random from the earlier ones."""
    from differential_attention_02_amd import workloads
    mask = workloads.make_block_selection(cfg.batch, cfg.q_heads // 2, cfg.seqlen, budget=16, sink=1, local=4, seed=0)
    return mask, workloads.block_pairs(mask, cfg.seqlen)


def _gpu_v2_sparse(steps, warmup):
    """The V2 4K forward over the seeded block selection; flop counted over
    the selected (query, key, pair) triples only."""
    import torch
    from differential_attention_02_amd import binding as B
    from differential_attention_02_amd import workloads
    cfg = workloads.CONFIGS["v2_prefill_4k"]
    inp = workloads.make_v2_prefill_inputs(cfg)
    mask, pairs = _sparse_selection(cfg)
    q, k, v, lam = (inp[n].cuda() for n in ("q", "k", "v", "lam"))
    idx, cnt = B.v2_block_lists(mask.cuda())
    out = torch.empty((cfg.batch, cfg.seqlen, cfg.q_heads // 2, cfg.head_dim), dtype=q.dtype, device="cuda")
    args = B.v2_fwd_args(q, k, v, lam, out, causal=cfg.causal)
    each = []
    wall, per = _time_launches(lambda: B.v2_fwd_sparse_launch(args, idx, cnt), steps, warmup, each)
    flops = pairs * FLOP_PER_PAIR_V2
    return {"wall_s": wall, "event_s_per_launch": per, "flop_per_step": flops, "density": pairs / (
            cfg.batch * (cfg.q_heads // 2) * cfg.pairs), "tflops": flops * steps / wall / 1e12,
            "event_tflops": flops / per / 1e12, "inputs": inp, "mask": mask,
            "median_ms": statistics.median(each) * 1e3, "min_ms": min(each) * 1e3}


def _gpu_fp8(steps, warmup):
    """The 4K forward with fp8 e4m3 attention logits (quantisation of Q1, K1,
    Q2, K2 included in every step)."""
    import torch
    from differential_attention_02_amd import binding as B
    from differential_attention_02_amd import workloads
    cfg = workloads.CONFIGS["prefill_4k"]
    inp = workloads.make_attn_inputs(cfg)
    x = [inp[k].cuda() for k in ("q1", "k1", "q2", "k2", "v")]
    vecs = [t.cuda() for t in inp["lambda_vecs"]]
    out = torch.empty_like(x[4])
    args = B.fwd_args(*x, out, lambda_init=B.lambda_init(cfg.layer), lambda_vecs=vecs, causal=cfg.causal,
                      norm=True, eps=cfg.eps)
    ws = B.fwd_fp8_workspace(args, x[0].device)
    each = []
    wall, per = _time_launches(lambda: B.fwd_fp8_launch(args, ws), steps, warmup, each)
    flops = cfg.batch * cfg.heads * cfg.pairs * FLOP_PER_PAIR_FWD
    return {"wall_s": wall, "event_s_per_launch": per, "flop_per_step": flops,
            "tflops": flops * steps / wall / 1e12, "event_tflops": flops / per / 1e12, "inputs": inp,
            "median_ms": statistics.median(each) * 1e3, "min_ms": min(each) * 1e3}


def _gpu_v2_train(steps, warmup):
    """One DIFF V2 training step at the 4K V2 workload: forward with the
    training saves, then the backward, on random upstream gradients."""
    import torch
    from differential_attention_02_amd import binding as B
    from differential_attention_02_amd import workloads
    cfg = workloads.CONFIGS["v2_prefill_4k"]
    inp = workloads.make_v2_prefill_inputs(cfg)
    q, k, v, lam = (inp[n].cuda() for n in ("q", "k", "v", "lam"))
    Bn, S, Hq, D = q.shape
    gen = torch.Generator().manual_seed(1)
    dout = torch.randn((Bn, S, Hq // 2, D), generator=gen).to(torch.bfloat16).cuda()
    f32 = dict(dtype=torch.float32, device="cuda")
    out = torch.empty((Bn, S, Hq // 2, D), dtype=q.dtype, device="cuda")
    saves = {"lse": torch.empty((Bn, Hq, S), **f32), "a_even": torch.empty((Bn, S, Hq // 2, D), **f32),
             "a_odd": torch.empty((Bn, S, Hq // 2, D), **f32)}
    fa = B.v2_fwd_args(q, k, v, lam, out, causal=cfg.causal, saves=saves)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dlam = torch.empty((Bn, S, Hq // 2), **f32)
    ba = B.v2_bwd_args(q, k, v, lam, dout, saves, dq, dk, dv, dlam, causal=cfg.causal)
    nbytes = B.v2_bwd_workspace_size(ba)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ba.workspace, ba.workspace_bytes = ws.data_ptr(), nbytes

    def step():
        B.v2_fwd_launch(fa)
        B.v2_bwd_launch(ba)

    each = []
    wall, per = _time_launches(step, steps, warmup, each)
    pairs = Bn * (Hq // 2) * cfg.pairs
    flops = pairs * (FLOP_PER_PAIR_V2 + FLOP_PER_PAIR_V2_BWD)
    return {"ms_per_step": wall / steps * 1e3, "tflops": flops * steps / wall / 1e12,
            "event_tflops": flops / per / 1e12, "flop_per_step": flops,
            "median_ms": statistics.median(each) * 1e3, "min_ms": min(each) * 1e3, "inputs": inp}


def _gpu_v1_decode(steps, warmup):
    import torch
    from differential_attention_02_amd import binding as B
    from differential_attention_02_amd import workloads
    cfg = workloads.CONFIGS["v1_decode"]
    inp = workloads.make_v1_decode_inputs(cfg)
    x = [inp[n].cuda() for n in ("q1", "q2", "k1_cache", "k2_cache", "v_cache")]
    vecs = [t.cuda() for t in inp["lambda_vecs"]]
    lam_rec = _seeded_lambda({"lambda_vecs": inp["lambda_vecs"], "cfg": cfg})
    del inp
    out = torch.empty((cfg.batch, cfg.heads, cfg.v_dim), dtype=x[0].dtype, device="cuda")
    args = B.v1_decode_args(*x, out, lambda_init=B.lambda_init(cfg.layer), lambda_vecs=vecs, eps=cfg.eps)
    nbytes = B.v1_decode_workspace_size(args)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), nbytes
    each = []
    wall, per = _time_launches(lambda: B.v1_decode_launch(args), steps, warmup, each)
    moved = (cfg.batch * cfg.kv_len * cfg.heads * (2 * cfg.head_dim + cfg.v_dim)
             + 2 * cfg.batch * cfg.heads * cfg.head_dim + cfg.batch * cfg.heads * cfg.v_dim) * 2
    return {"cfg": cfg, "bytes_per_step": moved, "gbs": moved * steps / wall / 1e9,
            "event_gbs": moved / per / 1e9, "event_s_per_launch": per, "splits": args.num_splits,
            "median_ms": statistics.median(each) * 1e3, "min_ms": min(each) * 1e3, "seeded_lambda": lam_rec}


def _seeded_lambda(inp):
    """The lambda that a V1 workload's seeded vectors give:
    exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init(layer), for the record."""
    import math
    from differential_attention_02_amd import binding as B
    lq1, lk1, lq2, lk2 = (t.double() for t in inp["lambda_vecs"])
    li = B.lambda_init(inp["cfg"].layer)
    return {"layer": inp["cfg"].layer, "lambda_init": li,
            "lambda": math.exp(float(lq1 @ lk1)) - math.exp(float(lq2 @ lk2)) + li}


def _host_info():
    """The host CPU's model name and the BLAS thread settings the oracle ran with."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    libs = []
    try:
        from threadpoolctl import threadpool_info
        libs = [{"library": p.get("internal_api"), "threads": p.get("num_threads")} for p in threadpool_info()
                if p.get("user_api") == "blas"]
    except Exception:
        pass
    env = {k: os.environ[k] for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
           if k in os.environ}
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "blas": libs, "thread_env": env}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


def _cpu_baseline_fwd(inp, budget_s=12.0):
    """The float64 oracle on whole heads of the 4K workload (all 4096 causal
    rows each, same inputs as the GPU run), one head at a time until about
    budget_s seconds have passed or all 48 heads are done."""
    import oracle
    cfg = inp["cfg"]
    li = oracle.lambda_init(cfg.layer)
    lam = oracle.lambda_value(*[t.double().numpy() for t in inp["lambda_vecs"]], li)
    done, dt = 0, 0.0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            x = [inp[k][b:b + 1, :, h:h + 1].double().numpy() for k in ("q1", "k1", "q2", "k2", "v")]
            t0 = time.perf_counter()
            oracle.diff_attn_fwd(*x, lam, li, causal=True, norm=True, eps=cfg.eps)
            dt += time.perf_counter() - t0
            done += 1
            if dt >= budget_s:
                break
        if dt >= budget_s:
            break
    flops = done * cfg.pairs * FLOP_PER_PAIR_FWD
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"prefill_4k: {done} of 48 (batch, head) slices, all 4096 causal rows each; "
                      f"{dt:.1f} s of oracle time"}


def _cpu_baseline_fp8(inp, budget_s=10.0):
    """The float64 oracle of the fp8-logit forward (per-row e4m3 quantisation
    of Q1, K1, Q2, K2, then the forward) on whole heads of the 4K workload,
    one head at a time until about budget_s seconds have passed."""
    import oracle
    cfg = inp["cfg"]
    li = oracle.lambda_init(cfg.layer)
    lam = oracle.lambda_value(*[t.double().numpy() for t in inp["lambda_vecs"]], li)
    done, dt = 0, 0.0
    for h in range(cfg.heads):
        x = [inp[k][0:1, :, h:h + 1].double().numpy() for k in ("q1", "k1", "q2", "k2", "v")]
        t0 = time.perf_counter()
        oracle.diff_attn_fwd_fp8_logits(*x, lam, li, causal=True, norm=True, eps=cfg.eps)
        dt += time.perf_counter() - t0
        done += 1
        if dt >= budget_s:
            break
    flops = done * cfg.pairs * FLOP_PER_PAIR_FWD
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"prefill_4k_fp8: {done} of 48 (batch, head) slices (batch 0), all 4096 causal rows, "
                      f"quantisation included; {dt:.1f} s of oracle time"}


def _cpu_baseline_64k(inp, heads=2):
    """The float64 oracle on a stratified sample of the 64K workload: 1024
    query rows (512 evenly spaced and the last 512) of each of the first
    `heads` heads, each row against all of its causal keys.  Reports the rate
    on the sample and the full forward's oracle time extrapolated from it."""
    import numpy as np
    import oracle
    cfg = inp["cfg"]
    S = cfg.seqlen
    rows = np.unique(np.concatenate([np.linspace(0, S - 513, 512).astype(np.int64), np.arange(S - 512, S)]))
    li = oracle.lambda_init(cfg.layer)
    lam = oracle.lambda_value(*[t.double().numpy() for t in inp["lambda_vecs"]], li)
    dt = 0.0
    for h in range(heads):
        x = [inp[k][:, :, h:h + 1].double().numpy() for k in ("q1", "k1", "q2", "k2", "v")]
        t0 = time.perf_counter()
        oracle.diff_attn_fwd(*x, lam, li, causal=True, norm=True, eps=cfg.eps, rows=rows)
        dt += time.perf_counter() - t0
    flops = heads * int((rows + 1).sum()) * FLOP_PER_PAIR_FWD
    full = cfg.batch * cfg.heads * cfg.pairs * FLOP_PER_PAIR_FWD
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"prefill_64k: {len(rows)} query rows (512 evenly spaced + the last 512) of {heads} of "
                      f"{cfg.batch * cfg.heads} heads, all causal keys; {dt:.1f} s of oracle time",
            "extrapolated_full_forward_s": full / (flops / dt)}


def _cpu_baseline_train(inp):
    """The float64 oracle's forward and backward on one (batch, head) slice of
    the 8K training workload (all 8192 causal rows), same inputs as the GPU."""
    import oracle
    cfg = inp["cfg"]
    li = oracle.lambda_init(cfg.layer)
    vecs = [t.double().numpy() for t in inp["lambda_vecs"]]
    lam = oracle.lambda_value(*vecs, li)
    x = [inp[k][0:1, :, 0:1].double().numpy() for k in ("q1", "k1", "q2", "k2", "v")]
    dy = inp["dy"][0:1, :, 0:1].double().numpy()
    t0 = time.perf_counter()
    oracle.diff_attn_fwd(*x, lam, li, causal=True, norm=True, eps=cfg.eps)
    oracle.diff_attn_bwd(*x, dy, lam_init=li, lam_vectors=vecs, causal=True, norm=True, eps=cfg.eps)
    dt = time.perf_counter() - t0
    flops = cfg.pairs * (FLOP_PER_PAIR_FWD + FLOP_PER_PAIR_BWD)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"train_8k: 1 of {cfg.batch * cfg.heads} (batch, head) slices, all {cfg.seqlen} causal "
                      f"rows, forward and backward; {dt:.1f} s of oracle time"}


def _cpu_baseline_v2_prefill(inp, with_bwd=False):
    """The float64 oracle on one (batch, pair) slice of the V2 4K workload
    (all 4096 causal rows of both heads), forward, or forward and backward."""
    import oracle
    cfg = inp["cfg"]
    sl = [inp["q"][0:1, :, 0:2], inp["k"][0:1, :, 0:1], inp["v"][0:1, :, 0:1], inp["lam"][0:1, :, 0:1]]
    x = [t.double().numpy() for t in sl]
    t0 = time.perf_counter()
    oracle.v2_prefill_fwd(*x, causal=True)
    if with_bwd:
        gen = __import__("torch").Generator().manual_seed(2)
        dy = __import__("torch").randn((1, cfg.seqlen, 1, cfg.head_dim), generator=gen).double().numpy()
        oracle.v2_prefill_bwd(*x, dy, causal=True)
    dt = time.perf_counter() - t0
    flops = cfg.pairs * (FLOP_PER_PAIR_V2 + (FLOP_PER_PAIR_V2_BWD if with_bwd else 0))
    what = "forward and backward" if with_bwd else "forward"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"v2_prefill_4k: 1 of {cfg.batch * cfg.q_heads // 2} (batch, pair) slices, all "
                      f"{cfg.seqlen} causal rows, {what}; {dt:.1f} s of oracle time"}


def _cpu_baseline_v2_sparse(inp, mask):
    """The float64 oracle's block-sparse forward on one (batch, pair) slice of
    the block-sparse workload (all 4096 rows of both heads)."""
    import oracle
    from differential_attention_02_amd import workloads
    cfg = inp["cfg"]
    sl = [inp["q"][0:1, :, 0:2], inp["k"][0:1, :, 0:1], inp["v"][0:1, :, 0:1], inp["lam"][0:1, :, 0:1]]
    x = [t.double().numpy() for t in sl]
    m = mask[0:1, 0:1]
    t0 = time.perf_counter()
    oracle.v2_prefill_fwd_block_sparse(*x, m.numpy(), causal=True)
    dt = time.perf_counter() - t0
    flops = workloads.block_pairs(m, cfg.seqlen) * FLOP_PER_PAIR_V2
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"v2_sparse_4k: 1 of {cfg.batch * cfg.q_heads // 2} (batch, pair) slices, all "
                      f"{cfg.seqlen} rows, selected pairs only; {dt:.1f} s of oracle time"}


def _cpu_baseline_v1_decode(budget_s=8.0):
    """The float64 oracle on whole sequences of the V1 decode workload, one
    sequence at a time (float64 up-conversion included) until about budget_s
    seconds have passed."""
    import oracle
    from differential_attention_02_amd import workloads
    cfg = workloads.CONFIGS["v1_decode"]
    inp = workloads.make_v1_decode_inputs(cfg, batch=8)
    li = oracle.lambda_init(cfg.layer)
    lam = oracle.lambda_value(*[t.double().numpy() for t in inp["lambda_vecs"]], li)
    names = ("q1", "q2", "k1_cache", "k2_cache", "v_cache")
    done, dt = 0, 0.0
    for b in range(8):
        t0 = time.perf_counter()
        x = [inp[n][b:b + 1].double().numpy() for n in names]
        oracle.v1_decode(*x, lam, li, eps=cfg.eps)
        dt += time.perf_counter() - t0
        done += 1
        if dt >= budget_s:
            break
    moved = done * (cfg.kv_len * cfg.heads * (2 * cfg.head_dim + cfg.v_dim) + 2 * cfg.heads * cfg.head_dim
                    + cfg.heads * cfg.v_dim) * 2
    return {"value": moved / dt / 1e9, "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"v1_decode sequences 0-{done - 1} of {cfg.batch} (same recipe, seed 0, batch drawn 8), "
                      f"bf16 byte count, including float64 up-conversion; {dt:.2f} s wall"}


def _cpu_baseline_decode(sample, cfg):
    """The float64 oracle on the first 16 of the 64 sequences of the decode
    workload (same inputs as the GPU run)."""
    import oracle
    nb = sample["q"].shape[0]
    t0 = time.perf_counter()
    for b in range(0, nb, 4):   # 4 sequences at a time bounds the float64 copies
        a = [sample[k][b:b + 4].double().numpy() for k in ("q", "k_cache", "v_cache")]
        oracle.v2_decode(*a, sample["lam"].double().numpy())
    dt = time.perf_counter() - t0
    moved = (2 * nb * cfg.kv_len * cfg.kv_heads * cfg.head_dim + nb * cfg.q_heads * cfg.head_dim * 1.5) * 2
    return {"value": moved / dt / 1e9, "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"v2_decode sequences 0-{nb - 1} of 64, bf16 byte count, including float64 "
                      f"up-conversion; {dt:.2f} s wall"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 200 untimed launches by default: after 20 (8 ms of work at 4K) the clock had not settled and the
    # 4K forward read ~5 % below its steady rate.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--only", choices=["prefill_4k", "prefill_64k", "train_8k", "v2_decode", "v2_prefill_4k",
                                       "v2_train_4k", "v1_decode", "prefill_4k_fp8", "v2_sparse_4k"],
                    default=None,
                    help="time one workload only (for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first copy a device buffer of this many MiB (reference kernel for HBM byte counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        return 2
    from differential_attention_02_amd import binding
    binding.lib()   # fails loudly if the HIP library is missing
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)   # reads and writes calib_copy_mib MiB each
        torch.cuda.synchronize()
        del src, dst

    if args.only is not None:
        if args.only in ("prefill_4k", "prefill_64k"):
            r = _gpu_attn(args.only, args.steps, args.warmup)
            print(json.dumps({"workload": args.only, "tflops": r["tflops"], "event_tflops": r["event_tflops"]}))
        elif args.only == "train_8k":
            r = _gpu_train(args.steps, args.warmup)
            r.pop("inputs", None)
            print(json.dumps({"workload": "train_8k", **r}))
        elif args.only == "prefill_4k_fp8":
            r = _gpu_fp8(args.steps, args.warmup)
            r.pop("inputs", None)
            print(json.dumps({"workload": "prefill_4k_fp8", **r}))
        elif args.only == "v1_decode":
            r = _gpu_v1_decode(args.steps, args.warmup)
            print(json.dumps({"workload": "v1_decode", "gbs": r["gbs"], "event_gbs": r["event_gbs"],
                              "median_ms": r["median_ms"], "min_ms": r["min_ms"]}))
        elif args.only == "v2_train_4k":
            r = _gpu_v2_train(args.steps, args.warmup)
            r.pop("inputs", None)
            print(json.dumps({"workload": "v2_train_4k", **r}))
        elif args.only == "v2_sparse_4k":
            r = _gpu_v2_sparse(args.steps, args.warmup)
            print(json.dumps({"workload": "v2_sparse_4k", "tflops": r["tflops"], "event_tflops": r["event_tflops"],
                              "density": r["density"], "median_ms": r["median_ms"], "min_ms": r["min_ms"]}))
        elif args.only == "v2_prefill_4k":
            r = _gpu_v2_prefill(args.steps, args.warmup)
            print(json.dumps({"workload": "v2_prefill_4k", "tflops": r["tflops"], "event_tflops": r["event_tflops"],
                              "median_ms": r["median_ms"], "min_ms": r["min_ms"]}))
        else:
            r = _gpu_decode(args.steps, args.warmup)
            print(json.dumps({"workload": "v2_decode", "gbs": r["gbs"], "event_gbs": r["event_gbs"]}))
        return 0

    main_r = _gpu_attn("prefill_4k", args.steps, args.warmup)
    cfg = main_r["cfg"]
    achieved = main_r["flop_per_step"] / main_r["event_s_per_launch"] / 1e12
    traffic = _traffic_from_profile("fwd_onepass_prefill_4k_pmc.md", FWD_SOURCES)
    extra = {}
    # The long legs get a few warmup launches too: after one, the clock had not settled.
    n64 = max(5, args.steps // 5)
    r64 = _gpu_attn("prefill_64k", n64, 3)
    extra["prefill_64k"] = {"metric": "fwd TFLOP/s", "value": r64["tflops"], "unit": "TFLOP/s",
                            "config": {"workload": "prefill_64k: batch 1, seq 65536 causal, 16 heads, d 64, dv 128, "
                                                   "bf16, lambda_init at layer 24", "seeded_lambda": _seeded_lambda(r64["inputs"])},
                            "frac_of_bf16_peak": r64["event_tflops"] / PEAK_BF16_TFLOPS,
                            "ms_per_step": r64["wall_s"] / n64 * 1e3,
                            "roofline": {"bound": "mfma", "achieved": r64["event_tflops"], "peak": PEAK_BF16_TFLOPS,
                                         "unit": "TFLOP/s", "frac": r64["event_tflops"] / PEAK_BF16_TFLOPS,
                                         "traffic": _traffic_from_profile("fwd_onepass_prefill_64k_pmc.md",
                                                                          FWD_SOURCES)}}
    tr = _gpu_train(max(10, args.steps // 2), 5)
    extra["train_8k"] = {"metric": "fwd+bwd TFLOP/s", "value": tr["tflops"], "unit": "TFLOP/s",
                         "config": {"workload": "train_8k: forward with training saves then backward",
                                    "seeded_lambda": _seeded_lambda(tr["inputs"])},
                         "ms_per_step": tr["ms_per_step"], "frac_of_bf16_peak": tr["tflops"] / PEAK_BF16_TFLOPS,
                         "roofline": {"bound": "mfma", "achieved": tr["event_tflops"], "peak": PEAK_BF16_TFLOPS,
                                      "unit": "TFLOP/s", "frac": tr["event_tflops"] / PEAK_BF16_TFLOPS,
                                      "traffic": _traffic_from_profile("train_step_train_8k_pmc.md", BWD_SOURCES),
                                      "note": "traffic is the dK/dV kernel's (the step's longest), per launch"},
                         "median_ms": tr["median_ms"], "min_ms": tr["min_ms"]}
    dec = _gpu_decode(args.steps, args.warmup)
    dec_traffic = _traffic_from_profile("decode_split_v2_decode_pmc.md", DEC_SOURCES)
    extra["v2_decode"] = {
        "metric": "V2 decode HBM GB/s", "value": dec["gbs"], "unit": "GB/s",
        "ms_per_step": dec["event_s_per_launch"] * 1e3,
        "config": {"workload": "v2_decode: B64, 32 query heads over 16 KV heads, D 128, KV 8192, bf16",
                   "num_splits": "auto"},
        "roofline": {"bound": "hbm", "achieved": dec["event_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": dec["event_gbs"] / PEAK_HBM_GBS, "traffic": dec_traffic},
    }
    v2p = _gpu_v2_prefill(args.steps, args.warmup)
    extra["v2_prefill_4k"] = {
        "metric": "V2 prefill fwd TFLOP/s", "value": v2p["tflops"], "unit": "TFLOP/s",
        "ms_per_step": v2p["wall_s"] / args.steps * 1e3,
        "config": {"workload": "v2_prefill_4k: batch 4, seq 4096 causal, 24 query heads over 12 KV heads, "
                               "D 128, bf16, sigmoid input per token and pair"},
        "roofline": {"bound": "mfma", "achieved": v2p["event_tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": v2p["event_tflops"] / PEAK_BF16_TFLOPS,
                     "traffic": _traffic_from_profile("fwd_v2_v2_prefill_4k_pmc.md", V2P_SOURCES)},
        "median_ms": v2p["median_ms"], "min_ms": v2p["min_ms"],
    }
    v2s = _gpu_v2_sparse(args.steps, args.warmup)
    extra["v2_sparse_4k"] = {
        "metric": "block-sparse V2 prefill fwd TFLOP/s", "value": v2s["tflops"], "unit": "TFLOP/s",
        "ms_per_step": v2s["wall_s"] / args.steps * 1e3,
        "config": {"workload": "v2_sparse_4k: the v2_prefill_4k workload with one key-block selection per "
                               "(batch, head pair, 128-row query tile): 16 of the 64-key tiles (the first, the "
                               "four ending at the tile's last row, 11 random earlier ones; seed 0)",
                   "density": v2s["density"]},
        "roofline": {"bound": "mfma", "achieved": v2s["event_tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": v2s["event_tflops"] / PEAK_BF16_TFLOPS,
                     "traffic": _traffic_from_profile("fwd_v2_sparse_v2_sparse_4k_pmc.md", V2P_SOURCES),
                     "note": "1024 flop per selected (query, key, pair) triple"},
        "median_ms": v2s["median_ms"], "min_ms": v2s["min_ms"],
    }
    f8 = _gpu_fp8(args.steps, args.warmup)
    extra["prefill_4k_fp8"] = {
        "metric": "fwd TFLOP/s with fp8 e4m3 logits", "value": f8["tflops"], "unit": "TFLOP/s",
        "ms_per_step": f8["wall_s"] / args.steps * 1e3,
        "config": {"workload": "prefill_4k with Q1, K1, Q2, K2 quantised per row to fp8 e4m3 (power-of-two absmax "
                               "scale) inside every step; score products on scaled fp8 matrix instructions",
                   "seeded_lambda": _seeded_lambda(f8["inputs"])},
        "roofline": {"bound": "mfma", "achieved": f8["event_tflops"], "peak": PEAK_FP8_MIXED_TFLOPS,
                     "unit": "TFLOP/s", "frac": f8["event_tflops"] / PEAK_FP8_MIXED_TFLOPS,
                     "traffic": _traffic_from_profile("fwd_fp8_prefill_4k_pmc.md", FP8_SOURCES),
                     "note": "algorithmic 768 flop per pair against the mixed peak 768 / (256 / 5000 + 512 / 2500) "
                             "= 3000 TFLOP/s: the score products (256 flop) run on fp8 at 5.0 PFLOP/s, the PV "
                             "products (512 flop) stay fp16 at 2.5 PFLOP/s; traffic is the forward kernel's, per "
                             "launch (the quantisation kernel not counted)"},
        "median_ms": f8["median_ms"], "min_ms": f8["min_ms"],
    }
    v1d = _gpu_v1_decode(args.steps, args.warmup)
    extra["v1_decode"] = {
        "metric": "V1 decode HBM GB/s", "value": v1d["gbs"], "unit": "GB/s",
        "ms_per_step": v1d["event_s_per_launch"] * 1e3,
        "config": {"workload": "v1_decode: B64, 16 heads, K1/K2 width 64, V width 128, KV 8192, bf16, "
                               "lambda from 64-dim vectors, per-head RMSNorm", "num_splits": "auto",
                   "seeded_lambda": v1d["seeded_lambda"]},
        "roofline": {"bound": "hbm", "achieved": v1d["event_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": v1d["event_gbs"] / PEAK_HBM_GBS,
                     "traffic": _traffic_from_profile("v1dec_split_v1_decode_pmc.md", DEC_SOURCES)},
        "median_ms": v1d["median_ms"], "min_ms": v1d["min_ms"],
    }
    v2t = _gpu_v2_train(max(10, args.steps // 2), 5)
    extra["v2_train_4k"] = {"metric": "V2 fwd+bwd TFLOP/s", "value": v2t["tflops"], "unit": "TFLOP/s",
                            "ms_per_step": v2t["ms_per_step"], "frac_of_bf16_peak": v2t["tflops"] / PEAK_BF16_TFLOPS,
                            "config": {"workload": "v2_train_4k: the v2_prefill_4k workload, forward with training "
                                                   "saves then backward"},
                            "roofline": {"bound": "mfma", "achieved": v2t["event_tflops"], "peak": PEAK_BF16_TFLOPS,
                                         "unit": "TFLOP/s", "frac": v2t["event_tflops"] / PEAK_BF16_TFLOPS,
                                         "traffic": _traffic_from_profile("v2_train_step_v2_train_4k_pmc.md", V2B_SOURCES),
                                         "note": "traffic is the dK/dV kernel's (the step's longest), per launch"},
                            "median_ms": v2t["median_ms"], "min_ms": v2t["min_ms"]}
    cpu = None
    extra["v2_decode"]["median_ms"], extra["v2_decode"]["min_ms"] = dec["median_ms"], dec["min_ms"]
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline_fwd(main_r["inputs"])
        extra["v2_decode"]["cpu_baseline"] = _cpu_baseline_decode(dec["sample"], dec["cfg"])
        extra["train_8k"]["cpu_baseline"] = _cpu_baseline_train(tr["inputs"])
        extra["v2_prefill_4k"]["cpu_baseline"] = _cpu_baseline_v2_prefill(v2p["inputs"])
        extra["v2_train_4k"]["cpu_baseline"] = _cpu_baseline_v2_prefill(v2t["inputs"], with_bwd=True)
        extra["v1_decode"]["cpu_baseline"] = _cpu_baseline_v1_decode()
        extra["v2_sparse_4k"]["cpu_baseline"] = _cpu_baseline_v2_sparse(v2s["inputs"], v2s["mask"])
        extra["prefill_64k"]["cpu_baseline"] = _cpu_baseline_64k(r64["inputs"])
        extra["prefill_4k_fp8"]["cpu_baseline"] = _cpu_baseline_fp8(f8["inputs"])
        cpu["host"] = _host_info()
    line = {
        "metric": METRIC,
        "value": main_r["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["wall_s"] / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_4k: batch 4, seq 4096 causal, 12 heads, d 64, dv 128, bf16, "
                               "lambda from 64-dim vectors, lambda_init at layer 12, per-head RMSNorm",
                   "global_batch": cfg.batch, "seq_len": cfg.seqlen, "parallelism": "single GPU",
                   "seeded_lambda": _seeded_lambda(main_r["inputs"])},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "note": "768 flop per unmasked (query, key, head) over the launch's event time, which covers "
                             "both of its kernels: the fp16 V copy pass and the one-pass forward"},
        "cpu_baseline": cpu,
        "timing": {"median_ms": main_r["median_ms"], "min_ms": main_r["min_ms"],
                   "note": "per-launch HIP events, a second run of the same K launches"},
        "device": _device_info(),
        "extra": extra,
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
