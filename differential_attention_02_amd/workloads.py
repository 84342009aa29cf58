"""Seeded synthetic inputs for every workload (no arithmetic of the method).

Both the HIP path and the float64 oracle receive tensors made here; this module
computes no attention, lambda or normalisation.  All draws come from a CPU
torch.Generator seeded per call, in a fixed order:
q1, k1, q2, k2, v, then the four lambda vectors (lq1, lk1, lq2, lk2), then the
upstream gradient dy; for the V2 decode: q, k_cache, v_cache, lam; for the V2
prefill: q, k, v, lam (then dy when a gradient is asked for); for the V1
decode: q1, q2, k1_cache, k2_cache, v_cache, then the four lambda vectors.
Each tensor is drawn in float32 one batch entry at a time, multiplied by its
scale, and (for bf16 workloads) rounded once to bfloat16 (round to nearest
even).  The oracle upcasts those same rounded values exactly.
"""
from __future__ import annotations

import dataclasses
import math

import torch

__all__ = ["AttnConfig", "DecodeConfig", "V1DecodeConfig", "V2PrefillConfig", "CONFIGS", "make_attn_inputs",
           "make_decode_inputs", "make_v1_decode_inputs", "make_v2_prefill_inputs", "worked_example_inputs"]


@dataclasses.dataclass(frozen=True)
class AttnConfig:
    """A DIFF V1 attention workload ([batch, seq, head, channel] layout)."""
    name: str
    batch: int
    seqlen: int
    heads: int
    head_dim: int
    v_dim: int
    dtype: torch.dtype
    causal: bool
    layer: int                 # layer index l >= 1 for lambda_init
    input_scale: float         # q/k/v ~ N(0, 1) * input_scale
    lambda_vec_dim: int = 0    # 0: lambda fixed at lambda_fixed
    lambda_vec_std: float = 0.1
    lambda_fixed: float = 0.8
    with_dy: bool = False      # draw an upstream gradient dy ~ N(0, 1)
    eps: float = 1e-5

    @property
    def pairs(self) -> int:
        """(query, key) pairs per (batch, head) that the mask leaves in."""
        s = self.seqlen
        return s * (s + 1) // 2 if self.causal else s * s


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """A DIFF V2 decode workload: one query token per sequence."""
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    kv_len: int
    dtype: torch.dtype
    input_scale: float
    lam_shape: str = "per_head"   # "per_head" ([Hq/2]) or "per_batch_head"


@dataclasses.dataclass(frozen=True)
class V1DecodeConfig:
    """A DIFF V1 decode workload: one new token per sequence over a cache of
    K1, K2 (width d) and V (width dv)."""
    name: str
    batch: int
    heads: int
    head_dim: int
    v_dim: int
    kv_len: int
    dtype: torch.dtype
    input_scale: float
    layer: int
    lambda_vec_dim: int = 64
    lambda_vec_std: float = 0.1
    eps: float = 1e-5


@dataclasses.dataclass(frozen=True)
class V2PrefillConfig:
    """A DIFF V2 prefill workload: whole sequences, Hq query heads over Hkv KV
    heads, a sigmoid input per (batch, token, pair)."""
    name: str
    batch: int
    seqlen: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: torch.dtype
    causal: bool
    input_scale: float          # q/k/v ~ N(0, 1) * input_scale
    lam_std: float = 1.0        # lam ~ N(0, lam_std^2), float32 [B, S, Hq/2]
    with_dy: bool = False

    @property
    def pairs(self) -> int:
        s = self.seqlen
        return s * (s + 1) // 2 if self.causal else s * s


CONFIGS = {
    # Tiny single-head check in float32 (lambda fixed at 0.8, layer 1).
    "tiny_f32": AttnConfig("tiny_f32", 1, 64, 1, 8, 16, torch.float32, True, 1, 1.0),
    # 3B-class layer forward: 12 heads, d 64, value width 128, 4K causal.
    "prefill_4k": AttnConfig("prefill_4k", 4, 4096, 12, 64, 128, torch.bfloat16, True, 12,
                             1.0 / math.sqrt(64), lambda_vec_dim=64),
    # Long-context forward: 64K causal, 16 heads.
    "prefill_64k": AttnConfig("prefill_64k", 1, 65536, 16, 64, 128, torch.bfloat16, True, 24,
                              1.0 / 8.0, lambda_vec_dim=64),
    # Training step (forward + backward) at 8K, 16 heads.
    "train_8k": AttnConfig("train_8k", 2, 8192, 16, 64, 128, torch.bfloat16, True, 12,
                           1.0 / 8.0, lambda_vec_dim=64, with_dy=True),
    # DIFF V2 decode: 32 query heads over 16 KV heads, cache length 8192.
    "v2_decode": DecodeConfig("v2_decode", 64, 32, 16, 128, 8192, torch.bfloat16,
                              1.0 / math.sqrt(128)),
    # DIFF V1 decode over a K1/K2/V cache with the V2 decode's cache bytes:
    # 16 heads of K1, K2 (64 wide) and V (128 wide), cache length 8192.
    "v1_decode": V1DecodeConfig("v1_decode", 64, 16, 64, 128, 8192, torch.bfloat16, 1.0 / 8.0, 12),
    # DIFF V2 prefill at 4K: 24 query heads over 12 KV heads (one even/odd pair
    # per KV head), head width 128, causal.
    "v2_prefill_4k": V2PrefillConfig("v2_prefill_4k", 4, 4096, 24, 12, 128, torch.bfloat16, True,
                                     1.0 / math.sqrt(128)),
}


def _draw(gen: torch.Generator, shape, scale: float, dtype: torch.dtype) -> torch.Tensor:
    """N(0, 1) * scale, drawn in float32 per leading index, cast once to dtype."""
    out = torch.empty(shape, dtype=dtype)
    for i in range(shape[0]):
        x = torch.randn(shape[1:], generator=gen, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        out[i] = x.to(dtype)
    return out


def make_attn_inputs(cfg: AttnConfig | str, seed: int = 0, *, seqlen: int | None = None,
                     batch: int | None = None, heads: int | None = None) -> dict:
    """Inputs of a DIFF V1 workload on the CPU.

    Optional overrides shrink a workload (same recipe, fewer rows) for tests.
    Returns q1, k1, q2, k2 [B,S,H,d]; v [B,S,H,dv]; lambda_vecs (four float32
    vectors) or None; dy [B,S,H,dv] or None; and the config itself.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    B = cfg.batch if batch is None else batch
    S = cfg.seqlen if seqlen is None else seqlen
    H = cfg.heads if heads is None else heads
    gen = torch.Generator().manual_seed(seed)
    t = {}
    for name in ("q1", "k1", "q2", "k2"):
        t[name] = _draw(gen, (B, S, H, cfg.head_dim), cfg.input_scale, cfg.dtype)
    t["v"] = _draw(gen, (B, S, H, cfg.v_dim), cfg.input_scale, cfg.dtype)
    if cfg.lambda_vec_dim:
        t["lambda_vecs"] = tuple(
            torch.randn(cfg.lambda_vec_dim, generator=gen, dtype=torch.float32) * cfg.lambda_vec_std
            for _ in range(4))
    else:
        t["lambda_vecs"] = None
    t["dy"] = _draw(gen, (B, S, H, cfg.v_dim), 1.0, cfg.dtype) if cfg.with_dy else None
    t["cfg"] = cfg
    return t


def make_decode_inputs(cfg: DecodeConfig | str = "v2_decode", seed: int = 0, *,
                       batch: int | None = None, kv_len: int | None = None) -> dict:
    """Inputs of a DIFF V2 decode workload on the CPU: q [B,Hq,D],
    k_cache/v_cache [B,S_kv,Hkv,D], lam float32 [Hq/2] (or [B,Hq/2])."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    B = cfg.batch if batch is None else batch
    L = cfg.kv_len if kv_len is None else kv_len
    gen = torch.Generator().manual_seed(seed)
    t = {
        "q": _draw(gen, (B, cfg.q_heads, cfg.head_dim), cfg.input_scale, cfg.dtype),
        "k_cache": _draw(gen, (B, L, cfg.kv_heads, cfg.head_dim), cfg.input_scale, cfg.dtype),
        "v_cache": _draw(gen, (B, L, cfg.kv_heads, cfg.head_dim), cfg.input_scale, cfg.dtype),
    }
    lam_shape = (cfg.q_heads // 2,) if cfg.lam_shape == "per_head" else (B, cfg.q_heads // 2)
    t["lam"] = torch.randn(lam_shape, generator=gen, dtype=torch.float32)
    t["cfg"] = cfg
    return t


def make_v1_decode_inputs(cfg: V1DecodeConfig | str = "v1_decode", seed: int = 0, *,
                          batch: int | None = None, kv_len: int | None = None, heads: int | None = None) -> dict:
    """Inputs of a DIFF V1 decode workload on the CPU: q1, q2 [B,H,d],
    k1_cache, k2_cache [B,S_kv,H,d], v_cache [B,S_kv,H,dv], lambda_vecs."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    B = cfg.batch if batch is None else batch
    L = cfg.kv_len if kv_len is None else kv_len
    H = cfg.heads if heads is None else heads
    gen = torch.Generator().manual_seed(seed)
    t = {
        "q1": _draw(gen, (B, H, cfg.head_dim), cfg.input_scale, cfg.dtype),
        "q2": _draw(gen, (B, H, cfg.head_dim), cfg.input_scale, cfg.dtype),
        "k1_cache": _draw(gen, (B, L, H, cfg.head_dim), cfg.input_scale, cfg.dtype),
        "k2_cache": _draw(gen, (B, L, H, cfg.head_dim), cfg.input_scale, cfg.dtype),
        "v_cache": _draw(gen, (B, L, H, cfg.v_dim), cfg.input_scale, cfg.dtype),
    }
    t["lambda_vecs"] = tuple(torch.randn(cfg.lambda_vec_dim, generator=gen, dtype=torch.float32) * cfg.lambda_vec_std
                             for _ in range(4))
    t["cfg"] = cfg
    return t


def make_v2_prefill_inputs(cfg: V2PrefillConfig | str = "v2_prefill_4k", seed: int = 0, *,
                           batch: int | None = None, seqlen: int | None = None, q_heads: int | None = None,
                           kv_heads: int | None = None, input_scale: float | None = None) -> dict:
    """Inputs of a DIFF V2 prefill workload on the CPU: q [B,S,Hq,D], k, v
    [B,S,Hkv,D], lam float32 [B,S,Hq/2], dy [B,S,Hq/2,D] or None."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    B = cfg.batch if batch is None else batch
    S = cfg.seqlen if seqlen is None else seqlen
    Hq = cfg.q_heads if q_heads is None else q_heads
    Hkv = cfg.kv_heads if kv_heads is None else kv_heads
    sc = cfg.input_scale if input_scale is None else input_scale
    gen = torch.Generator().manual_seed(seed)
    t = {
        "q": _draw(gen, (B, S, Hq, cfg.head_dim), sc, cfg.dtype),
        "k": _draw(gen, (B, S, Hkv, cfg.head_dim), sc, cfg.dtype),
        "v": _draw(gen, (B, S, Hkv, cfg.head_dim), sc, cfg.dtype),
    }
    t["lam"] = torch.randn((B, S, Hq // 2), generator=gen, dtype=torch.float32) * cfg.lam_std
    t["dy"] = _draw(gen, (B, S, Hq // 2, cfg.head_dim), 1.0, cfg.dtype) if cfg.with_dy else None
    t["cfg"] = cfg
    return t


def make_block_selection(batch: int, pairs: int, seqlen: int, *, budget: int = 16, sink: int = 1, local: int = 4,
                         seed: int = 0, causal: bool = True, q_block: int = 128, k_block: int = 64) -> torch.Tensor:
    """A seeded key-block selection per (batch, head pair, query block): bool
    [B, P, ceil(S / q_block), ceil(S / k_block)].  Each query block keeps the
    first `sink` key blocks, the `local` key blocks that end at its own last
    row, and random other key blocks (uniform, without repeats) up to `budget`
    blocks; with causal set only key blocks that start at or before the query
    block's last row are eligible, so early query blocks keep all of theirs."""
    nqb = (seqlen + q_block - 1) // q_block
    nkb = (seqlen + k_block - 1) // k_block
    gen = torch.Generator().manual_seed(seed)
    score = torch.rand((batch, pairs, nqb, nkb), generator=gen)
    kb = torch.arange(nkb)[None, :]
    hi = torch.clamp((torch.arange(nqb)[:, None] + 1) * q_block, max=seqlen)   # one past the block's last row
    end = (hi + k_block - 1) // k_block                                        # key blocks up to that row
    forced = (kb < sink) | ((kb >= end - local) & (kb < end))
    eligible = kb < end if causal else torch.ones((nqb, nkb), dtype=torch.bool)
    score = torch.where(forced, torch.full_like(score, 2.0), score)
    score = torch.where(eligible, score, torch.full_like(score, -1.0))
    top = torch.topk(score, min(budget, nkb), dim=-1)
    mask = torch.zeros_like(score, dtype=torch.bool)
    mask.scatter_(-1, top.indices, top.values >= 0)
    return mask


def block_pairs(mask: torch.Tensor, seqlen: int, *, causal: bool = True, q_block: int = 128,
                k_block: int = 64) -> int:
    """Number of (query, key, pair) triples a block selection lets through."""
    nqb, nkb = mask.shape[-2:]
    rows = torch.arange(seqlen)
    keys = torch.arange(seqlen)
    per = torch.zeros((nqb, nkb), dtype=torch.int64)     # allowed pairs inside each (query block, key block)
    for t in range(nqb):
        r = rows[t * q_block:(t + 1) * q_block]
        for i in range(nkb):
            k = keys[i * k_block:(i + 1) * k_block]
            per[t, i] = int(((k[None, :] <= r[:, None]) if causal else torch.ones(len(r), len(k))).sum())
    return int((mask.to(torch.int64) * per).sum())


def seeded_normals(seed: int, shapes):
    """Standard-normal float32 tensors of the given shapes, drawn in order from
    one CPU generator seeded with `seed`."""
    gen = torch.Generator().manual_seed(seed)
    return [torch.randn(*shape, generator=gen) for shape in shapes]


def worked_example_inputs(n: int = 6, d: int = 8, seed: int = 0):
    """Inputs of the glossary page's worked example (Ultralytics glossary,
    "Differential Transformer", section "How differential attention works"),
    whose printed result (a row sum of 0.20, 13 of 36 negative weights) pins
    the oracle: one seeded generator, a [4, n, d] normal draw split into
    q1, k1, q2, k2, then an [n, 2d] draw for v."""
    qk, v = seeded_normals(seed, [(4, n, d), (n, 2 * d)])
    q1, k1, q2, k2 = qk
    return q1, k1, q2, k2, v
