"""float64 numpy oracle for multi-head differential attention (DIFF V1) and the
DIFF V2 decode and prefill combines.

Test infrastructure only: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  Shares no code with
the HIP library or its binding.  Every function is the plain definition written
out with numpy matrix products; there is no tiling, fusion or online softmax.

Sources (the pages describing the method):
  [G]  Ultralytics glossary, "Differential Transformer" (Korean and Russian
       editions), section "How differential attention works": two softmax maps
       with scale 1/sqrt(d), combined as (map1 - lambda*map2) @ V, V twice as
       wide as the query/key width; lambda_init schedule; per-head
       normalisation ("GroupNorm") scaled by (1 - lambda_init); halved head
       count with doubled value width.
  [V2] neuralnode.tistory.com, "Differential Transformer V2 (DIFF V2) technical
       innovations": section "DIFF V1 limits" (lambda re-parameterisation),
       section "DIFF V2 innovations" items 1, 2 and 5 (2h query heads over h KV
       heads, even/odd head split, sigmoid(lambda) combine), section "GQA
       compatibility" (pairs must share a KV head).
  [N]  esgcw.com.cn news write-up of the paper, sections on the differential
       attention operator and on multi-head differential attention (lambda
       shared by all heads of a layer, per-head RMSNorm, fixed multiplier
       (1 - lambda_init)).

Readings where the pages are silent (each listed in the design notes):
  * per-head RMSNorm has no learnable gain; eps sits inside the root and is an
    explicit argument;
  * causal means query i sees keys j <= i (equal query and key lengths);
  * layout is [batch, seq, head, channel];
  * the V2 decode uses scale 1/sqrt(D) and, for an empty sequence (length 0),
    returns zeros;
  * the backward is the chain rule of the forward below (the pages print no
    gradient formulas).

Parity pins live in tests/test_oracle_*.py; none of them re-types these formulas.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "lambda_init",
    "lambda_value",
    "sigmoid",
    "diff_weights",
    "diff_attn_fwd",
    "diff_attn_bwd",
    "v2_decode",
    "v2_prefill_fwd",
    "v2_prefill_bwd",
    "v1_decode",
    "v2_prefill_fwd_block_sparse",
    "fp8_quantize_rows",
    "fp8_decode",
    "diff_attn_fwd_fp8_logits",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def lambda_init(layer: int) -> float:
    """Depth schedule of lambda's starting value for layer l >= 1 ([G]; [V2]
    "DIFF V1 limits"; [N] differential attention section):
    0.8 - 0.6 * exp(-0.3 * (l - 1))."""
    if layer < 1:
        raise ValueError("layer index starts at 1")
    return 0.8 - 0.6 * math.exp(-0.3 * (layer - 1))


def lambda_value(lq1, lk1, lq2, lk2, lam_init: float) -> float:
    """Re-parameterised lambda from the four learnable vectors ([V2] "DIFF V1
    limits"; [N] differential attention section):
    exp(<lq1, lk1>) - exp(<lq2, lk2>) + lambda_init, the sums taken over the
    vector dimension.  One scalar per layer, shared by all heads ([N])."""
    a = float(np.dot(_f64(lq1), _f64(lk1)))
    b = float(np.dot(_f64(lq2), _f64(lk2)))
    return math.exp(a) - math.exp(b) + float(lam_init)


def sigmoid(x):
    """Logistic function used by the V2 combine ([V2] item 5)."""
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax of a score matrix whose masked entries are -inf."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool,
            rows: np.ndarray) -> np.ndarray:
    """scale * q[rows] @ k^T with keys j > i set to -inf when causal."""
    s = (q[rows] @ k.T) * scale
    if causal:
        cols = np.arange(k.shape[0])
        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
    return s


def diff_weights(q1, k1, q2, k2, lam: float, scale: float | None = None,
                 causal: bool = False) -> np.ndarray:
    """The combined attention map softmax(q1 k1^T s) - lam * softmax(q2 k2^T s)
    for one head ([G]), q*, k*: [n, d].  Rows sum to 1 - lam; entries may be
    negative."""
    q1, k1, q2, k2 = map(_f64, (q1, k1, q2, k2))
    d = q1.shape[-1]
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows = np.arange(q1.shape[0])
    p1 = _softmax_rows(_scores(q1, k1, s, causal, rows))
    p2 = _softmax_rows(_scores(q2, k2, s, causal, rows))
    return p1 - lam * p2


def diff_attn_fwd(q1, k1, q2, k2, v, lam: float, lam_init: float, *,
                  causal: bool = True, norm: bool = True, eps: float = 1e-5,
                  scale: float | None = None, rows=None,
                  return_aux: bool = False):
    """Multi-head differential attention forward.

    q1, k1, q2, k2: [B, S, H, d]; v: [B, S, H, dv] (dv = 2d in the pages' model,
    any dv accepted here).  lam is the layer's scalar lambda, lam_init the
    constant of the (1 - lambda_init) multiplier.

    Per batch b and head h ([G]; [N] multi-head section):
      P_m = softmax(scale * Q_m K_m^T)  (scale 1/sqrt(d), d = query/key width)
      O   = (P_1 - lam * P_2) @ V
      Y   = O / sqrt(mean_c O^2 + eps) * (1 - lam_init)   if norm, else O.

    rows: optional 1-D array of query positions to evaluate (all keys each row
    may see are still used); default all positions.
    Returns Y [B, R, H, dv]; with return_aux also a dict holding O, A1 = P_1 V,
    A2 = P_2 V, lse1, lse2 (natural-log partition functions of the scaled
    scores, [B, H, R]) and rstd ([B, H, R], ones when norm is off).
    """
    q1, k1, q2, k2, v = map(_f64, (q1, k1, q2, k2, v))
    B, S, H, d = q1.shape
    dv = v.shape[-1]
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    Y = np.empty((B, R, H, dv))
    aux = {key: np.empty((B, R, H, dv)) for key in ("O", "A1", "A2")}
    for key in ("lse1", "lse2", "rstd"):
        aux[key] = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            s1 = _scores(q1[b, :, h], k1[b, :, h], s, causal, rows)
            s2 = _scores(q2[b, :, h], k2[b, :, h], s, causal, rows)
            p1 = _softmax_rows(s1)
            p2 = _softmax_rows(s2)
            vv = v[b, :, h]
            a1 = p1 @ vv
            a2 = p2 @ vv
            o = (p1 - lam * p2) @ vv
            if norm:
                r = 1.0 / np.sqrt(np.mean(o * o, axis=-1) + eps)
                y = o * r[:, None] * (1.0 - lam_init)
            else:
                r = np.ones(R)
                y = o
            Y[b, :, h] = y
            if return_aux:
                aux["O"][b, :, h] = o
                aux["A1"][b, :, h] = a1
                aux["A2"][b, :, h] = a2
                m1 = np.max(s1, axis=-1)
                m2 = np.max(s2, axis=-1)
                aux["lse1"][b, h] = m1 + np.log(np.sum(np.exp(s1 - m1[:, None]), axis=-1))
                aux["lse2"][b, h] = m2 + np.log(np.sum(np.exp(s2 - m2[:, None]), axis=-1))
                aux["rstd"][b, h] = r
    if return_aux:
        return Y, aux
    return Y


def diff_attn_bwd(q1, k1, q2, k2, v, dy, *, lam_init: float,
                  lam_vectors=None, lam_fixed: float | None = None,
                  causal: bool = True, norm: bool = True, eps: float = 1e-5,
                  scale: float | None = None) -> dict:
    """Gradients of L = <dy, Y> for the forward above, by the chain rule.

    lambda comes either from lam_vectors = (lq1, lk1, lq2, lk2) (then the four
    vector gradients are returned) or from lam_fixed (then d lambda itself is
    returned).  No gradient flows into lambda_init or the (1 - lambda_init)
    multiplier, which the pages call a fixed multiplier ([N]).

    Steps, per (b, h), with a = 1 - lam_init:
      Y = a r O,  r = (mean_c O^2 + eps)^-1/2
      g = dL/dO = a r dy - a r^3 O (sum_c dy O) / dv        (g = dy if no norm)
      O = A1 - lam A2, A_m = P_m V:  dA1 = g, dA2 = -lam g,
                                      dlam += -sum(g * A2)
      dV  = P1^T dA1 + P2^T dA2,  dP_m = dA_m V^T
      dS_m = P_m * (dP_m - rowsum(P_m * dP_m))
      dQ_m = scale dS_m K_m,  dK_m = scale dS_m^T Q_m
      lam = e^al - e^be + lam_init, al = <lq1,lk1>, be = <lq2,lk2>:
      dlq1 = dlam e^al lk1, dlk1 = dlam e^al lq1,
      dlq2 = -dlam e^be lk2, dlk2 = -dlam e^be lq2.
    """
    q1, k1, q2, k2, v, dy = map(_f64, (q1, k1, q2, k2, v, dy))
    B, S, H, d = q1.shape
    dv_w = v.shape[-1]
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if lam_vectors is not None:
        lq1, lk1, lq2, lk2 = map(_f64, lam_vectors)
        lam = lambda_value(lq1, lk1, lq2, lk2, lam_init)
    else:
        if lam_fixed is None:
            raise ValueError("need lam_vectors or lam_fixed")
        lam = float(lam_fixed)
    rows = np.arange(S)
    out = {key: np.zeros_like(x) for key, x in
           (("dq1", q1), ("dk1", k1), ("dq2", q2), ("dk2", k2), ("dv", v))}
    dlam = 0.0
    a = 1.0 - lam_init
    for b in range(B):
        for h in range(H):
            Q1, K1, Q2, K2, V = (t[b, :, h] for t in (q1, k1, q2, k2, v))
            dY = dy[b, :, h]
            P1 = _softmax_rows(_scores(Q1, K1, s, causal, rows))
            P2 = _softmax_rows(_scores(Q2, K2, s, causal, rows))
            A1 = P1 @ V
            A2 = P2 @ V
            O = A1 - lam * A2
            if norm:
                r = 1.0 / np.sqrt(np.mean(O * O, axis=-1) + eps)
                dot = np.sum(dY * O, axis=-1)
                g = a * r[:, None] * dY - a * (r ** 3 * dot)[:, None] * O / dv_w
            else:
                g = dY
            dA1 = g
            dA2 = -lam * g
            dlam += -float(np.sum(g * A2))
            out["dv"][b, :, h] = P1.T @ dA1 + P2.T @ dA2
            for P, dA, Q, K, kq, kk in ((P1, dA1, Q1, K1, "dq1", "dk1"),
                                        (P2, dA2, Q2, K2, "dq2", "dk2")):
                dP = dA @ V.T
                dS = P * (dP - np.sum(P * dP, axis=-1, keepdims=True))
                out[kq][b, :, h] = s * (dS @ K)
                out[kk][b, :, h] = s * (dS.T @ Q)
    if lam_vectors is not None:
        ea = math.exp(float(np.dot(lq1, lk1)))
        eb = math.exp(float(np.dot(lq2, lk2)))
        out["dlq1"] = dlam * ea * lk1
        out["dlk1"] = dlam * ea * lq1
        out["dlq2"] = -dlam * eb * lk2
        out["dlk2"] = -dlam * eb * lq2
    out["dlambda"] = dlam
    out["lambda"] = lam
    return out


def diff_attn_lambda_grad(q1, k1, q2, k2, v, dy, *, lam_init: float,
                          lam_vectors=None, lam_fixed: float | None = None,
                          causal: bool = True, norm: bool = True, eps: float = 1e-5,
                          scale: float | None = None) -> dict:
    """The lambda part of diff_attn_bwd on its own (same chain rule, same
    steps, without dQ, dK, dV), for sizes where the full backward is too slow:
    per (b, h), O = A1 - lam A2 with A_m = P_m V, g = dL/dO through the
    per-head RMSNorm, dlam += -sum(g * A2); then the four vector gradients
    from lam = e^al - e^be + lam_init.  Returns dlambda, lambda and, with
    lam_vectors, dlq1, dlk1, dlq2, dlk2."""
    q1, k1, q2, k2, v, dy = map(_f64, (q1, k1, q2, k2, v, dy))
    B, S, H, d = q1.shape
    dv_w = v.shape[-1]
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if lam_vectors is not None:
        lq1, lk1, lq2, lk2 = map(_f64, lam_vectors)
        lam = lambda_value(lq1, lk1, lq2, lk2, lam_init)
    else:
        if lam_fixed is None:
            raise ValueError("need lam_vectors or lam_fixed")
        lam = float(lam_fixed)
    rows = np.arange(S)
    a = 1.0 - lam_init
    dlam = 0.0
    for b in range(B):
        for h in range(H):
            V = v[b, :, h]
            dY = dy[b, :, h]
            A1 = _softmax_rows(_scores(q1[b, :, h], k1[b, :, h], s, causal, rows)) @ V
            A2 = _softmax_rows(_scores(q2[b, :, h], k2[b, :, h], s, causal, rows)) @ V
            O = A1 - lam * A2
            if norm:
                r = 1.0 / np.sqrt(np.mean(O * O, axis=-1) + eps)
                dot = np.sum(dY * O, axis=-1)
                g = a * r[:, None] * dY - a * (r ** 3 * dot)[:, None] * O / dv_w
            else:
                g = dY
            dlam += -float(np.sum(g * A2))
    out = {"dlambda": dlam, "lambda": lam}
    if lam_vectors is not None:
        ea = math.exp(float(np.dot(lq1, lk1)))
        eb = math.exp(float(np.dot(lq2, lk2)))
        out["dlq1"] = dlam * ea * lk1
        out["dlk1"] = dlam * ea * lq1
        out["dlq2"] = -dlam * eb * lk2
        out["dlk2"] = -dlam * eb * lq2
    return out


def v2_decode(q, k_cache, v_cache, lam, seqlens=None, scale: float | None = None):
    """DIFF V2 decode step with grouped-query attention ([V2] items 1, 2, 5 and
    "GQA compatibility").

    q: [B, Hq, D] (one new token per sequence); k_cache, v_cache:
    [B, S_kv, Hkv, D]; query head t reads KV head t // (Hq / Hkv), the usual
    grouped-query assignment.  Every query head runs ordinary softmax
    attention over the first seqlens[b] cached keys (all S_kv by default);
    then heads are split into even and odd along the head axis and combined
    as attn[even] - sigmoid(lam) * attn[odd].  lam: [Hq/2] shared by the batch,
    or [B, Hq/2].  Returns [B, Hq/2, D].  A sequence of length 0 yields zeros.
    """
    q, k_cache, v_cache = map(_f64, (q, k_cache, v_cache))
    B, Hq, D = q.shape
    S_kv, Hkv = k_cache.shape[1], k_cache.shape[2]
    if Hq % Hkv or (Hq // Hkv) % 2:
        raise ValueError("each even/odd query-head pair must share a KV head")
    group = Hq // Hkv
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lam = _f64(lam)
    if lam.ndim == 1:
        lam = np.broadcast_to(lam, (B, Hq // 2))
    lens = np.full(B, S_kv) if seqlens is None else np.asarray(seqlens)
    attn = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(lens[b])
        for t in range(Hq):
            if n == 0:
                continue
            j = t // group
            K = k_cache[b, :n, j]
            V = v_cache[b, :n, j]
            sc = (K @ q[b, t]) * s
            p = np.exp(sc - np.max(sc))
            attn[b, t] = (p / np.sum(p)) @ V
    return attn[:, 0::2] - sigmoid(lam)[:, :, None] * attn[:, 1::2]


def v2_prefill_fwd(q, k, v, lam, *, causal: bool = True, scale: float | None = None, rows=None):
    """DIFF V2 forward over a whole sequence with grouped-query attention
    ([V2] section "DIFF V2 innovations" items 1, 2 and 5; section "GQA
    compatibility").

    q: [B, S, Hq, D]; k, v: [B, S, Hkv, D]; query head t reads KV head
    t // (Hq / Hkv), so each even/odd pair (2p, 2p + 1) shares one KV head.
    Every query head runs ordinary softmax attention (scale 1/sqrt(D), causal:
    query i sees keys j <= i); then out[b, i, p] = attn[2p] - sigmoid(lam) *
    attn[2p + 1] with lam per token and pair: lam is [B, S, Hq/2] or anything
    numpy broadcasts to it ([Hq/2] shares one vector across batch and tokens).
    No per-head normalisation (V2 drops it).  rows: optional query-row indices
    to evaluate (the output then has len(rows) rows).  Returns
    [B, S or len(rows), Hq/2, D].
    """
    q, k, v = map(_f64, (q, k, v))
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv or (Hq // Hkv) % 2:
        raise ValueError("each even/odd query-head pair must share a KV head")
    group = Hq // Hkv
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lam = np.broadcast_to(_f64(lam), (B, S, Hq // 2))
    rows = np.arange(S) if rows is None else np.asarray(rows)
    attn = np.zeros((B, len(rows), Hq, D))
    for b in range(B):
        for t in range(Hq):
            j = t // group
            sc = (q[b, rows, t] @ k[b, :, j].T) * s
            if causal:
                sc = np.where(np.arange(S)[None, :] > rows[:, None], -np.inf, sc)
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            attn[b, :, t] = (p / p.sum(axis=1, keepdims=True)) @ v[b, :, j]
    return attn[:, :, 0::2] - sigmoid(lam[:, rows])[..., None] * attn[:, :, 1::2]


def v2_prefill_bwd(q, k, v, lam, dout, *, causal: bool = True, scale: float | None = None) -> dict:
    """Gradients of L = <dout, out> for v2_prefill_fwd, by the chain rule (the
    pages print no gradient formulas; [V2] sections "DIFF V2 innovations"
    items 1, 2, 5 and "GQA compatibility" define the forward).

    Per batch entry and pair (even head e = 2p, odd head o = 2p + 1, both on KV
    head j), with sigma = sigmoid(lam) per token:
      out = A_e - sigma A_o,  A_t = P_t V,  P_t = softmax(s Q_t K^T)
      dA_e = dout,  dA_o = -sigma dout,  dlam = -sigma (1 - sigma) <dout, A_o>
      per head t:  dP_t = dA_t V^T,  dS_t = P_t * (dP_t - rowsum(P_t * dP_t))
                   dQ_t = s dS_t K,  dK += s dS_t^T Q_t,  dV += P_t^T dA_t
    (dK and dV sum over every query head that reads the KV head).  Returns
    dq [B, S, Hq, D], dk and dv [B, S, Hkv, D] and dlam [B, S, Hq/2] (the
    gradient for a separate lam value per (batch, token, pair); a broadcast
    lam's gradient is its sum over the broadcast axes).
    """
    q, k, v, dout = map(_f64, (q, k, v, dout))
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv or (Hq // Hkv) % 2:
        raise ValueError("each even/odd query-head pair must share a KV head")
    group = Hq // Hkv
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    sig = sigmoid(np.broadcast_to(_f64(lam), (B, S, Hq // 2)))
    rows = np.arange(S)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dlam = np.zeros((B, S, Hq // 2))
    for b in range(B):
        for p in range(Hq // 2):
            j = (2 * p) // group
            K, V = k[b, :, j], v[b, :, j]
            g = dout[b, :, p]
            sg = sig[b, :, p][:, None]
            for t, dA in ((2 * p, g), (2 * p + 1, -sg * g)):
                P = _softmax_rows(_scores(q[b, :, t], K, s, causal, rows))
                if t % 2:
                    dlam[b, :, p] = -(sg[:, 0] * (1.0 - sg[:, 0])) * np.sum(g * (P @ V), axis=-1)
                dP = dA @ V.T
                dS = P * (dP - np.sum(P * dP, axis=-1, keepdims=True))
                dq[b, :, t] = s * (dS @ K)
                dk[b, :, j] += s * (dS.T @ q[b, :, t])
                dv[b, :, j] += P.T @ dA
    return {"dq": dq, "dk": dk, "dv": dv, "dlam": dlam}


def v1_decode(q1, q2, k1_cache, k2_cache, v_cache, lam: float, lam_init: float, seqlens=None, *,
              norm: bool = True, eps: float = 1e-5, scale: float | None = None):
    """DIFF V1 decode step: the V1 operator for one new query token per
    sequence over a KV cache that holds K1, K2 and V ([G]; [N] multi-head
    section; [V2] "DIFF V1 limits" names the decode cost of this layout).

    q1, q2: [B, H, d]; k1_cache, k2_cache: [B, S_kv, H, d]; v_cache:
    [B, S_kv, H, dv].  Per batch b and head h, over the first seqlens[b] cached
    keys (all S_kv by default; the cache already holds the new token):
      P_m = softmax(scale q_m K_m^T),  O = (P_1 - lam P_2) V,
      Y = O / sqrt(mean_c O^2 + eps) (1 - lam_init)   if norm, else O.
    A sequence of length 0 yields zeros.  Returns Y [B, H, dv].
    """
    q1, q2, k1_cache, k2_cache, v_cache = map(_f64, (q1, q2, k1_cache, k2_cache, v_cache))
    B, H, d = q1.shape
    S_kv, dv = k1_cache.shape[1], v_cache.shape[-1]
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lens = np.full(B, S_kv) if seqlens is None else np.asarray(seqlens)
    out = np.zeros((B, H, dv))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(H):
            maps = []
            for q, kc in ((q1, k1_cache), (q2, k2_cache)):
                sc = (kc[b, :n, h] @ q[b, h]) * s
                e = np.exp(sc - np.max(sc))
                maps.append(e / np.sum(e))
            o = (maps[0] - lam * maps[1]) @ v_cache[b, :n, h]
            if norm:
                o = o / np.sqrt(np.mean(o * o) + eps) * (1.0 - lam_init)
            out[b, h] = o
    return out


def v2_prefill_fwd_block_sparse(q, k, v, lam, block_mask, *, q_block: int = 128, k_block: int = 64,
                                causal: bool = True, scale: float | None = None, rows=None):
    """DIFF V2 forward restricted to selected key blocks, one selection per
    even/odd head pair ([V2] "practical considerations": DIFF V2 works with
    sparse attention frameworks by selecting blocks per head pair inside a GQA
    group; [G]'s neighbouring glossary entry: sparse attention scores only a
    fixed subset of token pairs and sets every other weight to 0).

    block_mask: bool [B, Hq/2, ceil(S / q_block), ceil(S / k_block)]; query i
    of pair p may attend key j iff block_mask[b, p, i // q_block, j // k_block]
    (and j <= i when causal).  Both heads of the pair use the pair's
    selection; each head's softmax runs over its allowed keys only.  A row
    with no allowed key gives zeros.  rows: optional query positions to
    evaluate (default all).  Returns [B, R, Hq/2, D].
    """
    q, k, v = map(_f64, (q, k, v))
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv or (Hq // Hkv) % 2:
        raise ValueError("each even/odd query-head pair must share a KV head")
    group = Hq // Hkv
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lam = np.broadcast_to(_f64(lam), (B, S, Hq // 2))
    block_mask = np.asarray(block_mask, dtype=bool)
    keys = np.arange(S)
    rows = keys if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, rows.shape[0], Hq // 2, D))
    for b in range(B):
        for p in range(Hq // 2):
            allowed = block_mask[b, p][rows[:, None] // q_block, keys[None, :] // k_block]
            if causal:
                allowed &= keys[None, :] <= rows[:, None]
            live = allowed.any(axis=1)
            attn = []
            for t in (2 * p, 2 * p + 1):
                j = t // group
                sc = np.where(allowed, (q[b, rows, t] @ k[b, :, j].T) * s, -np.inf)
                m = np.where(live, sc.max(axis=1), 0.0)
                e = np.where(allowed, np.exp(sc - m[:, None]), 0.0)
                den = np.where(live, e.sum(axis=1), 1.0)
                attn.append((e / den[:, None]) @ v[b, :, j])
            out[b, :, p] = attn[0] - sigmoid(lam[b, rows, p])[:, None] * attn[1]
    return out


# ---------------------------------------------------------------------------
# Low-bit attention logits ([N]'s quantisation discussion and [V2]'s outlook
# name absmax dynamic post-training quantisation of the attention logits to
# 8/6/4 bits and a low-bit FlashAttention as the kernel it enables).  The
# reading here: Q1, K1, Q2, K2 are quantised per row (one token of one head) to
# fp8 e4m3 with an absmax scale rounded up to a power of two, and the score
# products use the dequantised values; everything after the scores is the
# ordinary forward.

E4M3_MAX = 448.0


def _e4m3_table():
    t = np.empty(256)
    for c in range(256):
        sgn = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sgn * m * 2.0 ** -9
        else:
            t[c] = sgn * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3 = _e4m3_table()


def fp8_decode(codes) -> np.ndarray:
    """Values of fp8 e4m3 codes (uint8)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def _round_half_even(x):
    return np.round(x)   # numpy rounds halves to even


def _e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round float values with |v| <= 448 to the nearest e4m3 code, ties to the
    even code (OCP 8-bit floating point, E4M3: 3 mantissa bits, exponent bias
    7, subnormal step 2^-9, largest finite 448)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX):
        raise ValueError("value beyond the e4m3 range")
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ex = np.maximum(ex, -6.0)                      # subnormals share the 2^-6 binade's step
    ulp = 2.0 ** (ex - 3)
    q = _round_half_even(a / ulp) * ulp            # exact: a / ulp is a float with few bits
    # encode q
    codes = np.zeros(a.shape, dtype=np.uint8)
    nz = q > 0
    e_q = np.floor(np.log2(np.where(nz, q, 1.0)))
    sub = nz & (e_q < -6)
    norm = nz & ~sub
    codes[sub] = (q[sub] / 2.0 ** -9).astype(np.uint8)
    en = (e_q[norm] + 7).astype(np.int64)
    mn = np.round((q[norm] / 2.0 ** e_q[norm] - 1.0) * 8).astype(np.int64)
    codes[norm] = (en << 3 | mn).astype(np.uint8)
    # The format has a signed zero: a negative value keeps its sign bit even
    # when it rounds to zero.
    codes |= np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return codes


def fp8_quantize_rows(x):
    """Per-row (last axis) absmax quantisation to fp8 e4m3 with a power-of-two
    scale: e is the smallest integer with max|x_row| * 2^-e <= 448 (clamped to
    [-120, 120]; 0 for an all-zero row), codes = RNE_e4m3(x * 2^-e).
    Returns (codes uint8 with x's shape, e int32 with the row shape); the
    dequantised row is fp8_decode(codes) * 2^e."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1)
    m, E = np.frexp(amax)                    # amax = m 2^E, m in [0.5, 1)
    mant, E = 2.0 * m, E - 1                 # amax = mant 2^E, mant in [1, 2)
    e = E - 8 + (mant > 1.75)
    e = np.where(amax > 0, np.clip(e, -120, 120), 0).astype(np.int32)
    codes = _e4m3_encode(x * 2.0 ** (-e[..., None].astype(np.float64)))
    return codes, e


def diff_attn_fwd_fp8_logits(q1, k1, q2, k2, v, lam: float, lam_init: float, **kw):
    """diff_attn_fwd with Q1, K1, Q2, K2 replaced by their per-row fp8 e4m3
    quantisations (fp8_quantize_rows, dequantised); V and everything after the
    scores as in diff_attn_fwd."""
    deq = []
    for t in (q1, k1, q2, k2):
        c, e = fp8_quantize_rows(t)
        deq.append(fp8_decode(c) * 2.0 ** e[..., None].astype(np.float64))
    return diff_attn_fwd(deq[0], deq[1], deq[2], deq[3], v, lam, lam_init, **kw)
