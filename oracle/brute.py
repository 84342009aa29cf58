"""Scalar pure-Python twins of the oracle for tiny shapes.

Test infrastructure only.  Written independently of diffattn_oracle.py: plain
nested loops, math.fsum for every sum, and softmax taken directly as
exp(s_j) / sum_k exp(s_k) without the max shift (so a shift mistake in either
version shows up as a disagreement; callers keep logits within about +-600).
Same definitions as the vectorised oracle (see its module docstring for the
pages each step follows).
"""
from __future__ import annotations

import math


def _dot(x, y):
    return math.fsum(a * b for a, b in zip(x, y))


def _softmax(scores):
    e = [math.exp(t) for t in scores]
    z = math.fsum(e)
    return [t / z for t in e]


def brute_diff_attn_fwd(q1, k1, q2, k2, v, lam, lam_init, causal=True,
                        norm=True, eps=1e-5, scale=None):
    """Nested lists or arrays q*: [B][S][H][d], v: [B][S][H][dv]; returns a
    nested list Y[B][S][H][dv] as floats."""
    B, S, H = len(q1), len(q1[0]), len(q1[0][0])
    d = len(q1[0][0][0])
    dv = len(v[0][0][0])
    s = 1.0 / math.sqrt(d) if scale is None else scale
    Y = [[[[0.0] * dv for _ in range(H)] for _ in range(S)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(S):
                keys = range(i + 1) if causal else range(S)
                w1 = _softmax([s * _dot(q1[b][i][h], k1[b][j][h]) for j in keys])
                w2 = _softmax([s * _dot(q2[b][i][h], k2[b][j][h]) for j in keys])
                o = []
                for c in range(dv):
                    o.append(math.fsum((w1[n] - lam * w2[n]) * float(v[b][j][h][c])
                                       for n, j in enumerate(keys)))
                if norm:
                    ms = math.fsum(x * x for x in o) / dv
                    f = (1.0 - lam_init) / math.sqrt(ms + eps)
                    o = [x * f for x in o]
                Y[b][i][h] = o
    return Y


def brute_v2_decode(q, k_cache, v_cache, lam, seqlens=None, scale=None):
    """q: [B][Hq][D]; caches: [B][S_kv][Hkv][D]; lam: [Hq/2] or [B][Hq/2].
    Returns out[B][Hq/2][D]."""
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    S_kv, Hkv = len(k_cache[0]), len(k_cache[0][0])
    group = Hq // Hkv
    s = 1.0 / math.sqrt(D) if scale is None else scale
    lam = [float(x) for x in lam] if not hasattr(lam[0], "__len__") else lam
    lam_rows = [lam] * B if not hasattr(lam[0], "__len__") else lam
    out = []
    for b in range(B):
        n = S_kv if seqlens is None else int(seqlens[b])
        heads = []
        for t in range(Hq):
            if n == 0:
                heads.append([0.0] * D)
                continue
            j = t // group
            w = _softmax([s * _dot(q[b][t], k_cache[b][x][j]) for x in range(n)])
            heads.append([math.fsum(w[x] * float(v_cache[b][x][j][c]) for x in range(n))
                          for c in range(D)])
        row = []
        for p in range(Hq // 2):
            sg = 1.0 / (1.0 + math.exp(-float(lam_rows[b][p])))
            row.append([heads[2 * p][c] - sg * heads[2 * p + 1][c] for c in range(D)])
        out.append(row)
    return out


def brute_v2_prefill_fwd(q, k, v, lam, causal=True, scale=None):
    """q: [B][S][Hq][D]; k, v: [B][S][Hkv][D]; lam: [B][S][Hq/2].
    Returns out[B][S][Hq/2][D]."""
    B, S, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    group = Hq // Hkv
    s = 1.0 / math.sqrt(D) if scale is None else scale
    out = []
    for b in range(B):
        seq = []
        for i in range(S):
            n = i + 1 if causal else S
            heads = []
            for t in range(Hq):
                j = t // group
                w = _softmax([s * _dot(q[b][i][t], k[b][x][j]) for x in range(n)])
                heads.append([math.fsum(w[x] * float(v[b][x][j][c]) for x in range(n)) for c in range(D)])
            row = []
            for p in range(Hq // 2):
                sg = 1.0 / (1.0 + math.exp(-float(lam[b][i][p])))
                row.append([heads[2 * p][c] - sg * heads[2 * p + 1][c] for c in range(D)])
            seq.append(row)
        out.append(seq)
    return out
