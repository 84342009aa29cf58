// DIFF V2 decode step: one new query token per sequence, 2h query heads over h
// KV heads, even/odd heads of one grouped-query group combined as
// attn_even - sigmoid(lambda) attn_odd (neuralnode.tistory.com "DIFF V2
// technical innovations", section "DIFF V2 innovations" items 1, 2 and 5;
// section "GQA compatibility").
//
// Decode is bound by HBM bandwidth (that page, item 1): the kernel's job is to
// stream the K and V cache exactly once at full rate.  Split-K layout:
//   decode_split: one workgroup per (key chunk, KV head (or part of its query
//     group), batch).  Up to four query heads of the group are served by the
//     same workgroup, so for groups of 2 or 4 heads each K/V byte is read
//     once for all of them; larger groups take several workgroups per KV head
//     whose repeated reads of a chunk are meant to hit the L2 (ordinary loads
//     there, non-temporal ones only for a chunk's single reader).  Phase 1
//     streams K (D / 8 lanes per key row, 16-byte loads, whole rows per load
//     instruction) and writes log2-domain scores to LDS; phase 2 takes each
//     head's max and sum over the chunk; phase 3 streams V and accumulates the
//     probability-weighted rows.  Arithmetic is float32.  The chunk's
//     (max, sum, un-normalised output) go to the workspace.
//   decode_combine: per (batch, pair) merges the chunks by log-sum-exp
//     rescaling, normalises, and applies the even/odd sigmoid(lambda) combine.
//
// DIFF V1 decode step (glossary page "Differential Transformer", section "How
// differential attention works"; news write-up, multi-head section; the V2
// page's section "DIFF V1 limits" names this layout's decode cost: a cache of
// K1, K2 and a double-width V, with V loaded once per map when each map is a
// separate attention call).  Same split-K layout with one workgroup per (key
// chunk, head, batch): phase 1 streams K1 and K2 rows together and scores
// both maps, phase 2 takes each map's max and sum, phase 3 streams V once and
// accumulates both maps' weighted rows.  The combine merges each map's chunks,
// forms (map1 - lambda map2) V, and applies the per-head RMSNorm times
// (1 - lambda_init).
#include "common.h"
#include "kernels.h"

#include <mutex>

namespace diffattn {
namespace {

constexpr int NT = 256;
constexpr int MAX_CHUNK = 2048;  // keys per split (LDS holds the chunk's scores)

template <typename T>
__device__ __forceinline__ void to_f32x8(const u32x4 &raw, float *f);

template <>
__device__ __forceinline__ void to_f32x8<bf16>(const u32x4 &raw, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(raw[i] << 16);
    f[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
  }
}

// float32 caches: the "8 values" of a lane are two 16-byte loads.
struct Raw8 {
  u32x4 a, b;
};

template <typename T, bool STREAM = true>
struct RowLoad;

// 16-byte loads of cache rows.  STREAM: the row is read once per call, so the
// load carries the non-temporal hint (the line is not kept in the caches for
// reuse, which lets the stream run about 10 % faster than ordinary loads).
// Without STREAM (rows that other workgroups of the same call read again)
// the loads are ordinary, so the repeats can hit the L2.
template <bool STREAM>
struct RowLoad<bf16, STREAM> {
  typedef u32x4 raw_t;
  static __device__ __forceinline__ raw_t load(const bf16 *p) {
    if constexpr (STREAM) return __builtin_nontemporal_load((const u32x4 *)p);
    else return *(const u32x4 *)p;
  }
  static __device__ __forceinline__ raw_t zero() { return u32x4{0, 0, 0, 0}; }
  static __device__ __forceinline__ void cvt(const raw_t &r, float *f) { to_f32x8<bf16>(r, f); }
};

template <bool STREAM>
struct RowLoad<float, STREAM> {
  typedef Raw8 raw_t;
  static __device__ __forceinline__ raw_t load(const float *p) {
    if constexpr (STREAM)
      return Raw8{__builtin_nontemporal_load((const u32x4 *)p), __builtin_nontemporal_load((const u32x4 *)(p + 4))};
    else return Raw8{*(const u32x4 *)p, *(const u32x4 *)(p + 4)};
  }
  static __device__ __forceinline__ raw_t zero() { return Raw8{{0, 0, 0, 0}, {0, 0, 0, 0}}; }
  static __device__ __forceinline__ void cvt(const raw_t &r, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(r.a[i]);
      f[4 + i] = __uint_as_float(r.b[i]);
    }
  }
};

// STREAM: this workgroup serves every query head of its KV head (the group
// has at most NH heads), so it is the only reader of its K/V chunk.
template <typename T, int D, int NH, bool STREAM>
__global__ __launch_bounds__(NT) void decode_split_kernel(DecodeParams p) {
  constexpr int LPK = D / 8;      // lanes per key row (8 channels each)
  constexpr int KPW = 64 / LPK;   // keys per wave per load step
  constexpr int U = 4;            // load steps in flight per lane
  constexpr int STEP = 4 * KPW * U;
  typedef RowLoad<T, STREAM> RL;
  typedef typename RL::raw_t raw_t;

  __shared__ float s_lds[NH][MAX_CHUNK];
  __shared__ float red[4][NH][D];
  __shared__ float stat[4][NH];

  const int split = blockIdx.x, grp = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = lane % LPK, kl = lane / LPK;
  const int G = p.Hq / p.Hkv, per = G / NH;
  const int j = grp / per, t0 = j * G + (grp % per) * NH;
  int len = p.L;
  if (p.seqlens) len = min(max(p.seqlens[b], 0), p.L);
  const int kb = split * p.chunk;
  const int n = max(0, min(len, kb + p.chunk) - kb);

  const float c = p.scale * kLog2e;
  float q[NH][8];
#pragma unroll
  for (int u = 0; u < NH; ++u) {
    const T *qp = (const T *)p.q + b * p.qs_b + (t0 + u) * p.qs_h + part * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) q[u][e] = (float)qp[e] * c;
  }
  const T *kbase = (const T *)p.k + b * p.kvs_b + j * p.kvs_h + (int64_t)kb * p.kvs_s + part * 8;
  const T *vbase = (const T *)p.v + b * p.kvs_b + j * p.kvs_h + (int64_t)kb * p.kvs_s + part * 8;

  // Phase 1: scores (log2 domain) of every key of the chunk.
  for (int base = wave * KPW * U; base < n; base += STEP) {
    raw_t r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * KPW + kl;
      r[u] = key < n ? RL::load(kbase + (int64_t)key * p.kvs_s) : RL::zero();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      RL::cvt(r[u], kf);
      const int key = base + u * KPW + kl;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(q[hh][e], kf[e], s);
#pragma unroll
        for (int o = 1; o < LPK; o <<= 1) s += __shfl_xor(s, o);
        if (part == 0 && key < n) s_lds[hh][key] = s;
      }
    }
  }
  __syncthreads();

  // Phase 2: per-head max and sum over the chunk; scores become 2^(s - m).
  float m[NH], l[NH];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    float mx = kNegInf;
    for (int i = tid; i < n; i += NT) mx = fmaxf(mx, s_lds[hh][i]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) stat[wave][hh] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
    m[hh] = fmaxf(fmaxf(stat[0][hh], stat[1][hh]), fmaxf(stat[2][hh], stat[3][hh]));
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    float sm = 0.f;
    for (int i = tid; i < n; i += NT) {
      const float e = fast_exp2(s_lds[hh][i] - m[hh]);
      s_lds[hh][i] = e;
      sm += e;
    }
    sm = wave_sum(sm);
    if (lane == 0) stat[wave][hh] = sm;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) l[hh] = (stat[0][hh] + stat[1][hh]) + (stat[2][hh] + stat[3][hh]);

  // Phase 3: un-normalised P V over the chunk.
  float acc[NH][8];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  for (int base = wave * KPW * U; base < n; base += STEP) {
    raw_t r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * KPW + kl;
      r[u] = key < n ? RL::load(vbase + (int64_t)key * p.kvs_s) : RL::zero();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * KPW + kl;
      if (key < n) {
        float vf[8];
        RL::cvt(r[u], vf);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          const float pr = s_lds[hh][key];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pr, vf[e], acc[hh][e]);
        }
      }
    }
  }
  // Reduce over the KPW key slots of the wave, then over the 4 waves.
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[hh][e];
      for (int o = LPK; o < 64; o <<= 1) x += __shfl_xor(x, o);
      acc[hh][e] = x;
    }
  if (kl == 0) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][hh][part * 8 + e] = acc[hh][e];
  }
  __syncthreads();
  for (int i = tid; i < NH * D; i += NT) {
    const int hh = i / D, ch = i % D;
    const float x = (red[0][hh][ch] + red[1][hh][ch]) + (red[2][hh][ch] + red[3][hh][ch]);
    const int64_t slot = ((int64_t)b * p.Hq + t0 + hh) * p.splits + split;
    p.part_o[slot * D + ch] = x;
    if (ch == 0) {
      p.part_ml[slot * 2] = n > 0 ? m[hh] : kNegInf;
      p.part_ml[slot * 2 + 1] = n > 0 ? l[hh] : 0.f;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeParams p) {
  const int pr = blockIdx.x, b = blockIdx.y, ch = threadIdx.x;
  float a[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t slot0 = ((int64_t)b * p.Hq + 2 * pr + u) * p.splits;
    float M = kNegInf;
    for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.part_ml[(slot0 + s) * 2]);
    float L = 0.f, acc = 0.f;
    if (M != kNegInf) {
      for (int s = 0; s < p.splits; ++s) {
        const float w = fast_exp2(p.part_ml[(slot0 + s) * 2] - M);
        L = fmaf(p.part_ml[(slot0 + s) * 2 + 1], w, L);
        acc = fmaf(p.part_o[(slot0 + s) * D + ch], w, acc);
      }
    }
    a[u] = L > 0.f ? acc / L : 0.f;
  }
  const float lam = p.lam[b * p.lam_stride_b + pr];
  const float sg = 1.f / (1.f + expf(-lam));
  T *out = (T *)p.out + b * p.os_b + pr * p.os_h;
  out[ch] = (T)(a[0] - sg * a[1]);
}

template <typename T, int D>
hipError_t launch_typed(const DecodeParams &p, hipStream_t st) {
  const int G = p.Hq / p.Hkv;
  const int nh = (G % 4 == 0) ? 4 : 2;
  dim3 grid(p.splits, p.Hkv * (G / nh), p.B);
  // Groups of more than nh query heads take G / nh workgroups per KV head,
  // which read the same chunk: those loads stay ordinary so the repeats can
  // be served by the L2.
  const bool stream = G == nh;
  if (nh == 4 && stream)
    hipLaunchKernelGGL((decode_split_kernel<T, D, 4, true>), grid, dim3(NT), 0, st, p);
  else if (nh == 4)
    hipLaunchKernelGGL((decode_split_kernel<T, D, 4, false>), grid, dim3(NT), 0, st, p);
  else if (stream)
    hipLaunchKernelGGL((decode_split_kernel<T, D, 2, true>), grid, dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, 2, false>), grid, dim3(NT), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.Hq / 2, p.B), dim3(D), 0, st, p);
  return hipGetLastError();
}

constexpr int V1D = 64, V1DV = 128;

template <typename T>
__global__ __launch_bounds__(NT) void v1dec_split_kernel(V1DecodeParams p) {
  constexpr int LPK = V1D / 8, KPW = 64 / LPK;     // K rows: 8 lanes, 8 keys per wave step
  constexpr int LPV = V1DV / 8, KPV = 64 / LPV;    // V rows: 16 lanes, 4 keys per wave step
  constexpr int U = 4;
  typedef RowLoad<T> RL;
  typedef typename RL::raw_t raw_t;
  __shared__ float s_lds[2][MAX_CHUNK];
  __shared__ float red[4][2][V1DV];
  __shared__ float stat[4][2];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int len = p.L;
  if (p.seqlens) len = min(max(p.seqlens[b], 0), p.L);
  const int kb = split * p.chunk;
  const int n = max(0, min(len, kb + p.chunk) - kb);
  const float c = p.scale * kLog2e;

  // Phase 1: both maps' scores (log2 domain) of every key of the chunk.
  {
    const int part = lane % LPK, kl = lane / LPK;
    float q1[8], q2[8];
    const T *q1p = (const T *)p.q1 + b * p.qs_b + h * p.qs_h + part * 8;
    const T *q2p = (const T *)p.q2 + b * p.qs_b + h * p.qs_h + part * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q1[e] = (float)q1p[e] * c;
      q2[e] = (float)q2p[e] * c;
    }
    const int64_t koff = b * p.ks_b + h * p.ks_h + (int64_t)kb * p.ks_s + part * 8;
    const T *k1b = (const T *)p.k1 + koff, *k2b = (const T *)p.k2 + koff;
    for (int base = wave * KPW * U; base < n; base += 4 * KPW * U) {
      raw_t r1[U], r2[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = base + u * KPW + kl;
        r1[u] = key < n ? RL::load(k1b + (int64_t)key * p.ks_s) : RL::zero();
        r2[u] = key < n ? RL::load(k2b + (int64_t)key * p.ks_s) : RL::zero();
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float f1[8], f2[8];
        RL::cvt(r1[u], f1);
        RL::cvt(r2[u], f2);
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s1 = fmaf(q1[e], f1[e], s1);
          s2 = fmaf(q2[e], f2[e], s2);
        }
#pragma unroll
        for (int o = 1; o < LPK; o <<= 1) {
          s1 += __shfl_xor(s1, o);
          s2 += __shfl_xor(s2, o);
        }
        const int key = base + u * KPW + kl;
        if (part == 0 && key < n) {
          s_lds[0][key] = s1;
          s_lds[1][key] = s2;
        }
      }
    }
  }
  __syncthreads();

  // Phase 2: each map's max and sum over the chunk; scores become 2^(s - m).
  float m[2], l[2];
#pragma unroll
  for (int mp = 0; mp < 2; ++mp) {
    float mx = kNegInf;
    for (int i = tid; i < n; i += NT) mx = fmaxf(mx, s_lds[mp][i]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) stat[wave][mp] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int mp = 0; mp < 2; ++mp) m[mp] = fmaxf(fmaxf(stat[0][mp], stat[1][mp]), fmaxf(stat[2][mp], stat[3][mp]));
  __syncthreads();
#pragma unroll
  for (int mp = 0; mp < 2; ++mp) {
    float sm = 0.f;
    for (int i = tid; i < n; i += NT) {
      const float e = fast_exp2(s_lds[mp][i] - m[mp]);
      s_lds[mp][i] = e;
      sm += e;
    }
    sm = wave_sum(sm);
    if (lane == 0) stat[wave][mp] = sm;
  }
  __syncthreads();
#pragma unroll
  for (int mp = 0; mp < 2; ++mp) l[mp] = (stat[0][mp] + stat[1][mp]) + (stat[2][mp] + stat[3][mp]);

  // Phase 3: both maps' un-normalised P V over the chunk, V read once.
  const int part = lane % LPV, kl = lane / LPV;
  float a1[8], a2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a1[e] = a2[e] = 0.f;
  const T *vb = (const T *)p.v + b * p.vs_b + h * p.vs_h + (int64_t)kb * p.vs_s + part * 8;
  for (int base = wave * KPV * U; base < n; base += 4 * KPV * U) {
    raw_t r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * KPV + kl;
      r[u] = key < n ? RL::load(vb + (int64_t)key * p.vs_s) : RL::zero();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * KPV + kl;
      if (key < n) {
        float vf[8];
        RL::cvt(r[u], vf);
        const float p1 = s_lds[0][key], p2 = s_lds[1][key];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a1[e] = fmaf(p1, vf[e], a1[e]);
          a2[e] = fmaf(p2, vf[e], a2[e]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    for (int o = LPV; o < 64; o <<= 1) {
      a1[e] += __shfl_xor(a1[e], o);
      a2[e] += __shfl_xor(a2[e], o);
    }
  if (kl == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red[wave][0][part * 8 + e] = a1[e];
      red[wave][1][part * 8 + e] = a2[e];
    }
  }
  __syncthreads();
  for (int i = tid; i < 2 * V1DV; i += NT) {
    const int mp = i / V1DV, ch = i % V1DV;
    const float x = (red[0][mp][ch] + red[1][mp][ch]) + (red[2][mp][ch] + red[3][mp][ch]);
    const int64_t slot = (((int64_t)b * p.H + h) * 2 + mp) * p.splits + split;
    p.part_o[slot * V1DV + ch] = x;
    if (ch == 0) {
      p.part_ml[slot * 2] = n > 0 ? m[mp] : kNegInf;
      p.part_ml[slot * 2 + 1] = n > 0 ? l[mp] : 0.f;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(V1DV) void v1dec_combine_kernel(V1DecodeParams p) {
  __shared__ float ss_w[V1DV / 64];
  const int h = blockIdx.x, b = blockIdx.y, ch = threadIdx.x;
  const float lam = wave_lambda(p.lq1, p.lk1, p.lq2, p.lk2, p.lambda_dim, p.lambda_fixed, p.lambda_init);
  float a[2];
#pragma unroll
  for (int mp = 0; mp < 2; ++mp) {
    const int64_t slot0 = (((int64_t)b * p.H + h) * 2 + mp) * p.splits;
    float M = kNegInf;
    for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.part_ml[(slot0 + s) * 2]);
    float L = 0.f, acc = 0.f;
    if (M != kNegInf) {
      for (int s = 0; s < p.splits; ++s) {
        const float w = fast_exp2(p.part_ml[(slot0 + s) * 2] - M);
        L = fmaf(p.part_ml[(slot0 + s) * 2 + 1], w, L);
        acc = fmaf(p.part_o[(slot0 + s) * V1DV + ch], w, acc);
      }
    }
    a[mp] = L > 0.f ? acc / L : 0.f;
  }
  float o = fmaf(-lam, a[1], a[0]);
  if (p.norm) {
    const float ss = wave_sum(o * o);
    if ((ch & 63) == 0) ss_w[ch >> 6] = ss;
    __syncthreads();
    const float ms = (ss_w[0] + ss_w[1]) * (1.f / V1DV);
    o *= (1.f - p.lambda_init) / sqrtf(ms + p.eps);
  }
  T *out = (T *)p.out + b * p.os_b + h * p.os_h;
  out[ch] = (T)o;
}

}  // namespace

size_t v1_decode_workspace_bytes(int B, int H, int splits) {
  return (size_t)B * H * 2 * splits * (V1DV + 2) * sizeof(float);
}

hipError_t launch_v1_decode(const V1DecodeParams &p, int dtype, hipStream_t st) {
  dim3 grid(p.splits, p.H, p.B);
  if (dtype == 0)
    hipLaunchKernelGGL(v1dec_split_kernel<float>, grid, dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL(v1dec_split_kernel<bf16>, grid, dim3(NT), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == 0)
    hipLaunchKernelGGL(v1dec_combine_kernel<float>, dim3(p.H, p.B), dim3(V1DV), 0, st, p);
  else
    hipLaunchKernelGGL(v1dec_combine_kernel<bf16>, dim3(p.H, p.B), dim3(V1DV), 0, st, p);
  return hipGetLastError();
}

size_t decode_workspace_bytes(int B, int Hq, int D, int splits) {
  return (size_t)B * Hq * splits * (D + 2) * sizeof(float);
}

int decode_auto_splits(int B, int Hkv, int L) {
  const int min_splits = (L + MAX_CHUNK - 1) / MAX_CHUNK;
  const int units = max(B * Hkv, 1);
  // Aim for about 6144 workgroups over the 256 CUs: 5-7 resident per CU, so
  // several rounds and a short tail (the 64 x 16-head, 8192-key caches read
  // 2-3 % faster with 6 splits than with 4).
  int s = (6144 + units - 1) / units;
  s = max(s, min_splits);
  s = min(s, max(1, (L + 255) / 256));  // at least ~256 keys per split
  return max(max(s, min_splits), 1);
}

int decode_max_chunk() { return MAX_CHUNK; }

hipError_t launch_decode(const DecodeParams &p, int dtype, hipStream_t st) {
  if (dtype == 0) return p.D == 64 ? launch_typed<float, 64>(p, st) : launch_typed<float, 128>(p, st);
  return p.D == 64 ? launch_typed<bf16, 64>(p, st) : launch_typed<bf16, 128>(p, st);
}

// Fixed scratch of the allocation-free decode entry point (for callers that
// cannot allocate device memory): the split kernel's partial outputs and
// (max, sum) pairs.  Every GPU the library runs on holds its own copy until
// the process ends.  Host code uses the per-device address from
// hipGetSymbolAddress, never the array's name (a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

void *decode_scratch(hipError_t *err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    addr[dev] = ptr;
  }
  *err = hipSuccess;
  return addr[dev];
}

}  // namespace diffattn
