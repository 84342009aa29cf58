// Helpers shared by the fused attention kernels on gfx950 matrix cores that
// compute scores transposed, S^T = K Q^T with 32x32x16 instructions: a lane
// owns one query column (l % 32) in half h = l / 32, and its 16 score
// registers of a 32-key sub-tile are keys 8 h + 0..7 and 16 + 8 h + 0..7 -
// the k-slots of two PV steps O^T = V^T W^T (K rows are read in a permuted
// order inside each 16-row block to make that so).
#pragma once

#include "common.h"

namespace diffattn {
namespace {

// Row of the K tile that lane row index i (0..31) reads: bits 2 and 3 of the
// position inside each 16-row block are swapped.
__device__ __forceinline__ int k_row_perm(int i) {
  return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Key (relative to its 32-key sub-tile) held by score register r of a lane in
// half h.
__device__ __forceinline__ int key_of_reg(int r, int h) { return ((r & 8) << 1) + 8 * h + (r & 7); }

// Online log2-domain sum of one lane's share of a map's row against a lazily
// moved reference m: the sub-tile's terms 2^(s c - m) are summed directly,
// and only when their sum leaves [0, 2^64] (a score more than 64 above the
// reference, or no reference yet) is the reference raised to the sub-tile's
// top score and the sum redone.  l is always relative to m; m need not be the
// row's top score, only within 64 of it, so a map's weights 2^(s c - L) are
// bounded by 1, not by 2^(m - L).
__device__ __forceinline__ void lse_update(const f32x16 &s, float c, float &m, float &l) {
  float a[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) a[r] = fast_exp2(fmaf(s[r], c, -m));
#pragma unroll
  for (int r = 4; r < 16; ++r) a[r & 3] += fast_exp2(fmaf(s[r], c, -m));
  float t = (a[0] + a[1]) + (a[2] + a[3]);
  if (!(t <= 0x1p64f)) {  // also taken for NaN terms (m still -inf)
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float mn = fmaxf(m, mx * c);
    const float ms = mn == kNegInf ? 0.f : mn;
    l = m == kNegInf ? 0.f : l * fast_exp2(m - ms);
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = fast_exp2(fmaf(s[r], c, -ms));
#pragma unroll
    for (int r = 4; r < 16; ++r) a[r & 3] += fast_exp2(fmaf(s[r], c, -ms));
    t = (a[0] + a[1]) + (a[2] + a[3]);
    m = mn;
  }
  l += t;
}

// Full-row reference M (the larger of the two half-waves' references) and log2
// partition function L from the two half-waves' (m, l).
__device__ __forceinline__ void lse_finish(float m, float l, float &M, float &L) {
  const float mo = other_half(m), lo = other_half(l);
  M = fmaxf(m, mo);
  const float Ms = M == kNegInf ? 0.f : M;
  L = Ms + log2f(l * fast_exp2(m - Ms) + lo * fast_exp2(mo - Ms));
}

// Exponent sigma that brings a row whose largest |weight| is wmax just under
// 2^15.
__device__ __forceinline__ float row_scale_log2(float wmax) {
  return fminf(fmaxf(floorf(15.f - log2f(wmax)), -100.f), 100.f);
}

__device__ __forceinline__ f16x8 pack8(const float *w) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const f32x2 x = {w[i], w[i + 1]};
    const f16x2 y = __builtin_convertvector(x, f16x2);
    r[i] = y[0];
    r[i + 1] = y[1];
  }
  return r;
}

// w = hi + lo with both halves in fp16: lo carries the rounding residual of
// hi, so hi V + lo V is accurate to about 2^-22 of |w| |V|.
__device__ __forceinline__ void pack8_hilo(const float *w, f16x8 &hi, f16x8 &lo) {
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const f32x2 x = {w[i], w[i + 1]};
    const f16x2 y = __builtin_convertvector(x, f16x2);
    const f32x2 back = __builtin_convertvector(y, f32x2);
    const f16x2 z = __builtin_convertvector(x - back, f16x2);
    hi[i] = y[0];
    hi[i + 1] = y[1];
    lo[i] = z[0];
    lo[i + 1] = z[1];
  }
}

// O^T[ct] += V^T (channels 32 ct .. 32 ct + 31, keys of sub-tile chunk kc2)
// W^T for NCT channel tiles, V^T from a row-major fp16 tile with row stride
// VSTRIDE through LDS transpose reads.
template <int VSTRIDE, int NCT>
__device__ __forceinline__ void pv_step_tile(const f16 *vt, int sub, int lane, const f16x8 *wb, f32x16 *o) {
  const int h = lane >> 5, j = lane & 15, half16 = (lane >> 4) & 1;
#pragma unroll
  for (int kc2 = 0; kc2 < 2; ++kc2) {
    const int key0 = sub * 32 + kc2 * 16 + 8 * h + (j >> 2);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const f16 *p = vt + key0 * VSTRIDE + ct * 32 + 16 * half16 + 4 * (j & 3);
      const f16x4 lo = lds_read_tr16(p);
      const f16x4 hi = lds_read_tr16(p + 4 * VSTRIDE);
      const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[ct] = mfma32(a, wb[kc2], o[ct]);
    }
  }
}

// Scheduling fence for the double-buffered key loops: keeps the next tile's
// global loads above the current tile's compute and its LDS stores below it,
// so the load latency hides behind the compute (left to itself the compiler
// moved the stores, and the wait for the loads, ahead of the softmax work).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Masks one map's scores of keys past the sequence end or (causal) past the
// query.
__device__ __forceinline__ void mask_scores1(f32x16 &s, int sb, int h, int S, bool causal, int my_q) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = sb + key_of_reg(r, h);
    if (key >= S || (causal && key > my_q)) s[r] = kNegInf;
  }
}

// Masks the scores of keys past the sequence end or (causal) past the query.
__device__ __forceinline__ void mask_scores(f32x16 &s1, f32x16 &s2, int sb, int h, int S, bool causal, int my_q) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = sb + key_of_reg(r, h);
    if (key >= S || (causal && key > my_q)) {
      s1[r] = kNegInf;
      s2[r] = kNegInf;
    }
  }
}

}  // namespace
}  // namespace diffattn
