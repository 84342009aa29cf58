// Reference vector-ALU forward of multi-head differential attention.
//
// One lane per query row, two passes over the keys the row may see:
//   pass 1: running max and sum of 2^(s c) for each map (c = scale * log2 e),
//           giving each map's log2 partition function L_m;
//   pass 2: W_j = 2^(s1_j c - L1) - lambda 2^(s2_j c - L2) (the combined,
//           already normalised weight of key j) and O = sum_j W_j V_j.
// Then the per-head RMSNorm times (1 - lambda_init) when norm is set.  This is
// the operator of the glossary page ("How differential attention works") and
// of the news write-up's multi-head section, in float32 arithmetic.  It serves
// small head sizes (the 8/16 single-head case) and any supported (d, dv) in
// float32 or bf16 storage; the fused matrix-core kernel serves bf16 d = 64.
#include "common.h"
#include "kernels.h"

namespace diffattn {

template <typename T>
__device__ __forceinline__ float ld(const T *p) { return (float)(*p); }

template <typename T, int D, int DV>
__global__ __launch_bounds__(64) void fwd_generic_kernel(FwdParams p) {
  const int bh = blockIdx.y;
  const int b = bh / p.H, h = bh % p.H;
  const int i = blockIdx.x * 64 + threadIdx.x;
  const float lam = wave_lambda(p.lq1, p.lk1, p.lq2, p.lk2, p.lambda_dim, p.lambda_fixed, p.lambda_init);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && p.lambda_out) *p.lambda_out = lam;
  if (i >= p.S) return;

  const T *q1 = (const T *)p.q1 + b * p.qs_b + (int64_t)i * p.qs_s + h * p.qs_h;
  const T *q2 = (const T *)p.q2 + b * p.qs_b + (int64_t)i * p.qs_s + h * p.qs_h;
  const T *k1 = (const T *)p.k1 + b * p.ks_b + h * p.ks_h;
  const T *k2 = (const T *)p.k2 + b * p.ks_b + h * p.ks_h;
  const T *v = (const T *)p.v + b * p.vs_b + h * p.vs_h;
  const float c = p.scale * kLog2e;

  float a1[D], a2[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    a1[t] = ld(q1 + t) * c;
    a2[t] = ld(q2 + t) * c;
  }
  const int nk = p.causal ? i + 1 : p.S;

  // Pass 1: log2 partition function of each map.
  float m1 = kNegInf, l1 = 0.f, m2 = kNegInf, l2 = 0.f;
  for (int j = 0; j < nk; ++j) {
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int t = 0; t < D; ++t) {
      s1 = fmaf(a1[t], ld(k1 + (int64_t)j * p.ks_s + t), s1);
      s2 = fmaf(a2[t], ld(k2 + (int64_t)j * p.ks_s + t), s2);
    }
    if (s1 > m1) { l1 *= exp2f(m1 - s1); m1 = s1; }
    if (s2 > m2) { l2 *= exp2f(m2 - s2); m2 = s2; }
    l1 += exp2f(s1 - m1);
    l2 += exp2f(s2 - m2);
  }
  const float L1 = m1 + log2f(l1), L2 = m2 + log2f(l2);

  // Pass 2: combined normalised weights times V.
  float o[DV];
#pragma unroll
  for (int t = 0; t < DV; ++t) o[t] = 0.f;
  for (int j = 0; j < nk; ++j) {
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int t = 0; t < D; ++t) {
      s1 = fmaf(a1[t], ld(k1 + (int64_t)j * p.ks_s + t), s1);
      s2 = fmaf(a2[t], ld(k2 + (int64_t)j * p.ks_s + t), s2);
    }
    const float w = exp2f(s1 - L1) - lam * exp2f(s2 - L2);
#pragma unroll
    for (int t = 0; t < DV; ++t) o[t] = fmaf(w, ld(v + (int64_t)j * p.vs_s + t), o[t]);
  }

  float f = 1.f;
  if (p.norm) {
    float ss = 0.f;
#pragma unroll
    for (int t = 0; t < DV; ++t) ss = fmaf(o[t], o[t], ss);
    f = (1.f - p.lambda_init) / sqrtf(ss / DV + p.eps);
  }
  T *out = (T *)p.out + b * p.os_b + (int64_t)i * p.os_s + h * p.os_h;
#pragma unroll
  for (int t = 0; t < DV; ++t) out[t] = (T)(o[t] * f);
}

template <typename T>
static hipError_t launch_typed(const FwdParams &p, int d, int dv, hipStream_t st) {
  dim3 grid((p.S + 63) / 64, p.B * p.H), block(64);
#define DA_CASE(D_, DV_)                                                        \
  if (d == D_ && dv == DV_) {                                                   \
    hipLaunchKernelGGL((fwd_generic_kernel<T, D_, DV_>), grid, block, 0, st, p); \
    return hipGetLastError();                                                   \
  }
  DA_CASE(8, 16)
  DA_CASE(16, 32)
  DA_CASE(32, 64)
  DA_CASE(64, 128)
  DA_CASE(128, 256)
#undef DA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_generic(const FwdParams &p, int dtype, int d, int dv, hipStream_t st) {
  return dtype == 0 ? launch_typed<float>(p, d, dv, st) : launch_typed<bf16>(p, d, dv, st);
}

}  // namespace diffattn
