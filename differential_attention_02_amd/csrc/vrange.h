// Range of the fp16 copies of V that the forward kernels' PV products read.
//
// bf16 V converts to fp16 exactly only for magnitudes in [2^-14, 65504]:
// larger values would saturate and smaller ones lose significand bits.  Each
// workgroup therefore converts V 2^k instead, with k chosen from the largest
// |v| among the key rows it reads (a short pass over V first writes the
// largest magnitude of every 256-row chunk of every slice), and scales its
// result by 2^-k.  Out-of-range data get the largest magnitude brought just
// below 2^16 (bf16's largest value below 2^16 is 65280, under fp16's 65504),
// so every value within 2^-30 of it keeps fp16's full 11-bit significand and
// smaller ones contribute below the outputs' bf16 resolution.  The shift is
// exact (a power of two); in-range data (k = 0) take the plain conversion.
#pragma once

#include "common.h"

namespace diffattn {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Shift k for a largest magnitude given as bf16 bits.  No shift while it lies
// in [2^-4, 65280]: nothing saturates and every value within 2^-10 of it
// keeps full fp16 precision (the common case; results then equal the plain
// conversion's).  Otherwise the largest magnitude is brought just below 2^16.
__host__ __device__ inline int v_shift_of_max(unsigned m) {
  const int e = (int)(m >> 7);  // biased exponent
  if (e == 0 || (e >= 123 && e <= 142)) return 0;
  return 142 - e < 126 ? 142 - e : 126;
}

// Shift k (uniform across the wave) from the partial maxima of the first
// nparts row chunks of one slice (written by the range pass, vrange.hip):
// max|v| 2^k < 2^16; k = 0 when every value is zero.
__device__ __forceinline__ int v_shift(const unsigned *part, int nparts) {
  const int lane = __lane_id();
  unsigned m = 0;
  for (int i = lane; i < nparts; i += 64) m = part[i] > m ? part[i] : m;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned t = (unsigned)__shfl_xor((int)m, o);
    m = t > m ? t : m;
  }
  return __builtin_amdgcn_readfirstlane(v_shift_of_max(m));  // the same in every lane (a scalar from here on)
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The multiplier 2^k as the bf16 pairs (2^k, 0) and (0, 2^k); on: k != 0
// (uniform across the workgroup).
struct VScale {
  bf16x2 lo, hi;
  bool on;
  __device__ __forceinline__ explicit VScale(int k) : on(k != 0) {
    const __bf16 s = __builtin_bit_cast(__bf16, (unsigned short)((127 + k) << 7));
    lo = bf16x2{s, (__bf16)0.f};
    hi = bf16x2{(__bf16)0.f, s};
  }
};

// Two bf16 values (one word) times 2^k, to two fp16 values: the bf16 -> float
// step is a bf16 dot product with (2^k, 0) or (0, 2^k), exact (one nonzero
// product).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_mul(uint32_t w, const VScale &sc) {
  const bf16x2 a = __builtin_bit_cast(bf16x2, w);
  const float lo = __builtin_amdgcn_fdot2_f32_bf16(a, sc.lo, 0.f, false);
  const float hi = __builtin_amdgcn_fdot2_f32_bf16(a, sc.hi, 0.f, false);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// Eight bf16 values (four words) to fp16 times 2^k; SCALED = false is the
// plain conversion (k = 0).
template <bool SCALED>
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(const u32x4 &w, const VScale &sc) {
  if constexpr (SCALED)
    return u32x4{bf16x2_to_f16x2_mul(w[0], sc), bf16x2_to_f16x2_mul(w[1], sc), bf16x2_to_f16x2_mul(w[2], sc),
                 bf16x2_to_f16x2_mul(w[3], sc)};
  return u32x4{bf16x2_to_f16x2(w[0]), bf16x2_to_f16x2(w[1]), bf16x2_to_f16x2(w[2]), bf16x2_to_f16x2(w[3])};
}

// Either conversion, chosen per call by the (uniform) shift.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8_scaled(const u32x4 &w, const VScale &sc) {
  return sc.on ? bf16x8_to_f16x8<true>(w, sc) : bf16x8_to_f16x8<false>(w, sc);
}

}  // namespace diffattn
