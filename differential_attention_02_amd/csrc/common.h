// Device helpers shared by the gfx950 kernels of libdiffattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

#define DA_LDS __attribute__((address_space(3)))

// v_exp_f32: 2^x (hardware transcendental).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// D = A * B + C on a 32x32x16 bf16 tile.  Lane l holds A[l % 32][8 (l / 32) + i]
// and B[8 (l / 32) + i][l % 32], i = 0..7; D register r of lane l is row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// Same tile shape and lane layout with fp16 operands.
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two bf16 values (one 32-bit word) to two fp16 values.  bf16 carries 8
// significant bits, which fp16 holds exactly for magnitudes in [2^-14, 65504];
// smaller magnitudes lose bits below 2^-24 and larger ones saturate at 65504
// (round toward zero).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16),
                                                                  __uint_as_float(w & 0xffff0000u)));
}

// LDS transpose read of 4 x 16-bit values.  Within each group of 16 lanes,
// output lane i takes, for slot e = 0..3, element i % 4 of the 8-byte block
// addressed by source lane 4 e + i / 4.  Pointing source lane j at row
// (r0 + j / 4), column (c0 + 4 (j % 4)) of a row-major 16-bit matrix makes
// lane i receive column c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ f16x4 lds_read_tr16(const f16 *p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(p));
  return __builtin_bit_cast(f16x4, v);
}

// Value of x held by lane l ^ 32.
__device__ __forceinline__ float other_half(float x) {
  const int lane = __lane_id();
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Reductions over aligned groups of 16 lanes (one row of 128 channels at
// 8 channels per lane).
constexpr int kRowLanes = 16;

__device__ __forceinline__ float row_sum(float x) {
  for (int o = kRowLanes / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float row_max(float x) {
  for (int o = kRowLanes / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Eight bf16 values (one 16-byte load) to float32.
__device__ __forceinline__ void bf16x8_f32(const u32x4 &r, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(r[i] << 16);
    f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}

// Eight float32 values from a 16-byte aligned address.
__device__ __forceinline__ void load_f32x8(const float *p, float *f) {
  const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = a[i];
    f[4 + i] = b[i];
  }
}

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }  // round to nearest even

// lambda = exp(<lq1, lk1>) - exp(<lq2, lk2>) + lambda_init, or the fixed value
// when the vectors are absent.  Computed by every wave (same order, same value).
__device__ __forceinline__ float wave_lambda(const float *lq1, const float *lk1, const float *lq2,
                                             const float *lk2, int dim, float fixed, float init) {
  if (lq1 == nullptr) return fixed;
  const int lane = __lane_id();
  float a = 0.f, b = 0.f;
  for (int i = lane; i < dim; i += 64) {
    a = fmaf(lq1[i], lk1[i], a);
    b = fmaf(lq2[i], lk2[i], b);
  }
  a = wave_sum(a);
  b = wave_sum(b);
  return expf(a) - expf(b) + init;
}

}  // namespace diffattn
