// Passes over V for the forward kernels' fp16 operands (vrange.h):
//   vrange_kernel: the largest |v| (as the bits of a bf16 magnitude) of every
//     256-row chunk of every (batch, head) slice; the kernels that convert V
//     themselves pick their shift from these;
//   vconv_kernel: a converted fp16 copy of V with one power-of-two shift per
//     256-row chunk, for the one-pass forward.
// Each reads V once; no atomics, so nothing needs clearing.
#include "kernels.h"
#include "vrange.h"

namespace diffattn {
namespace {

constexpr int NT = 256;

template <int C>
__global__ __launch_bounds__(NT) void vrange_kernel(VRangeParams p) {
  constexpr int CPR = C / 8;  // 16-byte chunks per row
  __shared__ unsigned red[NT / 64];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, hd = bh % p.H;
  const int r0 = chunk * kVRangeRows;
  const int n = min(kVRangeRows, p.S - r0);
  const bf16 *base = (const bf16 *)p.v + b * p.vs_b + (int64_t)r0 * p.vs_s + hd * p.vs_h;
  u16x2 acc = {0, 0};
#pragma unroll 8
  for (int i = threadIdx.x; i < n * CPR; i += NT) {
    const int row = i / CPR, col = (i % CPR) * 8;
    const u32x4 w = *(const u32x4 *)(base + (int64_t)row * p.vs_s + col);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, w[k] & 0x7fff7fffu));
  }
  unsigned m = acc[0] > acc[1] ? acc[0] : acc[1];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned t = (unsigned)__shfl_xor((int)m, o);
    m = t > m ? t : m;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned mm = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) mm = red[w] > mm ? red[w] : mm;
    p.part[(int64_t)bh * vrange_chunks(p.S) + chunk] = mm;
  }
}

// V to a contiguous fp16 copy [B * H, S, 128], each 256-row chunk scaled by
// its own power of two 2^k (k per chunk into kexp[B * H][chunks], chosen as
// in v_shift from the chunk's own largest magnitude).  One workgroup per
// chunk holds the chunk in registers (64 KB: 16 words per thread), so V is
// read once.
__global__ __launch_bounds__(NT) void vconv_kernel(VConvParams p) {
  constexpr int C = 128, CPR = C / 8, PER = kVRangeRows * CPR / NT;  // 16-byte chunks per thread
  __shared__ unsigned red[NT / 64];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, hd = bh % p.H;
  const int r0 = chunk * kVRangeRows;
  const int n = min(kVRangeRows, p.S - r0);
  const bf16 *base = (const bf16 *)p.v + b * p.vs_b + (int64_t)r0 * p.vs_s + hd * p.vs_h;
  u32x4 w[PER];
  u16x2 acc = {0, 0};
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + NT * i, row = c / CPR, col = (c % CPR) * 8;
    w[i] = row < n ? *(const u32x4 *)(base + (int64_t)row * p.vs_s + col) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, w[i][k] & 0x7fff7fffu));
  }
  unsigned m = acc[0] > acc[1] ? acc[0] : acc[1];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned t = (unsigned)__shfl_xor((int)m, o);
    m = t > m ? t : m;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  unsigned mm = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) mm = red[i] > mm ? red[i] : mm;
  const int k = v_shift_of_max(mm);
  if (threadIdx.x == 0) p.kexp[(int64_t)bh * vrange_chunks(p.S) + chunk] = k;
  f16 *dst = p.v16 + ((int64_t)bh * p.S + r0) * C;
  const VScale sc(k);
  if (k != 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + NT * i, row = c / CPR, col = (c % CPR) * 8;
      if (row < n) *(u32x4 *)(dst + row * C + col) = bf16x8_to_f16x8<true>(w[i], sc);
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + NT * i, row = c / CPR, col = (c % CPR) * 8;
      if (row < n) *(u32x4 *)(dst + row * C + col) = bf16x8_to_f16x8<false>(w[i], sc);
    }
  }
}

}  // namespace

hipError_t launch_vconv(const VConvParams &p, hipStream_t st) {
  dim3 grid(vrange_chunks(p.S), p.B * p.H), block(NT);
  hipLaunchKernelGGL(vconv_kernel, grid, block, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_vrange(const VRangeParams &p, int channels, hipStream_t st) {
  dim3 grid(vrange_chunks(p.S), p.B * p.H), block(NT);
  if (channels == 128)
    hipLaunchKernelGGL(vrange_kernel<128>, grid, block, 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace diffattn
