// Global -> LDS staging of the DIFF V1 forward's key tiles (bf16, d = 64,
// dv = 128): 64 keys of K1, K2 and V per tile, 256 threads.  The loader is
// shared by the fp8-logit forward (which converts V to fp16 on its way into
// LDS) and the backward's dQ kernel (which stages K1, K2 and V as fp16).
#pragma once

#include "common.h"
#include "vrange.h"

namespace diffattn {
namespace v1s {

constexpr int D = 64, DV = 128, BN = 64, NT = 256;
constexpr int KST = D + 8;   // LDS row stride of a K tile, bf16 elements (144 B)
constexpr int VST = DV + 32; // LDS row stride of the V tile, fp16 elements (320 B)

struct Smem {
  bf16 k1[BN * KST];
  bf16 k2[BN * KST];
  f16 v[BN * VST];  // V tile converted to fp16
};

// One thread's share of a tile: two 16-byte chunks of K1 and of K2, four of V.
struct TileRegs {
  u32x4 k1[2], k2[2], v[4];
};

// Raw buffer loads: each (batch, head) slice of K1, K2 and V gets a buffer
// resource whose range ends at the slice's last key row, so rows past the
// sequence end read as zeros without a branch.  Each thread owns fixed rows
// and columns of the tile; its byte offsets are computed once and the tile
// base is added per load.
struct TileLoader {
  __amdgpu_buffer_rsrc_t rk1, rk2, rv;
  uint32_t ko[2], vo[4];   // this thread's byte offsets inside a tile
  uint32_t kstep, vstep;   // bytes per key row

  __device__ __forceinline__ void init(const bf16 *k1, const bf16 *k2, const bf16 *v, int64_t ks, int64_t vs,
                                       int S, int tid) {
    const uint32_t kbytes = (uint32_t)((int64_t)(S - 1) * ks * 2 + D * 2);
    const uint32_t vbytes = (uint32_t)((int64_t)(S - 1) * vs * 2 + DV * 2);
    rk1 = __builtin_amdgcn_make_buffer_rsrc((void *)k1, 0, kbytes, 0x00020000);
    rk2 = __builtin_amdgcn_make_buffer_rsrc((void *)k2, 0, kbytes, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void *)v, 0, vbytes, 0x00020000);
    kstep = (uint32_t)(ks * 2);
    vstep = (uint32_t)(vs * 2);
    const int kr = tid >> 3, vr = tid >> 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) ko[i] = (uint32_t)(kr + 32 * i) * kstep + (tid & 7) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) vo[i] = (uint32_t)(vr + 16 * i) * vstep + (tid & 15) * 16;
  }

  // Half-tile loads into one four-chunk register set: K1 and K2 (two chunks
  // each), or V (four chunks), in the same thread -> (row, column) layout as
  // load.
  __device__ __forceinline__ void load_k12(int kbase, u32x4 (&r)[4]) const {
    const uint32_t kb = (uint32_t)kbase * kstep;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk1, (int)(ko[i] + kb), 0, 0));
      r[2 + i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk2, (int)(ko[i] + kb), 0, 0));
    }
  }

  __device__ __forceinline__ void load_v(int kbase, u32x4 (&r)[4]) const {
    const uint32_t vb = (uint32_t)kbase * vstep;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(vo[i] + vb), 0, 0));
  }

  __device__ __forceinline__ void load(int kbase, bool with_v, TileRegs &r) const {
    const uint32_t kb = (uint32_t)kbase * kstep;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      r.k1[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk1, (int)(ko[i] + kb), 0, 0));
      r.k2[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk2, (int)(ko[i] + kb), 0, 0));
    }
    if (with_v) {
      const uint32_t vb = (uint32_t)kbase * vstep;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(vo[i] + vb), 0, 0));
    }
  }
};

// Register -> LDS half of the staging.  V is converted bf16 -> fp16 times the
// workgroup's power-of-two range shift (vrange.h).
__device__ __forceinline__ void store_tile(Smem &sm, const TileRegs &r, int tid, bool with_v, const VScale &vsc) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + NT * i, row = c >> 3, col = (c & 7) * 8;
    *(u32x4 *)(sm.k1 + row * KST + col) = r.k1[i];
    *(u32x4 *)(sm.k2 + row * KST + col) = r.k2[i];
  }
  if (with_v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + NT * i, row = c >> 4, col = (c & 15) * 8;
      const u32x4 h = bf16x8_to_f16x8_scaled(r.v[i], vsc);
      *(u32x4 *)(sm.v + row * VST + col) = h;
    }
  }
}

}  // namespace v1s
}  // namespace diffattn
