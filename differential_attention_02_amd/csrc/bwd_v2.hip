// Backward of the DIFF V2 prefill forward on gfx950 (bf16 storage, D = 128).
// The pages print no gradient formulas; these are the chain rule of the
// forward (tistory page on DIFF V2, section "DIFF V2 innovations" items 1, 2
// and 5; section "GQA compatibility").  Per batch entry and pair (even head
// e = 2p, odd head o = 2p + 1, both reading KV head j), sigma = sigmoid(lam)
// per token:
//   out = A_e - sigma A_o,  A_t = P_t V,  P_t = softmax(s Q_t K^T)
//   dlam = -sigma (1 - sigma) g . A_o                  (g = dout, per row)
//   dV = (P_e - sigma P_o)^T g                         (one product per pair)
//   dP = g V^T                                         (shared by both heads)
//   E_t = g . A_t  (each head's own output, saved by the forward in float32)
//   dS_e = P_e (dP - E_e),  dS_o = -sigma P_o (dP - E_o)
//   dQ_t = s dS_t K,  dK = s sum_t dS_t^T Q_t (over every head reading j)
//
// Kernels, in launch order:
//   v2b_pre    per (batch, pair, token) row: |g| and the largest |Q_e|,
//              |Q_o| (and |K|, |V| of the row's key when the pair is the
//              first on its KV head);
//   v2b_scales one workgroup per (batch, KV head): power-of-two scales that
//              keep the fp16 operands below 2^13: g by the largest row norm
//              of the pairs on the head, dS by the bound
//              |dS| <= 2 max|g| max|V| (|A_t| <= max|V|), W = P_e - sigma P_o
//              (|W| <= 1) by a fixed 2^12;
//   v2b_gconv  per row: dlam from the float32 g and the saved A_o;
//              g' = fp16(g 2^sg) and E_t = g' . A_t from that same
//              fp16 g' and A_t accumulated with head t's own weights (so
//              dS = P (dP - E) stays self-consistent where one key dominates a
//              row and dP - E cancels); also Q_e | Q_o in fp16 for the
//              key-outer kernel's staging;
//   v2b_dq     query-outer: 128 queries of one (batch, pair) per workgroup,
//              64-key tiles; dS and dQ of both heads in registers;
//   v2b_dkdv   key-outer: 128 keys of one (batch, KV head) per workgroup,
//              every pair of the head, 64-query chunks double-buffered in
//              LDS; dV and dK in registers.  No atomics: deterministic.
// Matrix-core operands are fp16 with float32 accumulation; Q, K and V enter
// fp16 times powers of two 2^kq, 2^kk, 2^kv chosen per (batch, KV head) from
// their largest magnitudes (v2b_pre, v2b_scales; vrange.h), so any finite bf16
// inputs convert without saturating or losing precision; results are unscaled
// exactly.
#include <cstddef>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "vrange.h"

namespace diffattn {
namespace {

constexpr int D = 128, NT = 256;
constexpr int QST = D + 8;   // LDS row stride (fp16) of Q / K tiles (272 B)
constexpr int GST = D + 32;  // LDS row stride (fp16) of g / V tiles (320 B, transpose-read friendly)

struct Ws2 {
  f16 *gh;               // [B, P, S, D]  g' = g 2^sg
  f16 *qh;               // [B, P, S, 2 D] Q_e (channels 0..127) | Q_o (128..255)
  float *ee, *eo, *gn;   // [B, P, S]  E_e, E_o (unscaled), |g|
  float *vn;             // [B, Hkv, S]  |V| rows
  float *qm;             // [B, P, S]  largest |Q_e|, |Q_o| of the row
  float *kvm;            // [B, Hkv, S][2]  largest |K|, |V| of the row
  float *scales;         // [B * Hkv][8]: sg, kappa, omega, kq, kk, kv, unused x2 (exponents of 2)
};

__host__ __device__ inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Ws2 carve2(void *base, int B, int S, int P, int Hkv) {
  char *c = static_cast<char *>(base);
  const size_t rows = (size_t)B * P * S;
  Ws2 w;
  w.gh = (f16 *)c; c += al256(rows * D * 2);
  w.qh = (f16 *)c; c += al256(rows * 2 * D * 2);
  w.ee = (float *)c; c += al256(rows * 4);
  w.eo = (float *)c; c += al256(rows * 4);
  w.gn = (float *)c; c += al256(rows * 4);
  w.vn = (float *)c; c += al256((size_t)B * Hkv * S * 4);
  w.qm = (float *)c; c += al256(rows * 4);
  w.kvm = (float *)c; c += al256((size_t)B * Hkv * S * 8);
  w.scales = (float *)c; c += al256((size_t)B * Hkv * 32);
  return w;
}

__host__ __device__ inline size_t ws2_bytes(int B, int S, int P, int Hkv) {
  const size_t rows = (size_t)B * P * S;
  return al256(rows * D * 2) + al256(rows * 2 * D * 2) + 3 * al256(rows * 4) + al256((size_t)B * Hkv * S * 4) +
         al256(rows * 4) + al256((size_t)B * Hkv * S * 8) + al256((size_t)B * Hkv * 32);
}

__device__ __forceinline__ float sigmoid_of(const V2BwdParams &p, int b, int s, int pr) {
  const float lam = p.lam[b * p.ls_b + (int64_t)s * p.ls_s + pr * p.ls_p];
  return 1.f / (1.f + expf(-lam));
}

// ---------------------------------------------------------------------------
// Row kernels (v2b_pre, v2b_gconv): 16 lanes per (b, pair, s) row, 8 channels
// per lane (16-byte bf16 and 32-byte float32 accesses), four rows per wave.
constexpr int RPB = NT / kRowLanes;  // rows per workgroup

__global__ __launch_bounds__(NT) void v2b_pre_kernel(V2BwdParams p, Ws2 w) {
  const int part = threadIdx.x & (kRowLanes - 1);
  const int P = p.Hq / 2;
  const int64_t row = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 4);  // over [B, P, S]
  if (row >= (int64_t)p.B * P * p.S) return;  // whole 16-lane groups leave together
  const int s = row % p.S;
  const int bp = row / p.S, b = bp / P, pr = bp % P;
  const int c = part * 8;
  float g[8], qe[8], qo[8];
  bf16x8_f32(*(const u32x4 *)((const bf16 *)p.dout + b * p.ds_b + (int64_t)s * p.ds_s + pr * p.ds_h + c), g);
  // Largest magnitudes of the row's Q_e, Q_o (and, once per KV head, K and V):
  // their fp16 copies are scaled by powers of two chosen from these (vrange.h).
  const bf16 *qp = (const bf16 *)p.q + b * p.qs_b + (int64_t)s * p.qs_s + 2 * pr * p.qs_h + c;
  bf16x8_f32(*(const u32x4 *)qp, qe);
  bf16x8_f32(*(const u32x4 *)(qp + p.qs_h), qo);
  float gg = 0.f, qmx = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    gg = fmaf(g[i], g[i], gg);
    qmx = fmaxf(qmx, fmaxf(fabsf(qe[i]), fabsf(qo[i])));
  }
  gg = row_sum(gg);
  qmx = row_max(qmx);
  if (part == 0) {
    w.gn[row] = sqrtf(gg);
    w.qm[row] = qmx;
  }
  const int ppk = p.Hq / p.Hkv / 2, j = pr / ppk;
  if (pr % ppk == 0) {  // uniform over the row's 16 lanes
    float v[8], k[8];
    bf16x8_f32(*(const u32x4 *)((const bf16 *)p.v + b * p.kvs_b + (int64_t)s * p.kvs_s + j * p.kvs_h + c), v);
    bf16x8_f32(*(const u32x4 *)((const bf16 *)p.k + b * p.kvs_b + (int64_t)s * p.kvs_s + j * p.kvs_h + c), k);
    float vv = 0.f, vmx = 0.f, kmx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      vv = fmaf(v[i], v[i], vv);
      vmx = fmaxf(vmx, fabsf(v[i]));
      kmx = fmaxf(kmx, fabsf(k[i]));
    }
    vv = row_sum(vv);
    vmx = row_max(vmx);
    kmx = row_max(kmx);
    const int64_t kr_row = ((int64_t)b * p.Hkv + j) * p.S + s;
    if (part == 0) {
      w.vn[kr_row] = sqrtf(vv);
      *(float2 *)(w.kvm + kr_row * 2) = make_float2(kmx, vmx);
    }
  }
}

// ---------------------------------------------------------------------------
// v2b_scales: one workgroup of NTS threads per (b, KV head j) (many loads in
// flight: the pass is latency-bound).
constexpr int NTS = 1024, NWS = NTS / 64;

__global__ __launch_bounds__(NTS) void v2b_scales_kernel(V2BwdParams p, Ws2 w) {
  __shared__ float red[5][NWS];
  const int bj = blockIdx.x, b = bj / p.Hkv, j = bj % p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = p.Hq / 2, ppk = p.Hq / p.Hkv / 2;  // pairs per KV head
  float gm = 0.f, qm = 0.f;
  for (int pp = 0; pp < ppk; ++pp) {
    const int64_t base = ((int64_t)b * P + j * ppk + pp) * p.S;
    for (int s = tid; s < p.S; s += NTS) {
      gm = fmaxf(gm, w.gn[base + s]);
      qm = fmaxf(qm, w.qm[base + s]);
    }
  }
  float vm = 0.f, km = 0.f, vx = 0.f;
  const float *vn = w.vn + (int64_t)bj * p.S;
  const float *kvm = w.kvm + (int64_t)bj * p.S * 2;
  for (int s = tid; s < p.S; s += NTS) {
    vm = fmaxf(vm, vn[s]);
    km = fmaxf(km, kvm[2 * s]);
    vx = fmaxf(vx, kvm[2 * s + 1]);
  }
  for (int o = 32; o > 0; o >>= 1) {
    gm = fmaxf(gm, __shfl_xor(gm, o));
    vm = fmaxf(vm, __shfl_xor(vm, o));
    qm = fmaxf(qm, __shfl_xor(qm, o));
    km = fmaxf(km, __shfl_xor(km, o));
    vx = fmaxf(vx, __shfl_xor(vx, o));
  }
  if (lane == 0) {
    red[0][wave] = gm;
    red[1][wave] = vm;
    red[2][wave] = qm;
    red[3][wave] = km;
    red[4][wave] = vx;
  }
  __syncthreads();
  if (tid == 0) {
    float mx[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      mx[i] = red[i][0];
#pragma unroll
      for (int k = 1; k < NWS; ++k) mx[i] = fmaxf(mx[i], red[i][k]);
    }
    gm = mx[0];
    vm = mx[1];
    const float kq = (float)v_shift_of_max(__float_as_uint(mx[2]) >> 16);
    const float kk = (float)v_shift_of_max(__float_as_uint(mx[3]) >> 16);
    const float kv = (float)v_shift_of_max(__float_as_uint(mx[4]) >> 16);
    const float sg = gm > 0.f ? fminf(fmaxf(floorf(13.f - log2f(gm)), -60.f), 60.f) : 0.f;
    const float x = 2.f * gm * vm;  // bound on |dS| before scaling by 2^sg
    // dP' = g' V' carries 2^(sg + kv): dS is scaled by 2^kappa on top of it.
    const float kap = x > 0.f ? fminf(fmaxf(floorf(13.f - log2f(x) - sg), -60.f), 60.f) - kv : 0.f;
    w.scales[bj * 8 + 0] = sg;
    w.scales[bj * 8 + 1] = kap;
    w.scales[bj * 8 + 2] = 12.f;
    w.scales[bj * 8 + 3] = kq;
    w.scales[bj * 8 + 4] = kk;
    w.scales[bj * 8 + 5] = kv;
  }
}

// ---------------------------------------------------------------------------
// v2b_gconv: per (b, pair, s) row, dlam, g' = fp16(g 2^sg) and E_e = g' . A_e,
// E_o = g' . A_o, stored unscaled; also the row's Q_e | Q_o in fp16.
__global__ __launch_bounds__(NT) void v2b_gconv_kernel(V2BwdParams p, Ws2 w) {
  const int part = threadIdx.x & (kRowLanes - 1);
  const int P = p.Hq / 2, ppk = p.Hq / p.Hkv / 2;
  const int64_t row = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 4);
  if (row >= (int64_t)p.B * P * p.S) return;  // whole 16-lane groups leave together
  const int s = row % p.S;
  const int bp = row / p.S, b = bp / P, pr = bp % P;
  const int bj = b * p.Hkv + pr / ppk;
  const int c = part * 8;
  const float sg = w.scales[bj * 8 + 0], f = fast_exp2(sg);
  float g[8], ae[8], ao[8];
  bf16x8_f32(*(const u32x4 *)((const bf16 *)p.dout + b * p.ds_b + (int64_t)s * p.ds_s + pr * p.ds_h + c), g);
  const int64_t srow = (((int64_t)b * p.S + s) * P + pr) * D;
  load_f32x8(p.a_even + srow + c, ae);
  load_f32x8(p.a_odd + srow + c, ao);
  // dlam = -sigma (1 - sigma) g . A_o from the float32 g (the fp16 g' would
  // cost dlam most of its precision where the sum cancels).
  float ga = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ga = fmaf(g[i], ao[i], ga);
  ga = row_sum(ga);
  f16x8 gh;
#pragma unroll
  for (int i = 0; i < 8; ++i) gh[i] = (f16)(g[i] * f);
  *(f16x8 *)(w.gh + row * D + c) = gh;
  float ee = 0.f, eo = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float gi = (float)gh[i];
    ee = fmaf(gi, ae[i], ee);
    eo = fmaf(gi, ao[i], eo);
  }
  ee = row_sum(ee);
  eo = row_sum(eo);
  // The row's Q_e | Q_o to fp16 times 2^kq for the key-outer kernel's
  // staging ([B, P, S, 2 D]), eight channels of each head per lane.
  const VScale sq((int)w.scales[bj * 8 + 3]);
  const bf16 *qp = (const bf16 *)p.q + b * p.qs_b + (int64_t)s * p.qs_s + 2 * pr * p.qs_h + c;
  *(u32x4 *)(w.qh + row * (2 * D) + c) = bf16x8_to_f16x8_scaled(*(const u32x4 *)qp, sq);
  *(u32x4 *)(w.qh + row * (2 * D) + D + c) = bf16x8_to_f16x8_scaled(*(const u32x4 *)(qp + p.qs_h), sq);
  if (part == 0) {
    const float un = fast_exp2(-sg);
    w.ee[row] = ee * un;
    w.eo[row] = eo * un;
    const float sig = sigmoid_of(p, b, s, pr);
    p.dlam[((int64_t)b * p.S + s) * P + pr] = -sig * (1.f - sig) * ga;
  }
}

// Permutation of rows 0..31 used for the A operand of score-like products so
// that a lane's 16 result registers are rows 8 h + 0..7 and 16 + 8 h + 0..7.
__device__ __forceinline__ int row_perm(int i) { return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1); }
__device__ __forceinline__ int row_of_reg(int r, int h) { return ((r & 8) << 1) + 8 * h + (r & 7); }

// Eight bf16 values to fp16 times 2^k (the fp16 copies' range shift).
__device__ __forceinline__ f16x8 to_f16x8(const u32x4 &raw, const VScale &sc) {
  return __builtin_bit_cast(f16x8, bf16x8_to_f16x8_scaled(raw, sc));
}

__device__ __forceinline__ f16x8 pack8h(const float *v) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const f32x2 x = {v[i], v[i + 1]};
    const f16x2 y = __builtin_convertvector(x, f16x2);
    r[i] = y[0];
    r[i + 1] = y[1];
  }
  return r;
}

// A operand (rows = the 32 matrix columns c0..c0+31 of a row-major fp16 tile,
// k = 16 consecutive tile rows starting at r0) through transpose reads:
// lane l receives column c0 + l % 32 of rows r0 + 8 (l / 32) + 0..7.
__device__ __forceinline__ f16x8 tr_operand(const f16 *tile, int stride, int r0, int c0, int lane) {
  const int h = lane >> 5, j = lane & 15, half16 = (lane >> 4) & 1;
  const f16 *ptr = tile + (r0 + 8 * h + (j >> 2)) * stride + c0 + 16 * half16 + 4 * (j & 3);
  const f16x4 lo = lds_read_tr16(ptr);
  const f16x4 hi = lds_read_tr16(ptr + 4 * stride);
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------------------
// v2b_dq: query-outer.  Workgroup = 128 queries of one (b, pair); wave w owns
// queries q0 + 32 w + 0..31 (lane l % 32).
constexpr int QB = 128, KT = 64;

struct SmemQ {
  f16 k[KT * QST];
  f16 v[KT * GST];
};

// One thread's share of a K/V tile in flight: 16 bytes of K and of V for four
// (key, column-chunk) slots.
struct KVRegs {
  u32x4 k[KT * (D / 8) / NT], v[KT * (D / 8) / NT];
};

// Bounded buffer loads of a (batch, KV head) slice's K and V rows: the
// resources end at the slice's last key row, so keys past the end read as
// zeros without a branch; byte offsets are 32-bit inside the slice.
struct KVLoader {
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t off[KT * (D / 8) / NT];  // this thread's byte offsets inside a tile
  uint32_t step;                    // bytes per key row

  __device__ __forceinline__ void init(const bf16 *kg, const bf16 *vg, int64_t kvs, int S, int tid) {
    const uint32_t bytes = (uint32_t)((int64_t)(S - 1) * kvs * 2 + D * 2);
    rk = __builtin_amdgcn_make_buffer_rsrc((void *)kg, 0, bytes, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void *)vg, 0, bytes, 0x00020000);
    step = (uint32_t)(kvs * 2);
#pragma unroll
    for (int i = 0; i < KT * (D / 8) / NT; ++i) {
      const int idx = tid + i * NT;
      off[i] = (uint32_t)(idx >> 4) * step + (idx & 15) * 16;
    }
  }

  __device__ __forceinline__ void load(KVRegs &r, int kbase) const {
    const uint32_t kb = (uint32_t)kbase * step;
#pragma unroll
    for (int i = 0; i < KT * (D / 8) / NT; ++i) {
      r.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(off[i] + kb), 0, 0));
      r.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(off[i] + kb), 0, 0));
    }
  }
};

__device__ __forceinline__ void store_kv(SmemQ &sm, const KVRegs &r, int tid, const VScale &sck,
                                         const VScale &scv) {
#pragma unroll
  for (int i = 0; i < KT * (D / 8) / NT; ++i) {
    const int idx = tid + i * NT, row = idx >> 4, col = (idx & 15) * 8;
    *(f16x8 *)(sm.k + row * QST + col) = to_f16x8(r.k[i], sck);
    *(f16x8 *)(sm.v + row * GST + col) = to_f16x8(r.v[i], scv);
  }
}

__global__ __launch_bounds__(NT, 1) void v2b_dq_kernel(V2BwdParams p, Ws2 w) {
  __shared__ SmemQ smb[3];  // tile kt in buffer kt % 3 (the pipeline reads two tiles while a third is staged)
  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = p.Hq / 2, ppk = p.Hq / p.Hkv / 2;
  const int BP = p.B * P;
  const int n_qt = (p.S + QB - 1) / QB;
  const int bp = blockIdx.x % BP;
  const int qt = p.causal ? n_qt - 1 - blockIdx.x / BP : blockIdx.x / BP;
  const int b = bp / P, pr = bp % P, j = pr / ppk, bj = b * p.Hkv + j;
  const int S = p.S;
  const bool causal = p.causal != 0;
  const int q0 = qt * QB, qw = q0 + wave * 32, my_q = qw + ln;
  const float sg = w.scales[bj * 8 + 0], kap = w.scales[bj * 8 + 1];
  const float kq = w.scales[bj * 8 + 3], kk = w.scales[bj * 8 + 4], kv = w.scales[bj * 8 + 5];
  const VScale scq((int)kq), sck((int)kk), scv((int)kv);
  // fp16 Q, K, V are Q 2^kq, K 2^kk, V 2^kv: S' = S 2^(kq + kk), dP' = dP 2^(sg + kv).
  const float c = p.scale * kLog2e * fast_exp2(-(kq + kk));
  const int64_t rowb = (int64_t)bp * S;  // row base in [B, P, S]
  const bool qok = my_q < S;

  // B operands: Q_e, Q_o (S^T = K Q^T) and g' (dP'^T = V g'^T), fp16.
  f16x8 qe[D / 16], qo[D / 16], gf[D / 16];
  {
    const bf16 *qp = (const bf16 *)p.q + b * p.qs_b + (int64_t)my_q * p.qs_s + 2 * pr * p.qs_h + 8 * h;
    const f16 *gp = w.gh + (rowb + my_q) * D + 8 * h;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qe[kc] = qok ? to_f16x8(*(const u32x4 *)(qp + kc * 16), scq) : f16x8{};
      qo[kc] = qok ? to_f16x8(*(const u32x4 *)(qp + p.qs_h + kc * 16), scq) : f16x8{};
      gf[kc] = qok ? *(const f16x8 *)(gp + kc * 16) : f16x8{};
    }
  }
  const int64_t lr = ((int64_t)b * p.Hq + 2 * pr) * S + my_q;
  // Row terms folded as in the key-outer kernel (store_chunk2): the score
  // loop forms P_e 2^kappa, sigma P_o 2^kappa and both dS terms directly.
  const float sig = qok ? sigmoid_of(p, b, my_q, pr) : 0.f;
  const float Le = qok ? fmaf(p.lse[lr], kLog2e, -kap) : __builtin_inff();
  const float Lo = qok ? fmaf(p.lse[lr + S], kLog2e, -(kap + log2f(sig))) : __builtin_inff();
  const float fE = fast_exp2(sg + kv);
  const float ee = qok ? w.ee[rowb + my_q] * fE : 0.f;
  const float eo = qok ? w.eo[rowb + my_q] * fE : 0.f;
  // Last key this query sees (the masks as one threshold per block).
  const int key_lim = causal ? min(my_q, S - 1) : S - 1;

  const int kend = causal ? min(S, q0 + QB) : S;
  const int n_kt = (kend + KT - 1) / KT;
  const int krow = row_perm(ln);
  const int q_last = qw + 31;
  const bf16 *kg = (const bf16 *)p.k + b * p.kvs_b + j * p.kvs_h;
  const bf16 *vg = (const bf16 *)p.v + b * p.kvs_b + j * p.kvs_h;

  f32x16 dqe[D / 32], dqo[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dqe[dt] = dqo[dt] = f32x16{};
  KVLoader ld;
  ld.init(kg, vg, p.kvs_s, S, tid);
  KVRegs nx;
  ld.load(nx, 0);
  store_kv(smb[0], nx, tid, sck, scv);
  __syncthreads();
  // One key tile; MASKED applies the causal and key-range masks, which only
  // the tiles from the query tile's start on (causal) and a partial last tile
  // need: two loops, so the interior one carries no mask arithmetic.
  auto tile = [&](auto masked, int kt) {
    constexpr bool MASKED = decltype(masked)::value;
    const SmemQ &sm = smb[kt % 3];
    if (kt + 1 < n_kt) ld.load(nx, (kt + 1) * KT);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int sb = kt * KT + sub * 32;
      if (sb >= S || (causal && sb > q_last)) continue;
      f32x16 s_e = {}, s_o = {}, dp = {};
      const f16 *ka = sm.k + (sub * 32 + krow) * QST + 8 * h;
      const f16 *va = sm.v + (sub * 32 + krow) * GST + 8 * h;
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        const f16x8 a = *(const f16x8 *)(ka + kc * 16);
        s_e = mfma32(a, qe[kc], s_e);
        s_o = mfma32(a, qo[kc], s_o);
        dp = mfma32(*(const f16x8 *)(va + kc * 16), gf[kc], dp);
      }
      float dse[16], dso[16];
      const int lim = key_lim - sb;  // key sb + o is masked iff o > lim
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // The mask selects the exponent (-inf), not the exponential (a select
        // of the exponential was compiled into branches).
        const bool dead = MASKED && row_of_reg(r, h) > lim;
        const float pe = fast_exp2(dead ? -__builtin_inff() : fmaf(s_e[r], c, -Le));  // P_e 2^kappa
        const float po = fast_exp2(dead ? -__builtin_inff() : fmaf(s_o[r], c, -Lo));  // sigma P_o 2^kappa
        dse[r] = pe * (dp[r] - ee);
        dso[r] = po * (eo - dp[r]);
      }
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        const f16x8 be = pack8h(dse + 8 * kc2), bo = pack8h(dso + 8 * kc2);
        const int r0 = sub * 32 + kc2 * 16;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const f16x8 a = tr_operand(sm.k, QST, r0, dt * 32, lane);
          dqe[dt] = mfma32(a, be, dqe[dt]);
          dqo[dt] = mfma32(a, bo, dqo[dt]);
        }
      }
    }
    if (kt + 1 < n_kt) store_kv(smb[(kt + 1) % 3], nx, tid, sck, scv);
    __syncthreads();
  };
  const int n_full = min(causal ? q0 / KT : n_kt, S / KT);  // tiles no query of the tile needs masked

  // The unmasked tiles run as a software pipeline over their 32-key
  // sub-tiles.  Step j, in two halves: the score and dP products of sub-tile
  // j beside the dS of sub-tile j - 1 (from its carried exponentials and dP),
  // then the dQ products of j - 1 beside the exponentials of j; one matrix
  // instruction and a share of the vector work at a time behind scheduling
  // fences (the single wave on each SIMD issues in order, so that order is
  // what overlaps the two units).  LDS operands are read two instructions
  // ahead from per-step base addresses.  Staging: the even step 2m stores the
  // K half of tile m + 1, the odd step its V half (then a barrier); each then
  // loads the same half of tile m + 2.  Tile m is complete from the end of
  // step 2m - 1 and last read in step 2m + 2.
  const int J = 2 * n_full;
  if (J > 0) {
    typedef DA_LDS const char lchar;
    const int jj = lane & 15, half16 = (lane >> 4) & 1;
    const uint32_t laK = (krow * QST + 8 * h) * 2, laV = (krow * GST + 8 * h) * 2;
    const uint32_t lcK = ((8 * h + (jj >> 2)) * QST + 16 * half16 + 4 * (jj & 3)) * 2;
    constexpr uint32_t OK = offsetof(SmemQ, k), OV = offsetof(SmemQ, v);
    // Base address of buffer `buf` plus a lane offset, opaque to the compiler
    // so that it keeps the constant parts in the instructions' offsets.
    auto lptr = [&](int buf, uint32_t lane_off) -> lchar * {
      lchar *q = (lchar *)(smb + buf) + lane_off;
      asm volatile("" : "+v"(q));
      return q;
    };
    auto tr8 = [&](lchar *q, uint32_t off) -> f16x8 {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(q + off));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(q + off + 8 * QST));
      const f16x4 a = __builtin_bit_cast(f16x4, lo), b = __builtin_bit_cast(f16x4, hi);
      return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    };
    // Staging halves: K (part 0) and V (part 1) rows of a tile.
    auto load_part = [&](int t, int part, u32x4 *r) {
      const uint32_t tb = (uint32_t)(t * KT) * ld.step;
#pragma unroll
      for (int i = 0; i < KT * (D / 8) / NT; ++i)
        r[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(part == 0 ? ld.rk : ld.rv, (int)(ld.off[i] + tb), 0, 0));
    };
    auto store_part = [&](int t, int part, const u32x4 *r) {
      SmemQ &sm = smb[t % 3];
#pragma unroll
      for (int i = 0; i < KT * (D / 8) / NT; ++i) {
        const int idx = tid + i * NT, row = idx >> 4, col = (idx & 15) * 8;
        if (part == 0) *(f16x8 *)(sm.k + row * QST + col) = to_f16x8(r[i], sck);
        else *(f16x8 *)(sm.v + row * GST + col) = to_f16x8(r[i], scv);
      }
    };
    u32x4 hreg[2][KT * (D / 8) / NT];
    if (1 < n_kt) {
      load_part(1, 0, hreg[0]);
      load_part(1, 1, hreg[1]);
    }
    // Exponentials and dP of a sub-tile, carried to the next step (two sets:
    // step j writes set j % 2 and reads the other).
    struct Carry {
      float pe[16], po[16];  // P_e 2^kappa, sigma P_o 2^kappa
      f32x16 dp;
    };
    Carry cr[2];
    f16x8 be[2], bo[2];  // dS operands of the previous sub-tile

    auto step = [&](auto has_prev, auto has_cur, auto parity, int j, const Carry &prv, Carry &cur) {
      constexpr bool HP = decltype(has_prev)::value;  // sub-tile j - 1 exists
      constexpr bool HJ = decltype(has_cur)::value;   // sub-tile j exists
      constexpr int SUB = decltype(parity)::value;    // j % 2
      constexpr int SUBP = 1 - SUB;
      const int t = j >> 1;
      lchar *pK = nullptr, *pV = nullptr, *pC = nullptr;
      if constexpr (HJ) {
        pK = lptr(t % 3, laK);
        pV = lptr(t % 3, laV);
      }
      if constexpr (HP) pC = lptr(((j - 1) >> 1) % 3, lcK);
      // Operand i of the score (i < 8: K columns 16 i) and dP (i >= 8: V
      // columns 16 (i - 8)) products; products m = 0..23: (K_i, head e),
      // (K_i, head o) for i < 8, then (V_(m - 16)).
      auto fa = [&](int i) -> f16x8 {
        if (i < 8) return *(const DA_LDS f16x8 *)(pK + OK + (SUB * 32 * QST + i * 16) * 2);
        return *(const DA_LDS f16x8 *)(pV + OV + (SUB * 32 * GST + (i - 8) * 16) * 2);
      };
      // Operand i (0..7) of the dQ products of sub-tile j - 1: K^T columns
      // 32 (i % 4), rows 16 (i / 4).
      auto fc = [&](int i) -> f16x8 { return tr8(pC, OK + ((SUBP * 32 + (i >> 2) * 16) * QST + (i & 3) * 32) * 2); };
      f16x8 oa[16], oc[8];
      f32x16 se = {}, so = {};
      if constexpr (HJ) {
        oa[0] = fa(0);
        oa[1] = fa(1);
        cur.dp = f32x16{};
      }
      // Half 1: products of j with the dS of j - 1.
      float pv[2][2];  // one pair of dS values awaiting conversion
#pragma unroll
      for (int m = 0; m < 24; ++m) {
        if constexpr (HJ) {
          const int i = m < 16 ? m >> 1 : m - 8;  // operand of product m
          const bool first = m < 16 ? !(m & 1) : true;
          if (first && i + 2 < 16) oa[i + 2] = fa(i + 2);
          if (m < 16) {
            if (m & 1) so = mfma32(oa[i], qo[i], so);
            else se = mfma32(oa[i], qe[i], se);
          } else {
            cur.dp = mfma32(oa[i], gf[i - 8], cur.dp);
          }
        }
        if constexpr (HP) {
          if (m >= 22) oc[m - 22] = fc(m - 22);
          if (m < 16) {
            const int r = m;
            pv[r & 1][0] = prv.pe[r] * (prv.dp[r] - ee);
            pv[r & 1][1] = prv.po[r] * (eo - prv.dp[r]);
            if (r & 1) {
              const int kc2 = r >> 3, e = r & 7;
              f16x2 a = __builtin_convertvector((f32x2{pv[0][0], pv[1][0]}), f16x2);
              f16x2 b = __builtin_convertvector((f32x2{pv[0][1], pv[1][1]}), f16x2);
              asm volatile("" : "+v"(a), "+v"(b));  // computed here, not at first use
              be[kc2][e - 1] = a[0];
              be[kc2][e] = a[1];
              bo[kc2][e - 1] = b[0];
              bo[kc2][e] = b[1];
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Half 2: dQ products of j - 1 with the exponentials of j.
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        if constexpr (HP) {
          const int i = m >> 1;
          if (!(m & 1) && i + 2 < 8) oc[i + 2] = fc(i + 2);
          const int kc2 = i >> 2, dt = i & 3;
          if (m & 1) dqo[dt] = mfma32(oc[i], bo[kc2], dqo[dt]);
          else dqe[dt] = mfma32(oc[i], be[kc2], dqe[dt]);
        }
        if constexpr (HJ) {
          const int r = m;
          cur.pe[r] = fast_exp2(fmaf(se[r], c, -Le));
          cur.po[r] = fast_exp2(fmaf(so[r], c, -Lo));
          asm volatile("" : "+v"(cur.pe[r]), "+v"(cur.po[r]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (HJ) {
        if (t + 1 < n_kt) store_part(t + 1, SUB, hreg[SUB]);
        if constexpr (SUB == 1) __syncthreads();
        if (t + 2 < n_kt) load_part(t + 2, SUB, hreg[SUB]);
      }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using T = std::true_type;
    using F = std::false_type;
    step(F{}, T{}, P0{}, 0, cr[1], cr[0]);
    for (int j = 1; j < J - 1; j += 2) {
      step(T{}, T{}, P1{}, j, cr[0], cr[1]);
      step(T{}, T{}, P0{}, j + 1, cr[1], cr[0]);
    }
    step(T{}, T{}, P1{}, J - 1, cr[0], cr[1]);
    step(T{}, F{}, P0{}, J, cr[1], cr[0]);  // the last sub-tile's dS and dQ products
  }
  for (int kt = n_full; kt < n_kt; ++kt) tile(std::true_type{}, kt);
  if (qok) {
    const float fq = p.scale * fast_exp2(-(kap + sg + kv + kk));
    bf16 *de = (bf16 *)p.dq + b * p.dqs_b + (int64_t)my_q * p.dqs_s + 2 * pr * p.dqs_h;
    bf16 *dO = de + p.dqs_h;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = dt * 32 + 8 * g + 4 * h;
        *(bf16x4 *)(de + ch) = bf16x4{f2bf(dqe[dt][4 * g] * fq), f2bf(dqe[dt][4 * g + 1] * fq),
                                      f2bf(dqe[dt][4 * g + 2] * fq), f2bf(dqe[dt][4 * g + 3] * fq)};
        *(bf16x4 *)(dO + ch) = bf16x4{f2bf(dqo[dt][4 * g] * fq), f2bf(dqo[dt][4 * g + 1] * fq),
                                      f2bf(dqo[dt][4 * g + 2] * fq), f2bf(dqo[dt][4 * g + 3] * fq)};
      }
  }
}

// ---------------------------------------------------------------------------
// v2b_dkdv: key-outer.  Workgroup = 128 keys of one (b, KV head); wave w owns
// keys kb + 32 w + 0..31 (lane l % 32).  Streams 64-query chunks of every
// pair on the head through LDS.
constexpr int KVB = 128, QCH = 64;

struct SmemC {
  f16 qe[QCH * QST];
  f16 qo[QCH * QST];
  f16 g[QCH * GST];
  float le[QCH], lo[QCH], ee[QCH], eo[QCH];
};

// One thread's share of a staged query chunk: eight 16-byte chunks of the
// fp16 Q_e | Q_o rows, four of g', and (threads 0..63) one row's statistics
// as loaded.  Nothing is computed from the loaded values until store_chunk2,
// so the loads stay in flight while the previous chunk is processed.
struct ChunkRegs2 {
  u32x4 q[8], g[4];
  float le, lo, ee, eo, lam;
};

// Loads the chunk of QCH query rows of pair pr starting at q0 (rows past the
// end read as zeros; their statistics are read from the last row and masked
// when stored).  The fp16 rows come through buffer loads over the pair's S
// rows (512 bytes of Q_e | Q_o, 256 of g' per row), whose range check gives
// the zeros: no per-row branches, 32-bit offsets.
__device__ __forceinline__ void load_chunk2(const V2BwdParams &p, const Ws2 &w, int b, int pr, int64_t rowb,
                                            int q0, int tid, ChunkRegs2 &r) {
  const int S = p.S;
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc((void *)(w.qh + rowb * (2 * D)), 0, (uint32_t)S * (4 * D), 0x00020000);
  const __amdgpu_buffer_rsrc_t rg =
      __builtin_amdgcn_make_buffer_rsrc((void *)(w.gh + rowb * D), 0, (uint32_t)S * (2 * D), 0x00020000);
#pragma unroll
  for (int k = 0; k < 8; ++k)
    r.q[k] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)((uint32_t)q0 * (4 * D) + (tid + NT * k) * 16), 0, 0));
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r.g[k] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, (int)((uint32_t)q0 * (2 * D) + (tid + NT * k) * 16), 0, 0));
  if (tid < QCH) {
    const int q = min(q0 + tid, S - 1);
    const int64_t lr = ((int64_t)b * p.Hq + 2 * pr) * S + q;
    r.le = p.lse[lr];
    r.lo = p.lse[lr + S];
    r.ee = w.ee[rowb + q];
    r.eo = w.eo[rowb + q];
    r.lam = p.lam[b * p.ls_b + (int64_t)q * p.ls_s + pr * p.ls_p];
  }
}

// Register -> LDS half of the staging.  The statistics are folded so that
// the score loop forms P_e 2^kappa, sigma P_o 2^kappa (sigma the row's
// sigmoid weight) and both dS terms with one exponential and one or two
// operations each:
//   le' = lse_e log2(e) - kappa,  lo' = lse_o log2(e) - kappa - log2(sigma),
//   E_e' = E_e fE,  E_o' = E_o fE;
// rows past the end get infinite lse' (zero probabilities).
__device__ __forceinline__ void store_chunk2(SmemC &sm, const ChunkRegs2 &r, int tid, int q0, int S, float fE,
                                             float kap) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = tid + NT * k, row = i >> 5, col = (i & 31) * 8;
    f16 *dq = col < D ? sm.qe + row * QST + col : sm.qo + row * QST + (col - D);
    *(u32x4 *)dq = r.q[k];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + NT * k, row = i >> 4, col = (i & 15) * 8;
    *(u32x4 *)(sm.g + row * GST + col) = r.g[k];
  }
  if (tid < QCH) {
    const bool ok = q0 + tid < S;
    const float sig = 1.f / (1.f + expf(-r.lam));
    sm.le[tid] = ok ? fmaf(r.le, kLog2e, -kap) : __builtin_inff();
    sm.lo[tid] = ok ? fmaf(r.lo, kLog2e, -(kap + log2f(sig))) : __builtin_inff();
    sm.ee[tid] = ok ? r.ee * fE : 0.f;
    sm.eo[tid] = ok ? r.eo * fE : 0.f;
  }
}

__global__ __launch_bounds__(NT, 1) void v2b_dkdv_kernel(V2BwdParams p, Ws2 w) {
  __shared__ SmemC smb[2];
  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = p.Hq / 2, ppk = p.Hq / p.Hkv / 2;
  // Workgroup id -> (key block, batch, KV head): key blocks with the most
  // causal work first across all heads; consecutive ids walk (batch, head).
  const int BJ = p.B * p.Hkv;
  const int bj = blockIdx.x % BJ, b = bj / p.Hkv, j = bj % p.Hkv;
  const int S = p.S;
  const bool causal = p.causal != 0;
  const int kb = (blockIdx.x / BJ) * KVB, kw = kb + wave * 32, my_key = kw + ln;
  const float sg = w.scales[bj * 8 + 0], kap = w.scales[bj * 8 + 1], om = w.scales[bj * 8 + 2];
  const float kq = w.scales[bj * 8 + 3], kk = w.scales[bj * 8 + 4], kv = w.scales[bj * 8 + 5];
  const VScale sck((int)kk), scv((int)kv);
  // fp16 Q, K, V are Q 2^kq, K 2^kk, V 2^kv: S' = S 2^(kq + kk), dP' = dP 2^(sg + kv).
  const float c = p.scale * kLog2e * fast_exp2(-(kq + kk));
  const float fE = fast_exp2(sg + kv);
  const float fW2 = fast_exp2(om - kap);  // wv = (P_e - sigma P_o) 2^kappa 2^(omega - kappa)

  // K (B operand of S = Q K^T) and V (B operand of dP' = g' V^T) for my key, fp16.
  f16x8 kf[D / 16], vf[D / 16];
  {
    const bool ok = my_key < S;
    const bf16 *kp = (const bf16 *)p.k + b * p.kvs_b + (int64_t)my_key * p.kvs_s + j * p.kvs_h + 8 * h;
    const bf16 *vp = (const bf16 *)p.v + b * p.kvs_b + (int64_t)my_key * p.kvs_s + j * p.kvs_h + 8 * h;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      kf[kc] = ok ? to_f16x8(*(const u32x4 *)(kp + kc * 16), sck) : f16x8{};
      vf[kc] = ok ? to_f16x8(*(const u32x4 *)(vp + kc * 16), scv) : f16x8{};
    }
  }

  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dv[i] = dk[i] = f32x16{};

  const int q_begin = causal ? (kb / QCH) * QCH : 0;
  const int n_ch = q_begin < S ? (S - q_begin + QCH - 1) / QCH : 0;
  const int n_it = n_ch * ppk;  // (pair, chunk) steps
  // Step order: every pair's masked chunks (the diagonal, or all chunks of
  // the last key block), pair-major, then every pair's unmasked chunks; step
  // i stages step i + 1 either way.
  const int n_mask = kb + KVB > S ? n_ch : (causal ? min(n_ch, KVB / QCH) : 0);
  const int n_un = n_ch - n_mask, M = ppk * n_mask;
  auto item_pair = [&](int i) { return j * ppk + (i < M ? i / n_mask : (i - M) / n_un); };
  auto item_q0 = [&](int i) { return q_begin + (i < M ? i % n_mask : n_mask + (i - M) % n_un) * QCH; };
  auto load_item = [&](int i, ChunkRegs2 &r) {
    const int pr = item_pair(i);
    load_chunk2(p, w, b, pr, ((int64_t)b * P + pr) * S, item_q0(i), tid, r);
  };
  const int prow = row_perm(ln);
  // Query chunks double-buffered in LDS: step n + 1 is loaded into registers
  // while step n is computed, then stored to the other buffer; one barrier
  // per step.
  ChunkRegs2 nxt;
  if (n_it > 0) {
    load_item(0, nxt);
    store_chunk2(smb[0], nxt, tid, item_q0(0), S, fE, kap);
  }
  __syncthreads();
  // One (pair, chunk) step; MASKED applies the key-range and causal masks,
  // which only the chunks on this workgroup's diagonal (the first KVB / QCH of
  // each pair under the causal mask) and, in the workgroup holding the last
  // keys, every chunk need: separate loops, so the others carry no mask
  // arithmetic and no branch.
  auto step = [&](auto masked, int it) {
    constexpr bool MASKED = decltype(masked)::value;
    SmemC &sm = smb[it & 1];
    const int q0 = item_q0(it);
    const bool more = it + 1 < n_it;
    if (more) load_item(it + 1, nxt);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int qs = q0 + sub * 32;
      if (qs >= S) continue;
      if (causal && qs + 31 < kw) continue;  // every query of this sub-chunk precedes my keys
      // S_e, S_o = Q K^T and dP' = g' V^T; lane = key, registers = queries.
      f32x16 s_e = {}, s_o = {}, dp = {};
      const f16 *qa = sm.qe + (sub * 32 + prow) * QST + 8 * h;
      const f16 *qb = sm.qo + (sub * 32 + prow) * QST + 8 * h;
      const f16 *ga = sm.g + (sub * 32 + prow) * GST + 8 * h;
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        s_e = mfma32(*(const f16x8 *)(qa + kc * 16), kf[kc], s_e);
        s_o = mfma32(*(const f16x8 *)(qb + kc * 16), kf[kc], s_o);
        dp = mfma32(*(const f16x8 *)(ga + kc * 16), vf[kc], dp);
      }
      // Query qs + o is masked for my key iff o < lo (keys past the end: all;
      // causal: queries before the key).  The mask selects the exponent
      // (-inf), not the exponential, which a select would turn into branches.
      const int lo = my_key >= S ? 32 : (causal ? my_key - qs : -1);
      float wv[16], dse[16], dso[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = sub * 32 + row_of_reg(r, h);
        const bool dead = MASKED && row_of_reg(r, h) < lo;
        const float ae = fmaf(s_e[r], c, -sm.le[qi]), ao = fmaf(s_o[r], c, -sm.lo[qi]);
        const float pe = fast_exp2(dead ? -__builtin_inff() : ae);  // P_e 2^kappa
        const float po = fast_exp2(dead ? -__builtin_inff() : ao);  // sigma P_o 2^kappa
        wv[r] = (pe - po) * fW2;
        dse[r] = pe * (dp[r] - sm.ee[qi]);
        dso[r] = po * (sm.eo[qi] - dp[r]);
      }
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        const f16x8 wb = pack8h(wv + 8 * kc2), be = pack8h(dse + 8 * kc2), bo = pack8h(dso + 8 * kc2);
        const int r0 = sub * 32 + kc2 * 16;
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          dv[ct] = mfma32(tr_operand(sm.g, GST, r0, ct * 32, lane), wb, dv[ct]);
          dk[ct] = mfma32(tr_operand(sm.qe, QST, r0, ct * 32, lane), be, dk[ct]);
          dk[ct] = mfma32(tr_operand(sm.qo, QST, r0, ct * 32, lane), bo, dk[ct]);
        }
      }
    }
    if (more) store_chunk2(smb[(it + 1) & 1], nxt, tid, item_q0(it + 1), S, fE, kap);
    __syncthreads();
  };
  for (int it = 0; it < M; ++it) step(std::true_type{}, it);

  // The unmasked chunks (steps M ..) run as a software pipeline over their
  // 32-query sub-chunks, as in the V1 key-outer kernel: step jp issues the
  // score and dP products of sub-chunk jp beside the dV weights and dS of
  // sub-chunk jp - 1 (from its carried exponentials and dP), then the dV, dK
  // products of jp - 1 beside the exponentials of jp; one matrix instruction
  // and a share of the vector work at a time behind scheduling fences.  Two
  // LDS buffers (step i in buffer i % 2): chunk c + 1 goes into the buffer of
  // chunk c - 1, which sub-chunk 2c last reads, so every step ends with a
  // barrier; it is loaded at the start of step 2c and stored at the start of
  // step 2c + 1.
  const int JP = 2 * (n_it - M);
  if (JP > 0) {
    typedef DA_LDS const char lchar;
    const int hq = 8 * h, jj = lane & 15, half16 = (lane >> 4) & 1;
    const uint32_t laQ = (prow * QST + hq) * 2, laG = (prow * GST + hq) * 2;
    const uint32_t lcQ = ((hq + (jj >> 2)) * QST + 16 * half16 + 4 * (jj & 3)) * 2;
    const uint32_t lcG = ((hq + (jj >> 2)) * GST + 16 * half16 + 4 * (jj & 3)) * 2;
    const uint32_t lst = hq * 4;
    constexpr uint32_t OQE = offsetof(SmemC, qe), OQO = offsetof(SmemC, qo), OG = offsetof(SmemC, g);
    constexpr uint32_t OLE = offsetof(SmemC, le), OLO = offsetof(SmemC, lo), OEE = offsetof(SmemC, ee),
                       OEO = offsetof(SmemC, eo);
    auto lptr = [&](int buf, uint32_t lane_off) -> lchar * {
      lchar *q = (lchar *)(smb + buf) + lane_off;
      asm volatile("" : "+v"(q));
      return q;
    };
    auto tr8 = [&](lchar *q, uint32_t off, int stride) -> f16x8 {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(q + off));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(q + off + 8 * stride));
      const f16x4 a = __builtin_bit_cast(f16x4, lo), bb = __builtin_bit_cast(f16x4, hi);
      return f16x8{a[0], a[1], a[2], a[3], bb[0], bb[1], bb[2], bb[3]};
    };
    struct Carry {
      float pe[16], po[16];  // P_e 2^kappa, sigma P_o 2^kappa
      f32x16 dp;
    };
    Carry cr[2];
    f16x8 wb[2], be[2], bo[2];  // dV / dK operands of the previous sub-chunk

    auto pstep = [&](auto has_prev, auto has_cur, auto parity, int jp, const Carry &prv, Carry &cur) {
      constexpr bool HP = decltype(has_prev)::value;  // sub-chunk jp - 1 exists
      constexpr bool HJ = decltype(has_cur)::value;   // sub-chunk jp exists
      constexpr int SUB = decltype(parity)::value;    // jp % 2
      constexpr int SUBP = 1 - SUB;
      const int ic = M + (jp >> 1);                   // step of sub-chunk jp
      lchar *pAq = nullptr, *pAg = nullptr, *pS = nullptr, *pCq = nullptr, *pCg = nullptr, *pSp = nullptr;
      if constexpr (HJ) {
        pAq = lptr(ic & 1, laQ);
        pAg = lptr(ic & 1, laG);
        pS = lptr(ic & 1, lst);
      }
      if constexpr (HP) {
        const int bc = (M + ((jp - 1) >> 1)) & 1;
        pCq = lptr(bc, lcQ);
        pCg = lptr(bc, lcG);
        pSp = lptr(bc, lst);
      }
      // Staging: the even step loads step ic + 1, the odd step stores it into
      // the other buffer (free since the barrier that ended the even step).
      if constexpr (HJ && SUB == 0) {
        if (ic + 1 < n_it) load_item(ic + 1, nxt);
      }
      if constexpr (HJ && SUB == 1) {
        if (ic + 1 < n_it) store_chunk2(smb[(ic + 1) & 1], nxt, tid, item_q0(ic + 1), S, fE, kap);
      }
      auto rbyte = [&](int sub, int g) -> uint32_t { return (sub * 32 + ((g & 2) << 3) + (g & 1) * 4) * 4; };
      // Product m (0..23) of sub-chunk jp: kc = m / 3; Q_e, Q_o or g' row
      // columns 16 kc against K, K, V.
      auto fa = [&](int m) -> f16x8 {
        const int kc = m / 3, kind = m % 3;
        if (kind == 2) return *(const DA_LDS f16x8 *)(pAg + OG + (SUB * 32 * GST + kc * 16) * 2);
        return *(const DA_LDS f16x8 *)(pAq + (kind ? OQO : OQE) + (SUB * 32 * QST + kc * 16) * 2);
      };
      // dV / dK product m (0..23) of sub-chunk jp - 1: kc2 = m / 12; then
      // channel tile ct and g' (dV), Q_e, Q_o (dK).
      auto fc = [&](int m) -> f16x8 {
        const int kc2 = m / 12, ct = (m % 12) / 3, kind = m % 3, r0 = SUBP * 32 + kc2 * 16;
        if (kind == 0) return tr8(pCg, OG + (r0 * GST + ct * 32) * 2, GST);
        return tr8(pCq, (kind == 1 ? OQE : OQO) + (r0 * QST + ct * 32) * 2, QST);
      };
      f16x8 oa[24], oc[24];
      f32x4 se[4][2], sl[4][2];  // E_e', E_o' of jp - 1; le', lo' of jp (four rows per group)
      auto fetch_e = [&](int g) {
        se[g][0] = *(const DA_LDS f32x4 *)(pSp + OEE + rbyte(SUBP, g));
        se[g][1] = *(const DA_LDS f32x4 *)(pSp + OEO + rbyte(SUBP, g));
      };
      auto fetch_l = [&](int g) {
        sl[g][0] = *(const DA_LDS f32x4 *)(pS + OLE + rbyte(SUB, g));
        sl[g][1] = *(const DA_LDS f32x4 *)(pS + OLO + rbyte(SUB, g));
      };
      f32x16 s_e = {}, s_o = {};
      if constexpr (HJ) {
        oa[0] = fa(0);
        oa[1] = fa(1);
        cur.dp = f32x16{};
      }
      if constexpr (HP) {
        fetch_e(0);
        fetch_e(1);
      }
      // Half 1: products of jp with the dV weights and dS of jp - 1.
      float pv[2][3];  // one pair of results awaiting conversion
#pragma unroll
      for (int m = 0; m < 24; ++m) {
        if constexpr (HJ) {
          if (m + 2 < 24) oa[m + 2] = fa(m + 2);
          const int kc = m / 3, kind = m % 3;
          if (kind == 0) s_e = mfma32(oa[m], kf[kc], s_e);
          else if (kind == 1) s_o = mfma32(oa[m], kf[kc], s_o);
          else cur.dp = mfma32(oa[m], vf[kc], cur.dp);
          if (m == 20) fetch_l(0);
          if (m == 22) fetch_l(1);
        }
        if constexpr (HP) {
          if (m >= 22) oc[m - 22] = fc(m - 22);
          if (m < 16) {
            if ((m & 3) == 0 && m / 4 + 2 < 4) fetch_e(m / 4 + 2);
            const int r = m;
            const float pe = prv.pe[r], po = prv.po[r], dpr = prv.dp[r];
            pv[r & 1][0] = (pe - po) * fW2;
            pv[r & 1][1] = pe * (dpr - se[r >> 2][0][r & 3]);
            pv[r & 1][2] = po * (se[r >> 2][1][r & 3] - dpr);
            if (r & 1) {
              const int kc2 = r >> 3, e = r & 7;
              f16x2 a = __builtin_convertvector((f32x2{pv[0][0], pv[1][0]}), f16x2);
              f16x2 bb = __builtin_convertvector((f32x2{pv[0][1], pv[1][1]}), f16x2);
              f16x2 d = __builtin_convertvector((f32x2{pv[0][2], pv[1][2]}), f16x2);
              asm volatile("" : "+v"(a), "+v"(bb), "+v"(d));  // computed here, not at first use
              wb[kc2][e - 1] = a[0];
              wb[kc2][e] = a[1];
              be[kc2][e - 1] = bb[0];
              be[kc2][e] = bb[1];
              bo[kc2][e - 1] = d[0];
              bo[kc2][e] = d[1];
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Half 2: dV, dK products of jp - 1 with the exponentials of jp.
#pragma unroll
      for (int m = 0; m < 24; ++m) {
        if constexpr (HP) {
          if (m + 2 < 24) oc[m + 2] = fc(m + 2);
          const int kc2 = m / 12, ct = (m % 12) / 3, kind = m % 3;
          if (kind == 0) dv[ct] = mfma32(oc[m], wb[kc2], dv[ct]);
          else if (kind == 1) dk[ct] = mfma32(oc[m], be[kc2], dk[ct]);
          else dk[ct] = mfma32(oc[m], bo[kc2], dk[ct]);
        }
        if constexpr (HJ) {
          if (m < 16) {
            if ((m & 3) == 0 && m / 4 + 2 < 4) fetch_l(m / 4 + 2);
            const int r = m;
            cur.pe[r] = fast_exp2(fmaf(s_e[r], c, -sl[r >> 2][0][r & 3]));
            cur.po[r] = fast_exp2(fmaf(s_o[r], c, -sl[r >> 2][1][r & 3]));
            asm volatile("" : "+v"(cur.pe[r]), "+v"(cur.po[r]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using T = std::true_type;
    using F = std::false_type;
    pstep(F{}, T{}, P0{}, 0, cr[1], cr[0]);
    for (int jp = 1; jp < JP - 1; jp += 2) {
      pstep(T{}, T{}, P1{}, jp, cr[0], cr[1]);
      pstep(T{}, T{}, P0{}, jp + 1, cr[1], cr[0]);
    }
    pstep(T{}, T{}, P1{}, JP - 1, cr[0], cr[1]);
    pstep(T{}, F{}, P0{}, JP, cr[1], cr[0]);  // the last sub-chunk's dV weights, dS and products
  }

  // Epilogue: lane = key, registers = channels 8 (r/4) + 4 h + r%4 of each tile.
  if (my_key < S) {
    const float fv = fast_exp2(-(om + sg));
    const float fk = p.scale * fast_exp2(-(kap + sg + kv + kq));
    bf16 *dvp = (bf16 *)p.dv + b * p.dkvs_b + (int64_t)my_key * p.dkvs_s + j * p.dkvs_h;
    bf16 *dkp = (bf16 *)p.dk + b * p.dkvs_b + (int64_t)my_key * p.dkvs_s + j * p.dkvs_h;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) {
        const int ch = ct * 32 + 8 * g + 4 * h;
        *(bf16x4 *)(dvp + ch) = bf16x4{f2bf(dv[ct][4 * g] * fv), f2bf(dv[ct][4 * g + 1] * fv),
                                       f2bf(dv[ct][4 * g + 2] * fv), f2bf(dv[ct][4 * g + 3] * fv)};
        *(bf16x4 *)(dkp + ch) = bf16x4{f2bf(dk[ct][4 * g] * fk), f2bf(dk[ct][4 * g + 1] * fk),
                                       f2bf(dk[ct][4 * g + 2] * fk), f2bf(dk[ct][4 * g + 3] * fk)};
      }
  }
}

}  // namespace

size_t v2_bwd_workspace_bytes(int B, int S, int Hq, int Hkv) { return ws2_bytes(B, S, Hq / 2, Hkv); }

hipError_t launch_v2_bwd(const V2BwdParams &p, hipStream_t st) {
  const int P = p.Hq / 2;
  Ws2 w = carve2(p.workspace, p.B, p.S, P, p.Hkv);
  const int64_t rows = (int64_t)p.B * P * p.S;
  hipLaunchKernelGGL(v2b_pre_kernel, dim3((rows + RPB - 1) / RPB), dim3(NT), 0, st, p, w);
  hipLaunchKernelGGL(v2b_scales_kernel, dim3(p.B * p.Hkv), dim3(NTS), 0, st, p, w);
  hipLaunchKernelGGL(v2b_gconv_kernel, dim3((rows + RPB - 1) / RPB), dim3(NT), 0, st, p, w);
  const int n_qt = (p.S + QB - 1) / QB;
  hipLaunchKernelGGL(v2b_dq_kernel, dim3(n_qt * p.B * P), dim3(NT), 0, st, p, w);
  hipLaunchKernelGGL(v2b_dkdv_kernel, dim3((p.S + KVB - 1) / KVB * p.B * p.Hkv), dim3(NT), 0, st, p, w);
  return hipGetLastError();
}

}  // namespace diffattn
