// Differential attention forward with fp8 attention logits on gfx950: the
// score products Q1 K1^T and Q2 K2^T run on fp8 e4m3 operands (scaled fp8
// matrix instructions, v_mfma_scale_f32_32x32x64_f8f6f4), everything after
// the scores in two passes (pass 1: each map's exact log-sum-exp; pass 2: the
// combined weight rounded once to fp16, fp16 V, per-head RMSNorm x
// (1 - lambda_init)).  bf16 storage, d = 64, dv = 128.
//
// Quantisation (the low-bit attention-logit study and the "low-bit
// FlashAttention" outlook on the pages: absmax dynamic post-training
// quantisation of the logits' inputs): each row of Q1, K1, Q2, K2 (one token of
// one head, 64 channels) is divided by 2^e, e the smallest integer with
// max|row| 2^-e <= 448 (the largest e4m3 value), and rounded to nearest-even
// e4m3.  With a power-of-two scale the division is exact, so the codes are a
// pure function of the bf16 inputs.  Dequantisation is free: the key rows'
// exponents enter the matrix instruction as its per-row E8M0 scale (127 + e),
// and the query rows' exponents fold into the per-lane softmax constant
// (scores are computed transposed, one query per lane).
//
// fp8q_kernel writes the codes (uint8 [4][B, H, S, 64]: Q1, K1, Q2, K2, rows
// contiguous per (batch, head)) and the exponents (int32 [4][B, H, S]) to the
// workspace; fwd_fp8_kernel is the bf16 forward's workgroup layout with 64-key
// tiles of K1, K2 codes (80-byte LDS rows: 16 consecutive rows fall on 16
// different 16-byte bank groups), their exponents, and the fp16 V tile.
#include "attn_tile.h"
#include "kernels.h"
#include "vrange.h"

namespace diffattn {
namespace {

constexpr int D = 64, DV = 128, BM = 128, BN = 64, NT = 256;
constexpr int KST8 = 80;       // LDS row stride of a K code tile, bytes
constexpr int VST = DV + 32;   // LDS row stride of the V tile, fp16 elements (320 B)

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct Fp8Ws {
  uint8_t *codes;  // [4][B, H, S, D]
  int *exps;       // [4][B, H, S]
};

__host__ __device__ inline size_t al256f(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Fp8Ws carve_fp8(void *base, int B, int S, int H) {
  const size_t rows = (size_t)B * H * S;
  Fp8Ws w;
  w.codes = static_cast<uint8_t *>(base);
  w.exps = reinterpret_cast<int *>(static_cast<char *>(base) + al256f(4 * rows * D));
  return w;
}

// ---------------------------------------------------------------------------
// Quantisation: 8 lanes per row of one tensor (t = 0..3: Q1, K1, Q2, K2), 8
// channels (one 16-byte load) per lane, 32 rows per workgroup.
__global__ __launch_bounds__(NT) void fp8q_kernel(FwdParams p, Fp8Ws w) {
  const int tid = threadIdx.x, part = tid & 7;
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  const int64_t gr = (int64_t)blockIdx.x * (NT / 8) + (tid >> 3);  // over [4][B, H, S]
  const bool ok = gr < 4 * rows;
  const int64_t g = ok ? gr : 0;
  const int t = g / rows;
  const int64_t row = g % rows;
  const int s = row % p.S, bh = row / p.S, b = bh / p.H, hd = bh % p.H;
  const bf16 *src;
  if (t == 0 || t == 2)
    src = (const bf16 *)(t == 0 ? p.q1 : p.q2) + b * p.qs_b + (int64_t)s * p.qs_s + hd * p.qs_h;
  else
    src = (const bf16 *)(t == 1 ? p.k1 : p.k2) + b * p.ks_b + (int64_t)s * p.ks_s + hd * p.ks_h;
  const u32x4 raw = *(const u32x4 *)(src + part * 8);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(raw[i] << 16);
    x[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
  }
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
  for (int o = 1; o < 8; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
  // e: smallest integer with a 2^-e <= 448, from a's exponent and mantissa bits.
  const uint32_t bits = __float_as_uint(a);
  const int ebits = (int)(bits >> 23) & 255;
  int e = 0;
  if (a > 0.f) {
    e = ebits == 0 ? -120 : (ebits - 127) - 8 + ((bits & 0x7fffff) > 0x600000u);
    e = min(max(e, -120), 120);
  }
  int lo = 0, hi = 0;  // exact scaling: |x 2^-e| <= 448
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[0], -e), ldexpf(x[1], -e), lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[2], -e), ldexpf(x[3], -e), lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4], -e), ldexpf(x[5], -e), hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[6], -e), ldexpf(x[7], -e), hi, true);
  if (ok) {
    *(u32x2 *)(w.codes + gr * D + part * 8) = u32x2{(uint32_t)lo, (uint32_t)hi};
    if (part == 0) w.exps[gr] = e;
  }
}

// ---------------------------------------------------------------------------
struct SmemF {
  uint8_t k1[BN * KST8];
  uint8_t k2[BN * KST8];
  int ek1[BN], ek2[BN];
  f16 v[BN * VST];
};

struct TileRegsF {
  u32x4 k1, k2, v[4];
  int ek;  // threads 0..127: one key exponent (map (tid >> 6), key tid & 63)
};

// Code tiles, exponents and V through raw buffer loads; ranges end at the
// slice's last row, so rows past the sequence end read as zeros.
struct LoaderF {
  __amdgpu_buffer_rsrc_t rk1, rk2, re1, re2, rv;
  uint32_t ko, vo[4];
  uint32_t vstep;
  int tid;

  __device__ __forceinline__ void init(const uint8_t *k1, const uint8_t *k2, const int *e1, const int *e2,
                                       const bf16 *v, int64_t vs, int S, int tid_) {
    tid = tid_;
    rk1 = __builtin_amdgcn_make_buffer_rsrc((void *)k1, 0, (uint32_t)S * D, 0x00020000);
    rk2 = __builtin_amdgcn_make_buffer_rsrc((void *)k2, 0, (uint32_t)S * D, 0x00020000);
    re1 = __builtin_amdgcn_make_buffer_rsrc((void *)e1, 0, (uint32_t)S * 4, 0x00020000);
    re2 = __builtin_amdgcn_make_buffer_rsrc((void *)e2, 0, (uint32_t)S * 4, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void *)v, 0, (uint32_t)((int64_t)(S - 1) * vs * 2 + DV * 2),
                                           0x00020000);
    vstep = (uint32_t)(vs * 2);
    ko = (uint32_t)tid * 16;  // 256 threads x 16 B = one 64 x 64-byte code tile
#pragma unroll
    for (int i = 0; i < 4; ++i) vo[i] = (uint32_t)((tid >> 4) + 16 * i) * vstep + (tid & 15) * 16;
  }

  __device__ __forceinline__ void load(int kbase, bool with_v, TileRegsF &r) const {
    const uint32_t kb = (uint32_t)kbase * D;
    r.k1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk1, (int)(ko + kb), 0, 0));
    r.k2 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk2, (int)(ko + kb), 0, 0));
    // One descriptor per branch: each is taken by whole waves (0 and 1).
    if (tid < BN)
      r.ek = __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(re1, (kbase + tid) * 4, 0, 0));
    else if (tid < 2 * BN)
      r.ek = __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(re2, (kbase + tid - BN) * 4, 0, 0));
    if (with_v) {
      const uint32_t vb = (uint32_t)kbase * vstep;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(vo[i] + vb), 0, 0));
    }
  }
};

__device__ __forceinline__ void store_tile(SmemF &sm, const TileRegsF &r, int tid, bool with_v,
                                           const VScale &vsc) {
  const int row = tid >> 2, col = (tid & 3) * 16;
  *(u32x4 *)(sm.k1 + row * KST8 + col) = r.k1;
  *(u32x4 *)(sm.k2 + row * KST8 + col) = r.k2;
  if (tid < BN) sm.ek1[tid] = r.ek;
  else if (tid < 2 * BN) sm.ek2[tid - BN] = r.ek;
  if (with_v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vr = (tid >> 4) + 16 * i, vc = (tid & 15) * 8;
      const u32x4 h = bf16x8_to_f16x8_scaled(r.v[i], vsc);
      *(u32x4 *)(sm.v + vr * VST + vc) = h;
    }
  }
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8 &a, const i32x8 &b, int scale_a) {
  // A and B fp8 e4m3 (format 0); A rows scaled by 2^(scale_a - 127), B unscaled.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, f32x16{}, 0, 0, 0, scale_a, 0, 127);
}

// S^T sub-tile (32 keys x 32 queries) of both maps: one scaled fp8 matrix
// instruction per map covers the whole 64-channel dot product.
__device__ __forceinline__ void scores_f(const SmemF &sm, int sub, int krow, int h, const i32x8 &qf1,
                                        const i32x8 &qf2, f32x16 &s1, f32x16 &s2) {
  const int r = sub * 32 + krow;
  const uint8_t *a1 = sm.k1 + r * KST8 + 32 * h, *a2 = sm.k2 + r * KST8 + 32 * h;
  const u32x4 a1l = *(const u32x4 *)a1, a1h = *(const u32x4 *)(a1 + 16);
  const u32x4 a2l = *(const u32x4 *)a2, a2h = *(const u32x4 *)(a2 + 16);
  const i32x8 A1 = {(int)a1l[0], (int)a1l[1], (int)a1l[2], (int)a1l[3], (int)a1h[0], (int)a1h[1], (int)a1h[2],
                    (int)a1h[3]};
  const i32x8 A2 = {(int)a2l[0], (int)a2l[1], (int)a2l[2], (int)a2l[3], (int)a2h[0], (int)a2h[1], (int)a2h[2],
                    (int)a2h[3]};
  s1 = mfma_fp8(A1, qf1, 127 + sm.ek1[r]);
  s2 = mfma_fp8(A2, qf2, 127 + sm.ek2[r]);
}

// Interior tiles (MASKED = false) issue both sub-tiles' score products before
// any softmax arithmetic, so the vector work of the first overlaps the matrix
// work of the second.
template <bool MASKED>
__device__ __forceinline__ void pass1_tile(const SmemF &sm, int kbase, int krow, int h, const i32x8 &qf1,
                                           const i32x8 &qf2, float c1, float c2, float &m1, float &l1, float &m2,
                                           float &l2, int S, bool causal, int qw, int my_q) {
  if constexpr (!MASKED) {
    f32x16 s1a, s2a, s1b, s2b;
    scores_f(sm, 0, krow, h, qf1, qf2, s1a, s2a);
    scores_f(sm, 1, krow, h, qf1, qf2, s1b, s2b);
    lse_update(s1a, c1, m1, l1);
    lse_update(s2a, c2, m2, l2);
    lse_update(s1b, c1, m1, l1);
    lse_update(s2b, c2, m2, l2);
  } else {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int sb = kbase + sub * 32;
      if (sb >= S || (causal && sb > qw + 31)) continue;
      f32x16 s1, s2;
      scores_f(sm, sub, krow, h, qf1, qf2, s1, s2);
      if ((causal && sb + 31 > qw) || sb + 32 > S) mask_scores(s1, s2, sb, h, S, causal, my_q);
      lse_update(s1, c1, m1, l1);
      lse_update(s2, c2, m2, l2);
    }
  }
}

__device__ __forceinline__ void pass2_sub(const SmemF &sm, int sub, int lane, const f32x16 &s1, const f32x16 &s2,
                                          float c1, float c2, float lam, float L1s, float L2s, f32x16 *o) {
  float w[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) w[r] = fast_exp2(fmaf(s1[r], c1, -L1s)) - lam * fast_exp2(fmaf(s2[r], c2, -L2s));
  const f16x8 wb[2] = {pack8(w), pack8(w + 8)};
  pv_step_tile<VST, 4>(sm.v, sub, lane, wb, o);
}

template <bool MASKED>
__device__ __forceinline__ void pass2_tile(const SmemF &sm, int kbase, int krow, int lane, const i32x8 &qf1,
                                           const i32x8 &qf2, float c1, float c2, float lam, float L1s, float L2s,
                                           f32x16 *o, int S, bool causal, int qw, int my_q) {
  const int h = lane >> 5;
  if constexpr (!MASKED) {
    f32x16 s1a, s2a, s1b, s2b;
    scores_f(sm, 0, krow, h, qf1, qf2, s1a, s2a);
    scores_f(sm, 1, krow, h, qf1, qf2, s1b, s2b);
    pass2_sub(sm, 0, lane, s1a, s2a, c1, c2, lam, L1s, L2s, o);
    pass2_sub(sm, 1, lane, s1b, s2b, c1, c2, lam, L1s, L2s, o);
  } else {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int sb = kbase + sub * 32;
      if (sb >= S || (causal && sb > qw + 31)) continue;
      f32x16 s1, s2;
      scores_f(sm, sub, krow, h, qf1, qf2, s1, s2);
      if ((causal && sb + 31 > qw) || sb + 32 > S) mask_scores(s1, s2, sb, h, S, causal, my_q);
      pass2_sub(sm, sub, lane, s1, s2, c1, c2, lam, L1s, L2s, o);
    }
  }
}

__global__ __launch_bounds__(NT, 2) void fwd_fp8_kernel(FwdParams p, Fp8Ws w) {
  __shared__ SmemF sm[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, h = lane >> 5;
  const int BH = p.B * p.H;
  const int n_qt = (p.S + BM - 1) / BM;
  const int bh = blockIdx.x % BH;
  const int qt_i = blockIdx.x / BH;
  const int qt = p.causal ? n_qt - 1 - qt_i : qt_i;
  const int b = bh / p.H, hd = bh % p.H;
  const int q0 = qt * BM, qw = q0 + wave * 32, my_q = qw + ln;
  const int S = p.S;
  const bool causal = p.causal != 0;
  const bool qok = my_q < S;

  const float lam = wave_lambda(p.lq1, p.lk1, p.lq2, p.lk2, p.lambda_dim, p.lambda_fixed, p.lambda_init);
  if (blockIdx.x == 0 && tid == 0 && p.lambda_out) *p.lambda_out = lam;

  const int64_t rows = (int64_t)BH * S;
  const int64_t rb = (int64_t)bh * S;  // this (batch, head)'s first row in [B, H, S]
  LoaderF ld;
  ld.init(w.codes + (1 * rows + rb) * D, w.codes + (3 * rows + rb) * D, w.exps + 1 * rows + rb,
          w.exps + 3 * rows + rb, (const bf16 *)p.v + b * p.vs_b + hd * p.vs_h, p.vs_s, S, tid);

  // B operands: the query's fp8 codes (channels 32 h .. 32 h + 31), and the
  // query exponents folded into the per-lane softmax constants.
  i32x8 qf1 = {}, qf2 = {};
  float c1 = p.scale * kLog2e, c2 = c1;  // rows past the end: zero queries, as in the bf16 forward
  if (qok) {
    const uint8_t *q1 = w.codes + (0 * rows + rb + my_q) * D + 32 * h;
    const uint8_t *q2 = w.codes + (2 * rows + rb + my_q) * D + 32 * h;
    const u32x4 x0 = *(const u32x4 *)q1, x1 = *(const u32x4 *)(q1 + 16);
    const u32x4 y0 = *(const u32x4 *)q2, y1 = *(const u32x4 *)(q2 + 16);
    qf1 = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    qf2 = i32x8{(int)y0[0], (int)y0[1], (int)y0[2], (int)y0[3], (int)y1[0], (int)y1[1], (int)y1[2], (int)y1[3]};
    c1 = ldexpf(p.scale * kLog2e, w.exps[0 * rows + rb + my_q]);
    c2 = ldexpf(p.scale * kLog2e, w.exps[2 * rows + rb + my_q]);
  }

  const int kend = causal ? min(S, q0 + BM) : S;
  const int n_kt = (kend + BN - 1) / BN;
  const int n_full = min(causal ? (q0 + 1) / BN : n_kt, S / BN);
  const int krow = k_row_perm(ln);
  // fp16 V is V 2^vk (range of bf16; see vrange.h); the epilogue removes it.
  const int vk = v_shift(p.vpart + (int64_t)bh * vrange_chunks(S), vrange_chunks(kend));
  const VScale vsc(vk);

  // ---------------- pass 1: per-map log2 partition functions ----------------
  float m1 = kNegInf, l1 = 0.f, m2 = kNegInf, l2 = 0.f;
  TileRegsF nxt;
  ld.load(0, false, nxt);
  store_tile(sm[0], nxt, tid, false, vsc);
  __syncthreads();
  for (int kt = 0; kt < n_full; ++kt) {
    ld.load((kt + 1) * BN, false, nxt);  // past the end: the buffer range gives zeros
    sched_fence();
    pass1_tile<false>(sm[kt & 1], kt * BN, krow, h, qf1, qf2, c1, c2, m1, l1, m2, l2, S, causal, qw, my_q);
    sched_fence();
    store_tile(sm[(kt + 1) & 1], nxt, tid, false, vsc);
    __syncthreads();
  }
  for (int kt = n_full; kt < n_kt; ++kt) {
    ld.load((kt + 1) * BN, false, nxt);
    sched_fence();
    pass1_tile<true>(sm[kt & 1], kt * BN, krow, h, qf1, qf2, c1, c2, m1, l1, m2, l2, S, causal, qw, my_q);
    sched_fence();
    store_tile(sm[(kt + 1) & 1], nxt, tid, false, vsc);
    __syncthreads();
  }
  float M1, L1, M2, L2;
  lse_finish(m1, l1, M1, L1);
  lse_finish(m2, l2, M2, L2);
  const float sg = row_scale_log2(1.f + fabsf(lam));  // a map's weights are at most 1
  const float L1s = L1 - sg, L2s = L2 - sg;

  // ---------------- pass 2: O = (P1 / l1 - lambda P2 / l2) V ----------------
  f32x16 o[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) o[ct] = f32x16{};
  ld.load(0, true, nxt);
  store_tile(sm[0], nxt, tid, true, vsc);
  __syncthreads();
  for (int kt = 0; kt < n_full; ++kt) {
    ld.load((kt + 1) * BN, true, nxt);
    sched_fence();
    pass2_tile<false>(sm[kt & 1], kt * BN, krow, lane, qf1, qf2, c1, c2, lam, L1s, L2s, o, S, causal, qw, my_q);
    sched_fence();
    store_tile(sm[(kt + 1) & 1], nxt, tid, true, vsc);
    __syncthreads();
  }
  for (int kt = n_full; kt < n_kt; ++kt) {
    ld.load((kt + 1) * BN, true, nxt);
    sched_fence();
    pass2_tile<true>(sm[kt & 1], kt * BN, krow, lane, qf1, qf2, c1, c2, lam, L1s, L2s, o, S, causal, qw, my_q);
    sched_fence();
    store_tile(sm[(kt + 1) & 1], nxt, tid, true, vsc);
    __syncthreads();
  }

  // ---------------- epilogue: per-head RMSNorm x (1 - lambda_init) ----------------
  const float unscale = __builtin_ldexpf(1.f, -vk) * fast_exp2(-sg);
  float ss = 0.f;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) ss = fmaf(o[ct][r], o[ct][r], ss);
  ss += other_half(ss);
  ss *= unscale * unscale;
  const float rstd = p.norm ? 1.f / sqrtf(ss * (1.f / DV) + p.eps) : 1.f;
  const float f = (p.norm ? rstd * (1.f - p.lambda_init) : 1.f) * unscale;
  if (qok) {
    bf16 *out = (bf16 *)p.out + b * p.os_b + (int64_t)my_q * p.os_s + hd * p.os_h;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = ct * 32 + 8 * g + 4 * h;
        bf16x4 y = {f2bf(o[ct][4 * g] * f), f2bf(o[ct][4 * g + 1] * f), f2bf(o[ct][4 * g + 2] * f),
                    f2bf(o[ct][4 * g + 3] * f)};
        *(bf16x4 *)(out + ch) = y;
      }
  }
}

}  // namespace

size_t fwd_fp8_workspace_bytes(int B, int S, int H) {
  const size_t rows = (size_t)B * H * S;
  return al256f(4 * rows * D) + al256f(4 * rows * 4) + vrange_bytes(B, S, H);
}

hipError_t launch_fwd_fp8(const FwdParams &p0, void *workspace, hipStream_t st) {
  Fp8Ws w = carve_fp8(workspace, p0.B, p0.S, p0.H);
  const int64_t rows = (int64_t)p0.B * p0.H * p0.S;
  FwdParams p = p0;
  p.vpart = reinterpret_cast<const unsigned *>(static_cast<char *>(workspace) + al256f(4 * rows * D) +
                                               al256f(4 * rows * 4));
  VRangeParams vr{p.v, p.vs_b, p.vs_s, p.vs_h, p.B, p.S, p.H, const_cast<unsigned *>(p.vpart)};
  hipError_t e = launch_vrange(vr, DV, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fp8q_kernel, dim3((4 * rows + NT / 8 - 1) / (NT / 8)), dim3(NT), 0, st, p, w);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_qt = (p.S + BM - 1) / BM;
  hipLaunchKernelGGL(fwd_fp8_kernel, dim3(n_qt * p.B * p.H), dim3(NT), 0, st, p, w);
  return hipGetLastError();
}

}  // namespace diffattn
