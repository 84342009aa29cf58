// Fused causal/non-causal training-mode forward of multi-head differential
// attention on gfx950 matrix cores: bf16 storage, d = 64 (query/key width),
// dv = 128; it also writes the saves the backward reads.  The inference
// forward (no saves) is the one-pass kernel of fwd_onepass.hip.
//
// The operator (glossary page "Differential Transformer", section "How
// differential attention works"; news write-up, multi-head section):
//   Y = RMSNorm_head((softmax(s Q1 K1^T) - lambda softmax(s Q2 K2^T)) V) (1 - lambda_init)
//
// Work split.  One workgroup of 4 waves owns 128 query rows of one (batch,
// head); wave w owns rows 32w .. 32w+31.  Causal tiles are issued longest
// first, and consecutive workgroup ids walk the (batch, head) index so every
// query tile of one head lands on the same XCD (workgroups are dealt to the 8
// XCDs round-robin), sharing that XCD's L2 for the head's K and V.
//
// Two passes over 64-key tiles staged through LDS:
//   pass 1 streams K1, K2 and computes, per map and query row, the log2
//          partition function L_m (online sum of 2^(s c) against a reference
//          that moves only when a score tops it by more than 64);
//   pass 2 streams K1, K2, V, recomputes the scores and forms the combined,
//          already normalised weight W = 2^(s1 c - L1) - lambda 2^(s2 c - L2)
//          in float32, rounds W once to fp16 and accumulates O = W V.
// Rounding the combined weight once (rather than each map's probabilities
// separately) keeps the error proportional to |map1 - lambda map2|: when
// lambda is near 1 the two maps cancel and per-map rounding error would be
// amplified by 1 / (1 - lambda).  W and V enter the PV product as fp16 (V is
// converted exactly from bf16 on its way into LDS), because bf16's 8-bit
// significand alone would spend most of the error budget.  W is scaled by a
// power of two 2^sigma with (1 + |lambda|) 2^sigma just under 2^15 (a map's
// weights are at most 1, so |W| <= 1 + |lambda|); even 64K-key rows of
// ~1/65536 weights then stay in fp16's normal range.  sigma folds into L for
// free and the epilogue removes it exactly.  Matrix-core work per (query, key) pair is 4 QK^T products of
// width 64 plus one PV product of width 128: 768 flop, the same as a one-pass
// form with two PV products.
//
// Scores are computed transposed, S^T = K Q^T (keys on rows), so that each lane
// owns one query column: row max, row sum and the online-softmax state are
// per-lane scalars, and the score registers are already in the B-operand
// layout of the PV product O^T = V^T W^T.  K rows are loaded in a permuted
// order inside each 16-row block so that a lane's 16 score registers are keys
// 8 h + 0..7 and 16 + 8 h + 0..7 (h = lane / 32), exactly the k-slots of two
// 32x32x16 PV steps.  V^T operands come from the row-major V tile through LDS
// transpose reads.  The epilogue (RMSNorm over the head's 128 channels) reduces
// inside the lane and across the two half-waves.  V enters fp16 times a
// power of two chosen per workgroup so bf16's whole range converts (vrange.h).
#include "attn_tile.h"
#include "kernels.h"
#include "v1_stage.h"

namespace diffattn {
namespace {

using namespace v1s;

constexpr int BM = 128;

// S^T sub-tile (32 keys x 32 queries) of both maps.
__device__ __forceinline__ void scores(const Smem &sm, int sub, int krow, int h, const bf16x8 *qf1,
                                       const bf16x8 *qf2, f32x16 &s1, f32x16 &s2) {
  const bf16 *a1 = sm.k1 + (sub * 32 + krow) * KST + 8 * h;
  const bf16 *a2 = sm.k2 + (sub * 32 + krow) * KST + 8 * h;
  s1 = f32x16{};
  s2 = f32x16{};
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    s1 = mfma32(*(const bf16x8 *)(a1 + kc * 16), qf1[kc], s1);
    s2 = mfma32(*(const bf16x8 *)(a2 + kc * 16), qf2[kc], s2);
  }
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

// O^T[ct] += V^T (channels ct*32.., keys of sub-tile chunk kc2) * W^T.
__device__ __forceinline__ void pv_step(const Smem &sm, int sub, int lane, const f16x8 *wb, f32x16 *o) {
  pv_step_tile<VST, 4>(sm.v, sub, lane, wb, o);
}

// Pass 1 over one staged 64-key tile.  MASKED = false: every key of the tile
// is visible to every query of the workgroup; both sub-tiles' score products
// are issued before any softmax arithmetic so the exponentials of the first
// overlap the matrix work of the second.
template <bool MASKED>
__device__ __forceinline__ void pass1_tile(const Smem &sm, int kbase, int krow, int h, const bf16x8 *qf1,
                                           const bf16x8 *qf2, float c, float &m1, float &l1, float &m2,
                                           float &l2, int S, bool causal, int qw, int my_q) {
  if constexpr (!MASKED) {
    f32x16 s1a, s2a, s1b, s2b;
    scores(sm, 0, krow, h, qf1, qf2, s1a, s2a);
    scores(sm, 1, krow, h, qf1, qf2, s1b, s2b);
    lse_update(s1a, c, m1, l1);
    lse_update(s2a, c, m2, l2);
    lse_update(s1b, c, m1, l1);
    lse_update(s2b, c, m2, l2);
  } else {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int sb = kbase + sub * 32;
      if (sb >= S || (causal && sb > qw + 31)) continue;
      f32x16 s1, s2;
      scores(sm, sub, krow, h, qf1, qf2, s1, s2);
      if ((causal && sb + 31 > qw) || sb + 32 > S) mask_scores(s1, s2, sb, h, S, causal, my_q);
      lse_update(s1, c, m1, l1);
      lse_update(s2, c, m2, l2);
    }
  }
}

// Combined weights of one sub-tile and their PV product.
template <bool SAVE>
__device__ __forceinline__ void pass2_sub(const Smem &sm, int sub, int lane, const f32x16 &s1, const f32x16 &s2,
                                          float c, float lam, float L1s, float L2s, float L2s2, f32x16 *o,
                                          f32x16 *o2) {
  float w[16];
#pragma unroll
  for (int r = 0; r < 16; ++r)
    w[r] = fast_exp2(fmaf(s1[r], c, -L1s)) - lam * fast_exp2(fmaf(s2[r], c, -L2s));
  if constexpr (!SAVE) {
    const f16x8 wb[2] = {pack8(w), pack8(w + 8)};
    pv_step(sm, sub, lane, wb, o);
  } else {
    // Training saves feed the backward, whose lambda gradient sums
    // g . A2 over every row with heavy cancellation: O and A2 are
    // accumulated from fp16 hi + lo weight pairs (two PV products each).
    f16x8 hi[2], lo[2];
    pack8_hilo(w, hi[0], lo[0]);
    pack8_hilo(w + 8, hi[1], lo[1]);
    pv_step(sm, sub, lane, hi, o);
    pv_step(sm, sub, lane, lo, o);
    float w2[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) w2[r] = fast_exp2(fmaf(s2[r], c, -L2s2));
    pack8_hilo(w2, hi[0], lo[0]);
    pack8_hilo(w2 + 8, hi[1], lo[1]);
    pv_step(sm, sub, lane, hi, o2);
    pv_step(sm, sub, lane, lo, o2);
  }
}

// Pass 2 over one staged tile: combined weights, PV accumulation (interior
// tiles issue both sub-tiles' score products first, as in pass 1).
template <bool MASKED, bool SAVE>
__device__ __forceinline__ void pass2_tile(const Smem &sm, int kbase, int krow, int lane, const bf16x8 *qf1,
                                           const bf16x8 *qf2, float c, float lam, float L1s, float L2s,
                                           float L2s2, f32x16 *o, f32x16 *o2, int S, bool causal, int qw,
                                           int my_q) {
  const int h = lane >> 5;
  if constexpr (!MASKED) {
    f32x16 s1a, s2a, s1b, s2b;
    scores(sm, 0, krow, h, qf1, qf2, s1a, s2a);
    scores(sm, 1, krow, h, qf1, qf2, s1b, s2b);
    pass2_sub<SAVE>(sm, 0, lane, s1a, s2a, c, lam, L1s, L2s, L2s2, o, o2);
    pass2_sub<SAVE>(sm, 1, lane, s1b, s2b, c, lam, L1s, L2s, L2s2, o, o2);
  } else {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int sb = kbase + sub * 32;
      if (sb >= S || (causal && sb > qw + 31)) continue;
      f32x16 s1, s2;
      scores(sm, sub, krow, h, qf1, qf2, s1, s2);
      if ((causal && sb + 31 > qw) || sb + 32 > S) mask_scores(s1, s2, sb, h, S, causal, my_q);
      pass2_sub<SAVE>(sm, sub, lane, s1, s2, c, lam, L1s, L2s, L2s2, o, o2);
    }
  }
}

template <bool SAVE>
__global__ __launch_bounds__(NT, SAVE ? 1 : 2) void fwd_mfma_kernel(FwdParams p) {
  __shared__ Smem sm[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  const float lam = wave_lambda(p.lq1, p.lk1, p.lq2, p.lk2, p.lambda_dim, p.lambda_fixed, p.lambda_init);
  if (blockIdx.x == 0 && tid == 0 && p.lambda_out) *p.lambda_out = lam;
  const float c = p.scale * kLog2e;

  TileLoader ld;
  ld.init((const bf16 *)p.k1 + b * p.ks_b + hd * p.ks_h, (const bf16 *)p.k2 + b * p.ks_b + hd * p.ks_h,
          (const bf16 *)p.v + b * p.vs_b + hd * p.vs_h, p.ks_s, p.vs_s, S, tid);

  bf16x8 qf1[4], qf2[4];
  {
    const bf16 *q1 = (const bf16 *)p.q1 + b * p.qs_b + (int64_t)my_q * p.qs_s + hd * p.qs_h + 8 * h;
    const bf16 *q2 = (const bf16 *)p.q2 + b * p.qs_b + (int64_t)my_q * p.qs_s + hd * p.qs_h + 8 * h;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      qf1[kc] = my_q < S ? *(const bf16x8 *)(q1 + kc * 16) : bf16x8{};
      qf2[kc] = my_q < S ? *(const bf16x8 *)(q2 + kc * 16) : bf16x8{};
    }
  }

  const int kend = causal ? min(S, q0 + BM) : S;
  const int n_kt = (kend + BN - 1) / BN;
  // fp16 V is V 2^vk (range of bf16; see vrange.h); the epilogue removes it.
  const int vk = v_shift(p.vpart + (int64_t)bh * vrange_chunks(S), vrange_chunks(kend));
  const VScale vsc(vk);
  // Tiles every query of the workgroup sees in full (no mask, no tail).
  const int n_full = min(causal ? (q0 + 1) / BN : n_kt, S / BN);
  const int krow = k_row_perm(ln);

  // ---------------- pass 1: per-map log2 partition functions ----------------
  // Double-buffered LDS: tile kt is computed from buffer kt % 2 while tile
  // kt + 1 (loaded into registers one tile ahead) is stored to the other
  // buffer; one barrier per tile.
  float m1 = kNegInf, l1 = 0.f, m2 = kNegInf, l2 = 0.f;
  TileRegs nxt;
  ld.load(0, false, nxt);
  store_tile(sm[0], nxt, tid, false, vsc);
  __syncthreads();
  // Interior tiles first (straight-line, no masks), then the diagonal / tail.
  for (int kt = 0; kt < n_full; ++kt) {
    ld.load((kt + 1) * BN, false, nxt);  // past the end: the buffer range gives zeros
    sched_fence();
    pass1_tile<false>(sm[kt & 1], kt * BN, krow, h, qf1, qf2, c, m1, l1, m2, l2, S, causal, qw, my_q);
    sched_fence();
    store_tile(sm[(kt + 1) & 1], nxt, tid, false, vsc);
    __syncthreads();
  }
  for (int kt = n_full; kt < n_kt; ++kt) {
    ld.load((kt + 1) * BN, false, nxt);
    sched_fence();
    pass1_tile<true>(sm[kt & 1], kt * BN, krow, h, qf1, qf2, c, m1, l1, m2, l2, S, causal, qw, my_q);
    sched_fence();
    store_tile(sm[(kt + 1) & 1], nxt, tid, false, vsc);
    __syncthreads();
  }
  float M1, L1, M2, L2;
  lse_finish(m1, l1, M1, L1);
  lse_finish(m2, l2, M2, L2);
  // Scale 2^sg for the fp16 weights (and 2^sg2 for the saved second map): a
  // map's weights are at most 1, so |W| <= 1 + |lambda|.
  const float sg = row_scale_log2(1.f + fabsf(lam));
  const float L1s = L1 - sg, L2s = L2 - sg;
  const float sg2 = SAVE ? row_scale_log2(1.f) : 0.f;
  const float L2s2 = L2 - sg2;

  // ---------------- pass 2: O = (P1 / l1 - lambda P2 / l2) V ----------------
  f32x16 o[4], o2[SAVE ? 4 : 1];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) o[ct] = f32x16{};
  if constexpr (SAVE) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) o2[ct] = f32x16{};
  }
  ld.load(0, true, nxt);
  store_tile(sm[0], nxt, tid, true, vsc);
  __syncthreads();
  for (int kt = 0; kt < n_full; ++kt) {
    ld.load((kt + 1) * BN, true, nxt);
    if constexpr (!SAVE) sched_fence();
    pass2_tile<false, SAVE>(sm[kt & 1], kt * BN, krow, lane, qf1, qf2, c, lam, L1s, L2s, L2s2, o, o2, S, causal,
                            qw, my_q);
    if constexpr (!SAVE) sched_fence();
    store_tile(sm[(kt + 1) & 1], nxt, tid, true, vsc);
    __syncthreads();
  }
  for (int kt = n_full; kt < n_kt; ++kt) {
    ld.load((kt + 1) * BN, true, nxt);
    if constexpr (!SAVE) sched_fence();
    pass2_tile<true, SAVE>(sm[kt & 1], kt * BN, krow, lane, qf1, qf2, c, lam, L1s, L2s, L2s2, o, o2, S, causal,
                           qw, my_q);
    if constexpr (!SAVE) sched_fence();
    store_tile(sm[(kt + 1) & 1], nxt, tid, true, vsc);
    __syncthreads();
  }

  // ---------------- epilogue: per-head RMSNorm x (1 - lambda_init) ----------------
  // o holds 2^(sg + vk) O; unscale exactly by powers of two.
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
  if (my_q < S) {
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
    if constexpr (SAVE) {
      const int64_t row = ((int64_t)b * S + my_q) * p.H + hd;
      float *op = p.o_pre + row * DV;
      float *ap = p.a2 + row * DV;
      const float un2 = __builtin_ldexpf(1.f, -vk) * fast_exp2(-sg2);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ch = ct * 32 + 8 * g + 4 * h;
          *(f32x4 *)(op + ch) = f32x4{o[ct][4 * g], o[ct][4 * g + 1], o[ct][4 * g + 2], o[ct][4 * g + 3]} * unscale;
          *(f32x4 *)(ap + ch) = f32x4{o2[ct][4 * g], o2[ct][4 * g + 1], o2[ct][4 * g + 2], o2[ct][4 * g + 3]} * un2;
        }
      if (h == 0) {
        const int64_t si = ((int64_t)b * p.H + hd) * S + my_q;
        p.lse1[si] = L1 * kLn2;
        p.lse2[si] = L2 * kLn2;
        p.rstd[si] = rstd;
      }
    }
  }
}

}  // namespace

size_t fwd_mfma_workspace_bytes(int B, int S, int H, bool training) {
  return training ? vrange_bytes(B, S, H) : vconv_bytes(B, S, H);
}

hipError_t launch_fwd_mfma(const FwdParams &p0, void *workspace, hipStream_t st) {
  FwdParams p = p0;
  if (!p.lse1) {  // inference: the one-pass kernel reads a converted fp16 copy of V
    VConvParams vc{p.v, p.vs_b, p.vs_s, p.vs_h, p.B, p.S, p.H, static_cast<f16 *>(workspace), nullptr};
    vc.kexp = reinterpret_cast<int *>(static_cast<char *>(workspace) +
                                      (((size_t)p.B * p.H * p.S * DV * 2 + 255) & ~(size_t)255));
    hipError_t e = launch_vconv(vc, st);
    if (e != hipSuccess) return e;
    p.v16 = vc.v16;
    p.vexp = vc.kexp;
    return launch_fwd_onepass(p, st);
  }
  p.vpart = static_cast<const unsigned *>(workspace);
  VRangeParams vr{p.v, p.vs_b, p.vs_s, p.vs_h, p.B, p.S, p.H, static_cast<unsigned *>(workspace)};
  hipError_t e = launch_vrange(vr, DV, st);
  if (e != hipSuccess) return e;
  const int n_qt = (p.S + BM - 1) / BM;
  dim3 grid(n_qt * p.B * p.H), block(NT);
  hipLaunchKernelGGL(fwd_mfma_kernel<true>, grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace diffattn
