// DIFF V2 prefill forward on gfx950 matrix cores: bf16 storage, head width
// D = 128 for queries, keys and values.
//
// The operator (tistory page on DIFF V2, section "DIFF V2 innovations" items
// 1, 2 and 5; section "GQA compatibility"): 2h query heads over h KV heads with
// grouped-query attention; every query head runs ordinary softmax attention
// (scale 1/sqrt(D), causal: query i sees keys j <= i); heads are then split
// into even and odd along the head axis and each pair (2p, 2p + 1), which
// shares one KV head, is combined per token as
//   out[i, p] = attn_2p[i] - sigmoid(lambda[i, p]) attn_2p+1[i],
// with no per-head normalisation.
//
// Work split.  One workgroup of 4 waves owns 128 query rows of one (batch,
// pair); wave w owns rows 32 w .. 32 w + 31 of both query heads of the pair,
// whose two maps read the same K and V tiles (one staged tile serves both).
// Causal tiles are issued longest first; consecutive workgroup ids walk the
// (batch, pair) index.
//
// Two passes over 64-key tiles staged through LDS (double-buffered, raw buffer
// loads, one barrier per tile), as in the V1 forward: pass 1 computes each
// map's log2 partition function per row; pass 2 recomputes the scores, forms
// the combined weight W = 2^(s_e c - L_e) - sigmoid(lambda) 2^(s_o c - L_o) in
// float32, scales it by a power of two ((1 + sigmoid(lambda)) 2^sigma just
// under 2^15, a head's weights being at most 1), rounds it once to fp16 and accumulates W V with fp16 V.  Rounding the
// combined weight keeps the error proportional to the combined map when
// sigmoid(lambda) is near 1 and the two heads nearly cancel.  Scores are
// computed transposed (S^T = K Q^T, lane = query); K rows are read in the
// permuted order of the shared tile helpers so a lane's score registers are
// the k-slots of the PV step; V^T comes through LDS transpose reads.
#include <cstddef>
#include <type_traits>

#include "attn_tile.h"
#include "kernels.h"
#include "vrange.h"

namespace diffattn {
namespace {

constexpr int D = 128, BM = 128, BN = 64, NT = 256;
constexpr int kMaxBlocks = 1024;  // key tiles a sparse query tile may list (64K keys)
constexpr int KST = D + 8;   // LDS row stride of the K tile, bf16 elements (272 B)
constexpr int VST = D + 32;  // LDS row stride of the V tile, fp16 elements (320 B)

struct SmemV2 {
  bf16 k[BN * KST];
  f16 v[BN * VST];  // V tile converted to fp16
};

// One thread's share of a staged tile: four 16-byte chunks of K and four of V.
struct TileRegsV2 {
  u32x4 k[4], v[4];
};

// Global -> register staging through raw buffer loads whose range ends at the
// (batch, KV head) slice's last key row (rows past the end read as zeros).
struct LoaderV2 {
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t off[4];  // this thread's byte offsets inside a tile (K and V alike)
  uint32_t step;    // bytes per key row

  __device__ __forceinline__ void init(const bf16 *k, const bf16 *v, int64_t kvs, int S, int tid) {
    const uint32_t bytes = (uint32_t)((int64_t)(S - 1) * kvs * 2 + D * 2);
    rk = __builtin_amdgcn_make_buffer_rsrc((void *)k, 0, bytes, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void *)v, 0, bytes, 0x00020000);
    step = (uint32_t)(kvs * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) off[i] = (uint32_t)((tid >> 4) + 16 * i) * step + (tid & 15) * 16;
  }

  __device__ __forceinline__ void load(int kbase, bool with_v, TileRegsV2 &r) const {
    const uint32_t b = (uint32_t)kbase * step;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(off[i] + b), 0, 0));
      if (with_v)
        r.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(off[i] + b), 0, 0));
    }
  }
};

__device__ __forceinline__ void store_tile(SmemV2 &sm, const TileRegsV2 &r, int tid, bool with_v,
                                           const VScale &vsc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 4) + 16 * i, col = (tid & 15) * 8;
    *(u32x4 *)(sm.k + row * KST + col) = r.k[i];
    if (with_v) {
      const u32x4 h = bf16x8_to_f16x8_scaled(r.v[i], vsc);
      *(u32x4 *)(sm.v + row * VST + col) = h;
    }
  }
}

// S^T sub-tile (32 keys x 32 queries) of both heads of the pair: one K
// operand per step serves the even and the odd head.
__device__ __forceinline__ void scores2(const SmemV2 &sm, int sub, int krow, int h, const bf16x8 *qe,
                                        const bf16x8 *qo, f32x16 &se, f32x16 &so) {
  const bf16 *a = sm.k + (sub * 32 + krow) * KST + 8 * h;
  se = f32x16{};
  so = f32x16{};
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    const bf16x8 ka = *(const bf16x8 *)(a + kc * 16);
    se = mfma32(ka, qe[kc], se);
    so = mfma32(ka, qo[kc], so);
  }
}

template <bool MASKED>
__device__ __forceinline__ void pass1_tile(const SmemV2 &sm, int kbase, int krow, int h, const bf16x8 *qe,
                                           const bf16x8 *qo, float c, float &me, float &le, float &mo, float &lo,
                                           int S, bool causal, int qw, int my_q) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int sb = kbase + sub * 32;
    if (MASKED && (sb >= S || (causal && sb > qw + 31))) continue;
    f32x16 se, so;
    scores2(sm, sub, krow, h, qe, qo, se, so);
    if (MASKED && ((causal && sb + 31 > qw) || sb + 32 > S)) mask_scores(se, so, sb, h, S, causal, my_q);
    lse_update(se, c, me, le);
    lse_update(so, c, mo, lo);
  }
}

template <bool MASKED, bool SAVE>
__device__ __forceinline__ void pass2_tile(const SmemV2 &sm, int kbase, int krow, int lane, const bf16x8 *qe,
                                           const bf16x8 *qo, float c, float sig, float Les, float Los, float fe,
                                           float fo, f32x16 *o, f32x16 *ae, f32x16 *ao, int S, bool causal, int qw,
                                           int my_q) {
  const int h = lane >> 5;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int sb = kbase + sub * 32;
    if (MASKED && (sb >= S || (causal && sb > qw + 31))) continue;
    f32x16 se, so;
    scores2(sm, sub, krow, h, qe, qo, se, so);
    if (MASKED && ((causal && sb + 31 > qw) || sb + 32 > S)) mask_scores(se, so, sb, h, S, causal, my_q);
    float w[16], we[16], wo[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float xe = fast_exp2(fmaf(se[r], c, -Les)), xo = fast_exp2(fmaf(so[r], c, -Los));
      w[r] = xe - sig * xo;
      if (SAVE) {
        we[r] = xe * fe;
        wo[r] = xo * fo;
      }
    }
    const f16x8 wb[2] = {pack8(w), pack8(w + 8)};
    pv_step_tile<VST, D / 32>(sm.v, sub, lane, wb, o);
    if (SAVE) {
      const f16x8 web[2] = {pack8(we), pack8(we + 8)}, wob[2] = {pack8(wo), pack8(wo + 8)};
      pv_step_tile<VST, D / 32>(sm.v, sub, lane, web, ae);
      pv_step_tile<VST, D / 32>(sm.v, sub, lane, wob, ao);
    }
  }
}

// Training mode (SAVE) also accumulates each head's own output A_even, A_odd
// with its own fp16 weights and writes, per row, both heads' natural-log
// partition functions and both outputs in float32: the backward needs
// g . A_t of each head consistent with that head's probabilities.
template <bool SAVE>
__global__ __launch_bounds__(NT, SAVE ? 1 : 2) void fwd_v2_kernel(V2FwdParams p) {
  // With SAVE (one workgroup per CU) a third buffer lets pass 2 run as a
  // software pipeline (see there).
  __shared__ SmemV2 sm[SAVE ? 3 : 2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave tests become scalar branches
  const int ln = lane & 31, h = lane >> 5;
  const int npair = p.Hq / 2;
  const int BP = p.B * npair;
  const int n_qt = (p.S + BM - 1) / BM;
  const int bp = blockIdx.x % BP;
  const int qt_i = blockIdx.x / BP;
  const int qt = p.causal ? n_qt - 1 - qt_i : qt_i;
  const int b = bp / npair, pr = bp % npair;
  const int te = 2 * pr, j = te / (p.Hq / p.Hkv);  // even head and the pair's KV head
  const int q0 = qt * BM, qw = q0 + wave * 32, my_q = qw + ln;
  const int S = p.S;
  const bool causal = p.causal != 0;
  const bool qok = my_q < S;
  const float c = p.scale * kLog2e;
  const float lam = qok ? p.lam[b * p.ls_b + (int64_t)my_q * p.ls_s + pr * p.ls_p] : 0.f;
  const float sig = 1.f / (1.f + expf(-lam));

  LoaderV2 ld;
  ld.init((const bf16 *)p.k + b * p.kvs_b + j * p.kvs_h, (const bf16 *)p.v + b * p.kvs_b + j * p.kvs_h, p.kvs_s, S,
          tid);

  bf16x8 qe[D / 16], qo[D / 16];
  {
    const bf16 *q = (const bf16 *)p.q + b * p.qs_b + (int64_t)my_q * p.qs_s + 8 * h;
    const bf16 *qev = q + te * p.qs_h, *qov = q + (te + 1) * p.qs_h;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qe[kc] = qok ? *(const bf16x8 *)(qev + kc * 16) : bf16x8{};
      qo[kc] = qok ? *(const bf16x8 *)(qov + kc * 16) : bf16x8{};
    }
  }

  const int kend = causal ? min(S, q0 + BM) : S;
  const int n_kt = (kend + BN - 1) / BN;
  const int n_full = min(causal ? (q0 + 1) / BN : n_kt, S / BN);
  const int krow = k_row_perm(ln);
  // fp16 V is V 2^vk (range of bf16; see vrange.h); the epilogue removes it.
  const int vk = v_shift(p.vpart + ((int64_t)b * p.Hkv + j) * vrange_chunks(S), vrange_chunks(kend));
  const VScale vsc(vk);
  const float unv = __builtin_ldexpf(1.f, -vk);

  // ---------------- pass 1: per-head log2 partition functions ----------------
  float me = kNegInf, le = 0.f, mo = kNegInf, lo = 0.f;
  TileRegsV2 nxt;
  ld.load(0, false, nxt);
  store_tile(sm[0], nxt, tid, false, vsc);
  __syncthreads();
  for (int kt = 0; kt < n_full; ++kt) {
    ld.load((kt + 1) * BN, false, nxt);  // past the end: the buffer range gives zeros
    sched_fence();
    pass1_tile<false>(sm[kt & 1], kt * BN, krow, h, qe, qo, c, me, le, mo, lo, S, causal, qw, my_q);
    sched_fence();
    store_tile(sm[(kt + 1) & 1], nxt, tid, false, vsc);
    __syncthreads();
  }
  for (int kt = n_full; kt < n_kt; ++kt) {
    ld.load((kt + 1) * BN, false, nxt);
    sched_fence();
    pass1_tile<true>(sm[kt & 1], kt * BN, krow, h, qe, qo, c, me, le, mo, lo, S, causal, qw, my_q);
    sched_fence();
    store_tile(sm[(kt + 1) & 1], nxt, tid, false, vsc);
    __syncthreads();
  }
  float Me, Le, Mo, Lo;
  lse_finish(me, le, Me, Le);
  lse_finish(mo, lo, Mo, Lo);
  // A head's weights are at most 1, so |W| <= 1 + sigma(lambda).
  const float sg = row_scale_log2(1.f + sig);
  const float Les = Le - sg, Los = Lo - sg;
  // Each head's own weights (at most 1) scaled just under 2^15 for A_even and A_odd.
  const float sge = SAVE ? row_scale_log2(1.f) : 0.f;
  const float sgo = SAVE ? row_scale_log2(1.f) : 0.f;
  const float fe = fast_exp2(sge - sg), fo = fast_exp2(sgo - sg);

  // ---------------- pass 2: O = (P_e - sigmoid(lambda) P_o) V ----------------
  f32x16 o[D / 32], ae[SAVE ? D / 32 : 1], ao[SAVE ? D / 32 : 1];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) o[ct] = f32x16{};
#pragma unroll
  for (int ct = 0; ct < (SAVE ? D / 32 : 1); ++ct) ae[ct] = ao[ct] = f32x16{};
  ld.load(0, true, nxt);
  store_tile(sm[0], nxt, tid, true, vsc);
  __syncthreads();
  constexpr int NB = SAVE ? 3 : 2;  // pass-2 buffers: tile kt in buffer kt % NB
  if constexpr (!SAVE) {
    for (int kt = 0; kt < n_full; ++kt) {
      ld.load((kt + 1) * BN, true, nxt);
      sched_fence();
      pass2_tile<false, SAVE>(sm[kt & 1], kt * BN, krow, lane, qe, qo, c, sig, Les, Los, fe, fo, o, ae, ao, S, causal,
                              qw, my_q);
      sched_fence();
      store_tile(sm[(kt + 1) & 1], nxt, tid, true, vsc);
      __syncthreads();
    }
  } else if (n_full > 0) {
    // The unmasked tiles as a software pipeline over 32-key sub-tiles.  Step
    // j, in two halves: the score products of sub-tile j beside the weights
    // of sub-tile j - 1 (from its carried exponentials), then the three PV
    // products of j - 1 beside the exponentials of j; one matrix instruction
    // and a share of the vector work at a time behind scheduling fences (the
    // single wave on each SIMD issues in order, so that order is what
    // overlaps the two units).  LDS operands are read two instructions ahead
    // from per-step base addresses.  Staging: the even step 2m stores the K
    // half of tile m + 1, the odd step its V half (then a barrier); each then
    // loads the same half of tile m + 2.  Tile m is complete from the end of
    // step 2m - 1 and last read in step 2m + 2.
    typedef DA_LDS const char lchar;
    const int jj = lane & 15, half16 = (lane >> 4) & 1;
    const uint32_t laK = (krow * KST + 8 * h) * 2;
    const uint32_t lcV = ((8 * h + (jj >> 2)) * VST + 16 * half16 + 4 * (jj & 3)) * 2;
    constexpr uint32_t OK = offsetof(SmemV2, k), OV = offsetof(SmemV2, v);
    auto lptr = [&](int buf, uint32_t lane_off) -> lchar * {
      lchar *q = (lchar *)(sm + buf) + lane_off;
      asm volatile("" : "+v"(q));
      return q;
    };
    // Staging halves: K (part 0, bf16 as loaded) and V (part 1, to fp16).
    auto load_part = [&](int t, int part, u32x4 *r) {
      const uint32_t tb = (uint32_t)(t * BN) * ld.step;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(part == 0 ? ld.rk : ld.rv, (int)(ld.off[i] + tb), 0, 0));
    };
    auto store_part = [&](int t, int part, const u32x4 *r) {
      SmemV2 &st = sm[t % NB];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 4) + 16 * i, col = (tid & 15) * 8;
        if (part == 0) *(u32x4 *)(st.k + row * KST + col) = r[i];
        else *(u32x4 *)(st.v + row * VST + col) = bf16x8_to_f16x8_scaled(r[i], vsc);
      }
    };
    u32x4 hreg[2][4];
    if (1 < n_kt) {
      load_part(1, 0, hreg[0]);
      load_part(1, 1, hreg[1]);
    }
    struct Carry {
      float xe[16], xo[16];  // each head's weight, exp2(s c - L)
    };
    Carry cr[2];
    f16x8 wb[2], web[2], wob[2];  // PV operands of the previous sub-tile

    auto step = [&](auto has_prev, auto has_cur, auto parity, int j, const Carry &prv, Carry &cur) {
      constexpr bool HP = decltype(has_prev)::value;  // sub-tile j - 1 exists
      constexpr bool HJ = decltype(has_cur)::value;   // sub-tile j exists
      constexpr int SUB = decltype(parity)::value;    // j % 2
      constexpr int SUBP = 1 - SUB;
      const int t = j >> 1;
      lchar *pK = nullptr, *pV = nullptr;
      if constexpr (HJ) pK = lptr(t % NB, laK);
      if constexpr (HP) pV = lptr(((j - 1) >> 1) % NB, lcV);
      auto fk = [&](int kc) -> bf16x8 { return *(const DA_LDS bf16x8 *)(pK + OK + (SUB * 32 * KST + kc * 16) * 2); };
      // PV operand i (0..7) of sub-tile j - 1: keys 16 (i / 4), channels 32 (i % 4).
      auto fv = [&](int i) -> f16x8 {
        const uint32_t off = OV + ((SUBP * 32 + (i >> 2) * 16) * VST + (i & 3) * 32) * 2;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(pV + off));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(pV + off + 8 * VST));
        const f16x4 a = __builtin_bit_cast(f16x4, lo), bb = __builtin_bit_cast(f16x4, hi);
        return f16x8{a[0], a[1], a[2], a[3], bb[0], bb[1], bb[2], bb[3]};
      };
      bf16x8 ok_[8];
      f16x8 ov[8];
      f32x16 se = {}, so = {};
      if constexpr (HJ) {
        ok_[0] = fk(0);
        ok_[1] = fk(1);
      }
      // Half 1: score products of j (K operand m / 2, heads alternating) with
      // the weights of j - 1.
      float pw[2][3];  // one pair of weights awaiting conversion
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        if constexpr (HJ) {
          const int kc = m >> 1;
          if (!(m & 1) && kc + 2 < 8) ok_[kc + 2] = fk(kc + 2);
          if (m & 1) so = mfma32(ok_[kc], qo[kc], so);
          else se = mfma32(ok_[kc], qe[kc], se);
        }
        if constexpr (HP) {
          if (m >= 14) ov[m - 14] = fv(m - 14);
          const int r = m;
          const float xe = prv.xe[r], xo = prv.xo[r];
          pw[r & 1][0] = xe - sig * xo;
          pw[r & 1][1] = xe * fe;
          pw[r & 1][2] = xo * fo;
          if (r & 1) {
            const int kc2 = r >> 3, e = r & 7;
            f16x2 a = __builtin_convertvector((f32x2{pw[0][0], pw[1][0]}), f16x2);
            f16x2 bb = __builtin_convertvector((f32x2{pw[0][1], pw[1][1]}), f16x2);
            f16x2 d = __builtin_convertvector((f32x2{pw[0][2], pw[1][2]}), f16x2);
            asm volatile("" : "+v"(a), "+v"(bb), "+v"(d));  // computed here, not at first use
            wb[kc2][e - 1] = a[0];
            wb[kc2][e] = a[1];
            web[kc2][e - 1] = bb[0];
            web[kc2][e] = bb[1];
            wob[kc2][e - 1] = d[0];
            wob[kc2][e] = d[1];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Half 2: the PV products of j - 1 (operand m / 3: O, A_even, A_odd)
      // with the exponentials of j.
#pragma unroll
      for (int m = 0; m < 24; ++m) {
        if constexpr (HP) {
          const int i = m / 3, kind = m % 3, kc2 = i >> 2, ct = i & 3;
          if (kind == 0 && i + 2 < 8) ov[i + 2] = fv(i + 2);
          if (kind == 0) o[ct] = mfma32(ov[i], wb[kc2], o[ct]);
          else if (kind == 1) ae[ct] = mfma32(ov[i], web[kc2], ae[ct]);
          else ao[ct] = mfma32(ov[i], wob[kc2], ao[ct]);
        }
        if constexpr (HJ) {
          if (m < 16) {
            const int r = m;
            cur.xe[r] = fast_exp2(fmaf(se[r], c, -Les));
            cur.xo[r] = fast_exp2(fmaf(so[r], c, -Los));
            asm volatile("" : "+v"(cur.xe[r]), "+v"(cur.xo[r]));
          }
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
    const int J = 2 * n_full;
    step(F{}, T{}, P0{}, 0, cr[1], cr[0]);
    for (int j = 1; j < J - 1; j += 2) {
      step(T{}, T{}, P1{}, j, cr[0], cr[1]);
      step(T{}, T{}, P0{}, j + 1, cr[1], cr[0]);
    }
    step(T{}, T{}, P1{}, J - 1, cr[0], cr[1]);
    step(T{}, F{}, P0{}, J, cr[1], cr[0]);  // the last sub-tile's weights and PV products
  }
  for (int kt = n_full; kt < n_kt; ++kt) {
    ld.load((kt + 1) * BN, true, nxt);
    if constexpr (!SAVE) sched_fence();
    pass2_tile<true, SAVE>(sm[kt % NB], kt * BN, krow, lane, qe, qo, c, sig, Les, Los, fe, fo, o, ae, ao, S, causal, qw,
                           my_q);
    if constexpr (!SAVE) sched_fence();
    store_tile(sm[(kt + 1) % NB], nxt, tid, true, vsc);
    __syncthreads();
  }

  // ---------------- epilogue: unscale, store bf16 (and the training saves) ----------------
  if (qok) {
    const float f = fast_exp2(-sg) * unv;
    bf16 *out = (bf16 *)p.out + b * p.os_b + (int64_t)my_q * p.os_s + pr * p.os_h;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = ct * 32 + 8 * g + 4 * h;
        const bf16x4 y = {f2bf(o[ct][4 * g] * f), f2bf(o[ct][4 * g + 1] * f), f2bf(o[ct][4 * g + 2] * f),
                          f2bf(o[ct][4 * g + 3] * f)};
        *(bf16x4 *)(out + ch) = y;
      }
    if (SAVE) {
      if (h == 0) {
        const int64_t lr = ((int64_t)b * p.Hq + te) * S + my_q;
        p.lse[lr] = Le * kLn2;
        p.lse[lr + S] = Lo * kLn2;
      }
      const float fa = fast_exp2(-sge) * unv, fb = fast_exp2(-sgo) * unv;
      const int64_t srow = (((int64_t)b * S + my_q) * npair + pr) * D;
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ch = ct * 32 + 8 * g + 4 * h;
          *(f32x4 *)(p.a_even + srow + ch) = f32x4{ae[ct][4 * g] * fa, ae[ct][4 * g + 1] * fa,
                                                   ae[ct][4 * g + 2] * fa, ae[ct][4 * g + 3] * fa};
          *(f32x4 *)(p.a_odd + srow + ch) = f32x4{ao[ct][4 * g] * fb, ao[ct][4 * g + 1] * fb,
                                                  ao[ct][4 * g + 2] * fb, ao[ct][4 * g + 3] * fb};
        }
    }
  }
}

// Block-sparse variant (one key-block selection per even/odd pair: sparse
// attention frameworks select blocks per head pair inside a GQA group, tistory
// page on DIFF V2, section on practical considerations).  The caller lists,
// per (batch, pair, 128-row query tile), the 64-key tiles the pair may attend
// (ascending); each head's softmax runs over the listed keys (with the causal
// mask inside them), every other weight being zero.  Entries outside the
// sequence, past the query tile (causal) or not above the previous accepted
// entry are skipped; a row that sees no key gets zeros.  Same two passes
// and staging as the dense kernel, walking the list instead of 0..n: the
// listed tiles that no row of the workgroup needs masked first, without mask
// arithmetic, then the rest.
__global__ __launch_bounds__(NT, 2) void fwd_v2_sparse_kernel(V2FwdParams p) {
  __shared__ SmemV2 sm[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, h = lane >> 5;
  const int npair = p.Hq / 2;
  const int BP = p.B * npair;
  const int n_qt = (p.S + BM - 1) / BM;
  const int bp = blockIdx.x % BP;
  const int qt_i = blockIdx.x / BP;
  const int qt = p.causal ? n_qt - 1 - qt_i : qt_i;
  const int b = bp / npair, pr = bp % npair;
  const int te = 2 * pr, j = te / (p.Hq / p.Hkv);
  const int q0 = qt * BM, qw = q0 + wave * 32, my_q = qw + ln;
  const int S = p.S;
  const bool causal = p.causal != 0;
  const bool qok = my_q < S;
  const float c = p.scale * kLog2e;
  const float lam = qok ? p.lam[b * p.ls_b + (int64_t)my_q * p.ls_s + pr * p.ls_p] : 0.f;
  const float sig = 1.f / (1.f + expf(-lam));

  // This query tile's list of key tiles (read by every thread; uniform).
  const int64_t li = (int64_t)bp * n_qt + qt;
  const int cnt = min(min(max(p.blk_cnt[li], 0), p.max_blocks), kMaxBlocks);
  const int32_t *lst = p.blk_idx + li * p.max_blocks;
  const int n_ktot = (S + BN - 1) / BN;
  const int kt_lim = causal ? min(n_ktot, (q0 + BM + BN - 1) / BN) : n_ktot;  // tiles past the last row see nothing

  LoaderV2 ld;
  ld.init((const bf16 *)p.k + b * p.kvs_b + j * p.kvs_h, (const bf16 *)p.v + b * p.kvs_b + j * p.kvs_h, p.kvs_s, S,
          tid);

  bf16x8 qe[D / 16], qo[D / 16];
  {
    const bf16 *q = (const bf16 *)p.q + b * p.qs_b + (int64_t)my_q * p.qs_s + 8 * h;
    const bf16 *qev = q + te * p.qs_h, *qov = q + (te + 1) * p.qs_h;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qe[kc] = qok ? *(const bf16x8 *)(qev + kc * 16) : bf16x8{};
      qo[kc] = qok ? *(const bf16x8 *)(qov + kc * 16) : bf16x8{};
    }
  }
  const int krow = k_row_perm(ln);
  // The valid list entries (tile index in [0, kt_lim)), compacted into LDS.
  __shared__ int tiles[kMaxBlocks];
  __shared__ int n_tiles, n_open;
  // Tiles below n_full need no mask for any row of the workgroup (as in the
  // dense kernel); being ascending, they lead the compacted list.
  const int n_full = min(causal ? (q0 + 1) / BN : n_ktot, S / BN);
  for (int i = tid; i < cnt; i += NT) tiles[i] = lst[i];  // all threads fetch, one thread compacts in place
  __syncthreads();
  if (tid == 0) {  // ascending, in range; entries not above the last accepted one are ignored
    int n = 0, last = -1, m = 0;
    for (int i = 0; i < cnt; ++i) {
      const int t = tiles[i];
      if (t > last && t < kt_lim) {
        tiles[n++] = last = t;
        m += t < n_full;
      }
    }
    n_tiles = n;
    n_open = m;
  }
  __syncthreads();
  const int n_valid = __builtin_amdgcn_readfirstlane(n_tiles);
  const int n_unm = __builtin_amdgcn_readfirstlane(n_open);
  // fp16 V is V 2^vk over every key row the list may name (see vrange.h).
  const int vk = v_shift(p.vpart + ((int64_t)b * p.Hkv + j) * vrange_chunks(S), vrange_chunks(min(S, kt_lim * BN)));
  const VScale vsc(vk);

  // ---------------- pass 1 ----------------
  float me = kNegInf, le = 0.f, mo = kNegInf, lo = 0.f;
  TileRegsV2 nxt;
  ld.load((n_valid > 0 ? tiles[0] : 0) * BN, false, nxt);
  store_tile(sm[0], nxt, tid, false, vsc);
  __syncthreads();
  auto p1 = [&](auto masked, int n) {
    constexpr bool MASKED = decltype(masked)::value;
    const int cur = __builtin_amdgcn_readfirstlane(tiles[n]);
    const int nk = __builtin_amdgcn_readfirstlane(n + 1 < n_valid ? tiles[n + 1] : cur);
    ld.load(nk * BN, false, nxt);
    sched_fence();
    pass1_tile<MASKED>(sm[n & 1], cur * BN, krow, h, qe, qo, c, me, le, mo, lo, S, causal, qw, my_q);
    sched_fence();
    store_tile(sm[(n + 1) & 1], nxt, tid, false, vsc);
    __syncthreads();
  };
  {
    int n = 0;
    for (; n < n_unm; ++n) p1(std::false_type{}, n);
    for (; n < n_valid; ++n) p1(std::true_type{}, n);
  }
  float Me, Le, Mo, Lo;
  lse_finish(me, le, Me, Le);
  lse_finish(mo, lo, Mo, Lo);
  const bool live = Le != kNegInf;  // the row saw at least one key (both heads see the same keys)
  const float sg = live ? row_scale_log2(1.f + sig) : 0.f;
  const float Les = live ? Le - sg : __builtin_inff(), Los = live ? Lo - sg : __builtin_inff();

  // ---------------- pass 2 ----------------
  f32x16 o[D / 32], dummy[1];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) o[ct] = f32x16{};
  ld.load((n_valid > 0 ? tiles[0] : 0) * BN, true, nxt);
  store_tile(sm[0], nxt, tid, true, vsc);
  __syncthreads();
  auto p2 = [&](auto masked, int n) {
    constexpr bool MASKED = decltype(masked)::value;
    const int cur = __builtin_amdgcn_readfirstlane(tiles[n]);
    const int nk = __builtin_amdgcn_readfirstlane(n + 1 < n_valid ? tiles[n + 1] : cur);
    ld.load(nk * BN, true, nxt);
    sched_fence();
    pass2_tile<MASKED, false>(sm[n & 1], cur * BN, krow, lane, qe, qo, c, sig, Les, Los, 1.f, 1.f, o, dummy, dummy,
                              S, causal, qw, my_q);
    sched_fence();
    store_tile(sm[(n + 1) & 1], nxt, tid, true, vsc);
    __syncthreads();
  };
  {
    int n = 0;
    for (; n < n_unm; ++n) p2(std::false_type{}, n);
    for (; n < n_valid; ++n) p2(std::true_type{}, n);
  }

  if (qok) {
    const float f = live ? fast_exp2(-sg) * __builtin_ldexpf(1.f, -vk) : 0.f;
    bf16 *out = (bf16 *)p.out + b * p.os_b + (int64_t)my_q * p.os_s + pr * p.os_h;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = ct * 32 + 8 * g + 4 * h;
        const bf16x4 y = {f2bf(o[ct][4 * g] * f), f2bf(o[ct][4 * g + 1] * f), f2bf(o[ct][4 * g + 2] * f),
                          f2bf(o[ct][4 * g + 3] * f)};
        *(bf16x4 *)(out + ch) = y;
      }
  }
}

}  // namespace

hipError_t launch_fwd_v2(const V2FwdParams &p, hipStream_t st) {
  VRangeParams vr{p.v, p.kvs_b, p.kvs_s, p.kvs_h, p.B, p.S, p.Hkv, const_cast<unsigned *>(p.vpart)};
  hipError_t e = launch_vrange(vr, D, st);
  if (e != hipSuccess) return e;
  const int n_qt = (p.S + BM - 1) / BM;
  if (p.blk_idx)
    hipLaunchKernelGGL(fwd_v2_sparse_kernel, dim3(n_qt * p.B * (p.Hq / 2)), dim3(NT), 0, st, p);
  else if (p.lse)
    hipLaunchKernelGGL(fwd_v2_kernel<true>, dim3(n_qt * p.B * (p.Hq / 2)), dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL(fwd_v2_kernel<false>, dim3(n_qt * p.B * (p.Hq / 2)), dim3(NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace diffattn
