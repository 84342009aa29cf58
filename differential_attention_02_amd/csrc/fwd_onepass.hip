// One-pass causal/non-causal forward of multi-head differential attention on
// gfx950 matrix cores: bf16 storage, d = 64, dv = 128; inference, or with the
// training saves the backward reads (lse1, lse2, rstd, O, A2).
//
// The operator (glossary page "Differential Transformer", section "How
// differential attention works"; news write-up, multi-head section):
//   Y = RMSNorm_head((softmax(s Q1 K1^T) - lambda softmax(s Q2 K2^T)) V) (1 - lambda_init)
//
// One sweep over the keys with two running softmax states per query row.
// With per-map references m1, m2 (log2 domain) and e_m = 2^(s_m c - m_m), the
// kernel accumulates, per row,
//   l1 = sum e1,  l2 = sum e2,  X = sum (e1 - kappa e2) V,  Y = sum e2 V,
// and finishes with O = X / l1 + (kappa / l1 - lambda / l2) Y, which is exact
// for any kappa.  kappa is kept within 2^-7 of lambda l1 / l2 (when it drifts,
// X += (kappa_old - kappa_new) Y re-bases it), so the fp16-rounded weight
// e1 - kappa e2 is l1 (p1 - lambda' p2) with lambda' ~ lambda: its rounding
// error is proportional to the combined map rather than to each map, which
// matters when lambda is near 1 and the two maps cancel; the Y term enters
// only with a coefficient of at most ~2^-7 lambda / l2.  The references move
// lazily: a reference is raised to the sub-tile's top score only when that
// tops it by more than 2^8 (so no term exceeds 2^8), and by whole powers of
// two when a row's merged sum passes bnd = 2^14 / (1 + |lambda|) (many keys
// near the reference); X or Y, l and kappa are rescaled with it.  Bounding
// l1 and l2 by bnd keeps every weight inside fp16 (e_m <= l_m and
// |kappa e2| <~ |lambda| l1).
// Matrix-core work per (query, key) pair: 2 QK^T products of width 64 and
// 2 PV products of width 128 (768 flop); two exponentials.  The training
// variant keeps kappa at 0 and splits both weights into fp16 hi + lo halves
// (4 PV products, 1280 flop issued per pair), so the saved O and A2 carry
// about 2^-22 relative error rather than fp16's 2^-11.
//
// Work split.  One workgroup of 8 waves (two per SIMD) owns 256 query rows of
// one (batch, head); each wave owns a 32-row block, the two waves sharing a
// SIMD holding one early and one late block so the causal diagonal is shared
// out evenly, and the second of them running half a sub-tile behind the
// first (see the key loop).  Causal tiles are issued longest first and consecutive workgroup
// ids walk the (batch, head) index (workgroups are dealt round-robin to the 8
// XCDs, so a head's query tiles share one L2).
//
// Scores are computed transposed, S^T = K Q^T (keys on rows): a lane owns one
// query column and its score registers are already the B operand of the PV
// product O^T = V^T W^T (K rows read in the permuted order of the shared tile
// helpers).  The two half-waves hold disjoint keys of the same rows; every
// decision (references, kappa) is taken on merged sums, so both halves agree.
// V comes from an fp16 copy written by a pass over V (vrange.hip) with one
// power-of-two shift per 256-row chunk, so V may take any finite bf16
// magnitude.
#include "attn_tile.h"
#include "kernels.h"
#include "vrange.h"

namespace diffattn {
namespace {

constexpr int D = 64, DV = 128, BN = 64, NW = 8, NT = 64 * NW, OBM = 32 * NW;
constexpr int NBUF = 3;  // LDS tile buffers
constexpr int KST = D + 8;   // LDS row stride of a K tile, bf16 elements (144 B)
constexpr int VST = DV + 32; // LDS row stride of the V tile, fp16 elements (320 B)

struct Smem {
  bf16 k1[BN * KST];
  bf16 k2[BN * KST];
  f16 v[BN * VST];
};

// One thread's share of a 64-key tile: KC 16-byte chunks of K1 and of K2,
// VC of V.
constexpr int KC = 8 * BN / NT, VC = 16 * BN / NT;
struct Stage {
  u32x4 k1[KC], k2[KC], v[VC];
};

// Raw buffer loads (K1, K2 bf16; V from its fp16 copy); each slice's buffer
// range ends at its last key row, so rows past the sequence end read as zeros.
struct Loader {
  __amdgpu_buffer_rsrc_t rk1, rk2, rv;
  uint32_t ko, vo;        // this thread's byte offsets inside a tile
  uint32_t kstep, vstep;  // bytes per key row

  __device__ __forceinline__ void init(const bf16 *k1, const bf16 *k2, const f16 *v, int64_t ks, int64_t vs,
                                       int S, int tid) {
    const uint32_t kbytes = (uint32_t)((int64_t)(S - 1) * ks * 2 + D * 2);
    const uint32_t vbytes = (uint32_t)((int64_t)(S - 1) * vs * 2 + DV * 2);
    rk1 = __builtin_amdgcn_make_buffer_rsrc((void *)k1, 0, kbytes, 0x00020000);
    rk2 = __builtin_amdgcn_make_buffer_rsrc((void *)k2, 0, kbytes, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void *)v, 0, vbytes, 0x00020000);
    kstep = (uint32_t)(ks * 2);
    vstep = (uint32_t)(vs * 2);
    ko = (uint32_t)(tid >> 3) * kstep + (tid & 7) * 16;
    vo = (uint32_t)(tid >> 4) * vstep + (tid & 15) * 16;
  }

  __device__ __forceinline__ void load(int kbase, Stage &r) const {
    const uint32_t kb = (uint32_t)kbase * kstep, vb = (uint32_t)kbase * vstep;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int o = (int)(ko + kb + i * (NT / 8) * kstep);
      r.k1[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk1, o, 0, 0));
      r.k2[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk2, o, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < VC; ++i)
      r.v[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(vo + vb + i * (NT / 16) * vstep), 0, 0));
  }
};

__device__ __forceinline__ void store_stage(Smem &sm, const Stage &r, int tid) {
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int row = (tid >> 3) + i * (NT / 8), col = (tid & 7) * 8;
    *(u32x4 *)(sm.k1 + row * KST + col) = r.k1[i];
    *(u32x4 *)(sm.k2 + row * KST + col) = r.k2[i];
  }
#pragma unroll
  for (int i = 0; i < VC; ++i) {
    const int row = (tid >> 4) + i * (NT / 16), col = (tid & 15) * 8;
    *(u32x4 *)(sm.v + row * VST + col) = r.v[i];
  }
}

// Running state of one query row, held by both lanes of the row (the
// references and kappa are identical in the two; l1, l2 are each lane's share).
struct RowState {
  float m1, m2, l1, l2, kap;
};

// e[r] = 2^(s[r] c - m); returns the lane's sum.
__device__ __forceinline__ float exps16(const f32x16 &s, float c, float m, float *e) {
  float a[4];
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] = fast_exp2(fmaf(s[r], c, -m));
#pragma unroll
  for (int r = 0; r < 4; ++r) a[r] = (e[r] + e[r + 4]) + (e[r + 8] + e[r + 12]);
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// S^T of one map over one 32-key sub-tile.
__device__ __forceinline__ f32x16 score_map(const bf16 *ktile, int sub, int krow, int h, const bf16x8 *qf) {
  const bf16 *a = ktile + (sub * 32 + krow) * KST + 8 * h;
  f32x16 s = {};
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) s = mfma32(*(const bf16x8 *)(a + kc * 16), qf[kc], s);
  return s;
}

// Merged (both half-waves) top scaled score of one map's sub-tile.
__device__ __forceinline__ float top_score(const f32x16 &s, float c) {
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx *= c;
  return fmaxf(mx, other_half(mx));
}

// Moves a reference to mn >= m; returns the factor for what was accumulated
// against the old one (0 when it was -inf: nothing was).
__device__ __forceinline__ float move_ref(float &m, float mn) {
  const float a = m == kNegInf ? 0.f : fast_exp2(m - mn);
  m = mn;
  return a;
}

// Scores of both maps over one 32-key sub-tile and the softmax bookkeeping;
// returns the fp16 B operands of the sub-tile's two PV products
// (w = e1 - kappa e2, and e2).  With SAVE kappa stays 0 (X = sum e1 V) and
// each weight is split into fp16 hi + lo halves (wb, eb the hi halves; wl, el
// the lo halves), so X and Y, and with them the saved O and A2, are
// accurate to about 2^-22 relative: the backward's lambda gradient sums
// g . A2 over every row with heavy cancellation.
template <bool MASKED, bool SAVE>
__device__ __forceinline__ void sub_softmax(const Smem &sm, int sub, int sb, int krow, int lane, const bf16x8 *q1f,
                                            const bf16x8 *q2f, float c, float lam, float bnd, RowState &st,
                                            f32x16 *x, f32x16 *y, int S, bool causal, int my_q, f16x8 *wb,
                                            f16x8 *eb, f16x8 *wl, f16x8 *el) {
  const int h = lane >> 5;
  f32x16 s1 = score_map(sm.k1, sub, krow, h, q1f);
  f32x16 s2 = score_map(sm.k2, sub, krow, h, q2f);
  if constexpr (MASKED) {
    mask_scores1(s1, sb, h, S, causal, my_q);
    mask_scores1(s2, sb, h, S, causal, my_q);
  }
  // A reference moves only when a score tops it by more than 2^8 (or there is
  // none yet), so no term exceeds 2^8.
  const float mx1 = top_score(s1, c), mx2 = top_score(s2, c);
  if (mx1 > st.m1 + 8.f || mx2 > st.m2 + 8.f) {  // rare; both lanes of a row agree
    const float a1 = mx1 > st.m1 + 8.f ? move_ref(st.m1, mx1) : 1.f;
    const float a2 = mx2 > st.m2 + 8.f ? move_ref(st.m2, mx2) : 1.f;
    st.l1 *= a1;
    st.l2 *= a2;
    // Fold kappa Y back into X first (X becomes sum e1 V, kappa 0): scaling
    // kappa by 1 / a2 instead could overflow when map 2's reference jumps far.
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      x[ct] = (x[ct] + st.kap * y[ct]) * a1;
      y[ct] *= a2;
    }
    st.kap = 0.f;
  }
  float e1[16], e2[16];
  float t1 = exps16(s1, c, st.m1 == kNegInf ? 0.f : st.m1, e1);
  float t2 = exps16(s2, c, st.m2 == kNegInf ? 0.f : st.m2, e2);
  float L1 = st.l1 + t1, L2 = st.l2 + t2;
  L1 += other_half(L1);
  L2 += other_half(L2);
  if (L1 > bnd || L2 > bnd) {  // rare; both lanes of a row agree (merged sums)
    // Many keys near the reference: raising it by whole powers of two (an
    // exact rescale) brings the merged sum to at most bnd / 2.
    if (L1 > bnd) {
      const float k = ceilf(log2f(L1 / bnd)) + 1.f, f = fast_exp2(-k);
#pragma unroll
      for (int r = 0; r < 16; ++r) e1[r] *= f;
      t1 *= f;
      st.l1 *= f;
      st.kap *= f;
      st.m1 += k;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) x[ct] *= f;
    }
    if (L2 > bnd) {
      const float k = ceilf(log2f(L2 / bnd)) + 1.f, f = fast_exp2(-k);
#pragma unroll
      for (int r = 0; r < 16; ++r) e2[r] *= f;
      t2 *= f;
      st.l2 *= f;
      st.kap *= fast_exp2(k);
      st.m2 += k;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) y[ct] *= f;
    }
    L1 = st.l1 + t1;
    L2 = st.l2 + t2;
    L1 += other_half(L1);
    L2 += other_half(L2);
  }
  st.l1 += t1;
  st.l2 += t2;
  if constexpr (SAVE) {
    pack8_hilo(e1, wb[0], wl[0]);
    pack8_hilo(e1 + 8, wb[1], wl[1]);
    pack8_hilo(e2, eb[0], el[0]);
    pack8_hilo(e2 + 8, eb[1], el[1]);
    return;
  }
  // kappa tracks lambda L1 / L2 (merged sums including this sub-tile).
  const float ks = L2 > 0.f ? lam * L1 * __builtin_amdgcn_rcpf(L2) : 0.f;
  if (fabsf(ks - st.kap) > 0x1p-7f * fabsf(ks)) {
    const float d = st.kap - ks;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) x[ct] += d * y[ct];
    st.kap = ks;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) e1[r] = fmaf(-st.kap, e2[r], e1[r]);
  wb[0] = pack8(e1);
  wb[1] = pack8(e1 + 8);
  eb[0] = pack8(e2);
  eb[1] = pack8(e2 + 8);
}

// X^T += V^T W^T and Y^T += V^T E^T over one sub-tile (with SAVE, the hi
// and lo halves of both weights: four products per V operand).
template <bool SAVE>
__device__ __forceinline__ void sub_pv(const Smem &sm, int sub, int lane, const f16x8 *wb, const f16x8 *eb,
                                       const f16x8 *wl, const f16x8 *el, f32x16 *x, f32x16 *y) {
  const int h = lane >> 5, j = lane & 15, half16 = (lane >> 4) & 1;
#pragma unroll
  for (int kc2 = 0; kc2 < 2; ++kc2) {
    const int key0 = sub * 32 + kc2 * 16 + 8 * h + (j >> 2);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f16 *p = sm.v + key0 * VST + ct * 32 + 16 * half16 + 4 * (j & 3);
      const f16x4 lo = lds_read_tr16(p);
      const f16x4 hi = lds_read_tr16(p + 4 * VST);
      const f16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      x[ct] = mfma32(va, wb[kc2], x[ct]);
      y[ct] = mfma32(va, eb[kc2], y[ct]);
      if constexpr (SAVE) {
        x[ct] = mfma32(va, wl[kc2], x[ct]);
        y[ct] = mfma32(va, el[kc2], y[ct]);
      }
    }
  }
}

// Moves the accumulators from V 2^vk products to V 2^(vk + dk) products.
__device__ __forceinline__ void rescale_acc(f32x16 *x, f32x16 *y, int dk, int &vk) {
  const float f = __builtin_ldexpf(1.f, dk);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    x[ct] *= f;
    y[ct] *= f;
  }
  vk += dk;
}

// SAVE also writes the training saves: lse_m = (m_m + log2 L_m) ln 2, the
// pre-norm output O, A2 = Y / L2 (the second map's attention output) and the
// RMSNorm's rstd.
template <bool SAVE>
__global__ __launch_bounds__(NT, 1) void fwd_onepass_kernel(FwdParams p) {
  __shared__ Smem sm[NBUF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, h = lane >> 5;
  const int BH = p.B * p.H;
  const int n_qt = (p.S + OBM - 1) / OBM;
  const int bh = blockIdx.x % BH;
  const int qt_i = blockIdx.x / BH;
  const int qt = p.causal ? n_qt - 1 - qt_i : qt_i;
  const int b = bh / p.H, hd = bh % p.H;
  const int q0 = qt * OBM;
  // Waves w and w + 4 share a SIMD: give them row blocks w and 7 - w.
  const int blk = wave < 4 ? wave : 11 - wave;
  const int qw = q0 + 32 * blk, my_q = qw + ln;
  const int S = p.S;
  const bool causal = p.causal != 0;

  const float lam = wave_lambda(p.lq1, p.lk1, p.lq2, p.lk2, p.lambda_dim, p.lambda_fixed, p.lambda_init);
  if (blockIdx.x == 0 && tid == 0 && p.lambda_out) *p.lambda_out = lam;
  const float c = p.scale * kLog2e;
  const float bnd = 0x1p14f / (1.f + fabsf(lam));

  Loader ld;
  ld.init((const bf16 *)p.k1 + b * p.ks_b + hd * p.ks_h, (const bf16 *)p.k2 + b * p.ks_b + hd * p.ks_h,
          p.v16 + (int64_t)bh * S * DV, p.ks_s, DV, S, tid);

  bf16x8 q1f[4], q2f[4];
  {
    const bf16 *q1 = (const bf16 *)p.q1 + b * p.qs_b + (int64_t)my_q * p.qs_s + hd * p.qs_h + 8 * h;
    const bf16 *q2 = (const bf16 *)p.q2 + b * p.qs_b + (int64_t)my_q * p.qs_s + hd * p.qs_h + 8 * h;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      q1f[kc] = my_q < S ? *(const bf16x8 *)(q1 + kc * 16) : bf16x8{};
      q2f[kc] = my_q < S ? *(const bf16x8 *)(q2 + kc * 16) : bf16x8{};
    }
  }

  const int kend = causal ? min(S, q0 + OBM) : S;
  const int n_kt = (kend + BN - 1) / BN;
  // The fp16 copy of V holds each 256-row chunk c times 2^vexp[c]; the
  // accumulators hold sums against the current tile's shift, rescaled (rarely)
  // when a tile's chunk has another one.  Each tile's shift is read one tile
  // ahead.
  const int *vexp = p.vexp + (int64_t)bh * vrange_chunks(S);
  // Tiles every row of the workgroup sees in full (no mask, no tail).
  const int n_full = min(causal ? (q0 + 1) / BN : n_kt, S / BN);
  const int krow = k_row_perm(ln);

  f32x16 x[4], y[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    x[ct] = f32x16{};
    y[ct] = f32x16{};
  }
  RowState st = {kNegInf, kNegInf, 0.f, 0.f, 0.f};

  // Three LDS buffers: tile kt is read from buffer kt % 3 while tile kt + 1
  // (loaded into registers one tile ahead) is stored into buffer (kt + 1) % 3.
  // The waves of the second group (one per SIMD) run half a sub-tile behind
  // the first: they defer the PV products of each tile's second sub-tile to
  // the start of the next tile (buffer (kt - 1) % 3, still intact), so that on
  // every SIMD one wave's matrix work overlaps the other's softmax arithmetic
  // instead of both waves reaching each phase together after the barrier.
  // (Not with SAVE: its hi/lo weights would double the deferred registers.)
  const bool lag = !SAVE && wave >= 4;
  bool pending = false;
  f16x8 pw[2], pe[2], pwl[SAVE ? 2 : 1], pel[SAVE ? 2 : 1];
  int cur = 0, prv = NBUF - 1, nxb = 1;
  Stage nxt;
  ld.load(0, nxt);
  store_stage(sm[0], nxt, tid);
  __syncthreads();
  int vk = __builtin_amdgcn_readfirstlane(vexp[0]);
  int ktile = vk;  // shift of the tile about to be computed
  for (int kt = 0; kt < n_full; ++kt) {
    ld.load((kt + 1) * BN, nxt);  // past the end: the buffer range gives zeros
    sched_fence();
    if (pending) sub_pv<SAVE>(sm[prv], 1, lane, pw, pe, pwl, pel, x, y);
    if (ktile != vk) rescale_acc(x, y, ktile - vk, vk);
    ktile = __builtin_amdgcn_readfirstlane(vexp[min((kt + 1) * BN, kend - 1) / kVRangeRows]);
    {
      f16x8 wb[2], eb[2], wl[SAVE ? 2 : 1], el[SAVE ? 2 : 1];
      sub_softmax<false, SAVE>(sm[cur], 0, kt * BN, krow, lane, q1f, q2f, c, lam, bnd, st, x, y, S, causal, my_q,
                               wb, eb, wl, el);
      sub_pv<SAVE>(sm[cur], 0, lane, wb, eb, wl, el, x, y);
    }
    sub_softmax<false, SAVE>(sm[cur], 1, kt * BN + 32, krow, lane, q1f, q2f, c, lam, bnd, st, x, y, S, causal, my_q,
                             pw, pe, pwl, pel);
    pending = lag;
    if (!lag) sub_pv<SAVE>(sm[cur], 1, lane, pw, pe, pwl, pel, x, y);
    sched_fence();
    store_stage(sm[nxb], nxt, tid);
    __syncthreads();
    prv = cur;
    cur = nxb;
    nxb = nxb == NBUF - 1 ? 0 : nxb + 1;
  }
  for (int kt = n_full; kt < n_kt; ++kt) {
    ld.load((kt + 1) * BN, nxt);
    sched_fence();
    if (pending) sub_pv<SAVE>(sm[prv], 1, lane, pw, pe, pwl, pel, x, y);
    pending = false;
    if (ktile != vk) rescale_acc(x, y, ktile - vk, vk);
    ktile = __builtin_amdgcn_readfirstlane(vexp[min((kt + 1) * BN, kend - 1) / kVRangeRows]);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int sb = kt * BN + sub * 32;
      if (sb >= S || (causal && sb > qw + 31)) continue;  // wave-uniform
      f16x8 wb[2], eb[2], wl[SAVE ? 2 : 1], el[SAVE ? 2 : 1];
      if ((causal && sb + 31 > qw) || sb + 32 > S)
        sub_softmax<true, SAVE>(sm[cur], sub, sb, krow, lane, q1f, q2f, c, lam, bnd, st, x, y, S, causal, my_q, wb,
                                eb, wl, el);
      else
        sub_softmax<false, SAVE>(sm[cur], sub, sb, krow, lane, q1f, q2f, c, lam, bnd, st, x, y, S, causal, my_q, wb,
                                 eb, wl, el);
      sub_pv<SAVE>(sm[cur], sub, lane, wb, eb, wl, el, x, y);
    }
    sched_fence();
    store_stage(sm[nxb], nxt, tid);
    __syncthreads();
    prv = cur;
    cur = nxb;
    nxb = nxb == NBUF - 1 ? 0 : nxb + 1;
  }
  if (pending) sub_pv<SAVE>(sm[prv], 1, lane, pw, pe, pwl, pel, x, y);  // only when there was no masked tile

  // O = X / L1 + (kappa / L1 - lambda / L2) Y; per-head RMSNorm x (1 - lambda_init).
  const float L1 = st.l1 + other_half(st.l1);
  const float L2 = st.l2 + other_half(st.l2);
  const float unv = __builtin_ldexpf(1.f, -vk);  // the accumulators hold V 2^vk products
  const float i1 = unv / L1;
  const float cy = (st.kap / L1 - lam / L2) * unv;
  float ss = 0.f;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[ct][r] = fmaf(x[ct][r], i1, cy * y[ct][r]);
      ss = fmaf(x[ct][r], x[ct][r], ss);
    }
  ss += other_half(ss);
  const float rstd = p.norm ? 1.f / sqrtf(ss * (1.f / DV) + p.eps) : 1.f;
  const float f = p.norm ? rstd * (1.f - p.lambda_init) : 1.f;
  if (my_q < S) {
    bf16 *out = (bf16 *)p.out + b * p.os_b + (int64_t)my_q * p.os_s + hd * p.os_h;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = ct * 32 + 8 * g + 4 * h;
        bf16x4 yv = {f2bf(x[ct][4 * g] * f), f2bf(x[ct][4 * g + 1] * f), f2bf(x[ct][4 * g + 2] * f),
                     f2bf(x[ct][4 * g + 3] * f)};
        *(bf16x4 *)(out + ch) = yv;
      }
    if constexpr (SAVE) {
      const int64_t row = ((int64_t)b * S + my_q) * p.H + hd;  // saves are [B, S, H, DV]
      float *op = p.o_pre + row * DV;
      float *ap = p.a2 + row * DV;
      const float i2 = unv / L2;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ch = ct * 32 + 8 * g + 4 * h;
          *(f32x4 *)(op + ch) = f32x4{x[ct][4 * g], x[ct][4 * g + 1], x[ct][4 * g + 2], x[ct][4 * g + 3]};
          *(f32x4 *)(ap + ch) = f32x4{y[ct][4 * g], y[ct][4 * g + 1], y[ct][4 * g + 2], y[ct][4 * g + 3]} * i2;
        }
      if (h == 0) {
        const int64_t si = ((int64_t)b * p.H + hd) * S + my_q;  // [B, H, S]
        p.lse1[si] = (st.m1 + log2f(L1)) * kLn2;
        p.lse2[si] = (st.m2 + log2f(L2)) * kLn2;
        p.rstd[si] = rstd;
      }
    }
  }
}

}  // namespace

size_t fwd_workspace_bytes(int B, int S, int H) { return vconv_bytes(B, S, H); }

hipError_t launch_fwd(const FwdParams &p0, void *workspace, hipStream_t st) {
  // The fp16 copy of V (with its per-chunk shifts) is written first; the
  // one-pass kernel reads it.
  FwdParams p = p0;
  VConvParams vc{p.v, p.vs_b, p.vs_s, p.vs_h, p.B, p.S, p.H, static_cast<f16 *>(workspace), nullptr};
  vc.kexp = reinterpret_cast<int *>(static_cast<char *>(workspace) +
                                    (((size_t)p.B * p.H * p.S * DV * 2 + 255) & ~(size_t)255));
  hipError_t e = launch_vconv(vc, st);
  if (e != hipSuccess) return e;
  p.v16 = vc.v16;
  p.vexp = vc.kexp;
  const int n_qt = (p.S + OBM - 1) / OBM;
  dim3 grid(n_qt * p.B * p.H), block(NT);
  if (p.lse1)
    hipLaunchKernelGGL(fwd_onepass_kernel<true>, grid, block, 0, st, p);
  else
    hipLaunchKernelGGL(fwd_onepass_kernel<false>, grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace diffattn
