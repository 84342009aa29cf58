// Backward of multi-head differential attention on gfx950 (bf16 storage,
// d = 64, dv = 128).  The pages print no gradient formulas; these are the
// chain rule of the forward (glossary page "Differential Transformer",
// section "How differential attention works"; news write-up, multi-head
// section):
//   Y = a r O,  a = 1 - lambda_init,  r = (mean_c O^2 + eps)^-1/2
//   g = dL/dO = a r dY - a r^3 O (sum_c dY O) / dv        (g = dY without norm)
//   O = A1 - lambda A2,  A_m = P_m V
//   E_m = g . A_m = sum_j P_m dP  (per query row)
//   dL/dlambda = -sum_rows g . A2
//   dV = (P1 - lambda P2)^T g                     (one product for both maps)
//   dP = g V^T                                    (shared: dP2 = -lambda dP1)
//   dS1 = P1 (dP - E1),  dS2 = -lambda P2 (dP - E2)
//   dQ_m = s dS_m K_m,  dK_m = s dS_m^T Q_m,  s = softmax scale
//   lambda = e^al - e^be + lambda_init:  dlq1 = dlam e^al lk1, dlk1 = dlam e^al lq1,
//   dlq2 = -dlam e^be lk2, dlk2 = -dlam e^be lq2.
//
// Kernels, in launch order:
//   bwd_pre    per query row: |g| (g formed from dY, the saved O and rstd;
//              never stored), |V_row| and the row's largest |Q|, |K|, |V|;
//   bwd_scales one workgroup per (batch, head): power-of-two scales that keep
//              the fp16 operands below 2^13 (g by its largest row norm; dS by
//              the bound |dS| <= max(1,|lambda|) (|g| |V| + |E|) <= 2 max(1,|lambda|)
//              max|g| max|V|; W = P1 - lambda P2 by 1 + |lambda|);
//   bwd_gconv  per row: g formed again as in bwd_pre; the row's share -g.A2
//              of dL/dlambda from that float32 g and the forward's float32 A2
//              (the sum over rows cancels by orders of magnitude, so it takes
//              float32 g rather than the fp16 copy the matrix products use);
//              g' = fp16(g 2^sg) and
//              E_m = g' . A_m (A2 saved by the forward, A1 = O + lambda A2):
//              from the same fp16 g' the matrix products use, E equals
//              sum_j P_m dP' up to float32 rounding, so dS = P (dP - E) stays
//              self-consistent where one key dominates a row and dP - E
//              cancels; also the row's Q1 | Q2 in fp16 for the key-outer
//              kernel's staging and its K1 | K2 and V in fp16 for the
//              query-outer kernel's (converted once here rather than once per
//              query tile that reads them);
//   bwd_dq     query-outer (the forward's layout): each workgroup owns 128
//              queries and streams 64-key tiles through swizzled LDS tiles:
//              dS and dQ1, dQ2 accumulated in registers;
//   bwd_dkdv   KV-outer: each workgroup owns 128 keys (4 waves x 32) and
//              streams 64-query chunks: recomputes P1, P2 and dP, accumulates
//              dV, dK1, dK2 in registers; past the diagonal, one sub-chunk's
//              elementwise work runs under the matrix products of its
//              neighbours.  Recomputing rather than accumulating dQ with
//              atomics keeps every result deterministic;
//   bwd_dlsum  one workgroup per (batch, head): the sum of its rows' shares
//              in a fixed order;
//   bwd_lambda one workgroup: dL/dlambda = sum of the (batch, head) sums in a
//              fixed order, then the chain rule into the four lambda vectors.
// Matrix-core operands are fp16 with float32 accumulation: bf16 rounding of g,
// W and dS alone would spend most of the bf16 error budget.  Q, K and V enter
// fp16 times powers of two 2^kq, 2^kk, 2^kv chosen per (batch, head) from
// their largest magnitudes (bwd_pre, bwd_scales; vrange.h), so any finite bf16
// inputs convert without saturating or losing precision, and every result is
// unscaled exactly.
#include <cstddef>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "vrange.h"

namespace diffattn {
namespace {

constexpr int D = 64, DV = 128, NT = 256;
constexpr int QST = D + 8;    // LDS row stride (fp16) of Q / K tiles
constexpr int GST = DV + 32;  // LDS row stride (fp16) of g / V tiles (tr16-friendly)

struct Ws {
  f16 *gh;         // [B, H, S, DV] fp16, g * 2^sg
  f16 *qh;         // [B, H, S, 2 D] fp16: Q1 (channels 0..63) and Q2 (64..127), times 2^kq
  f16 *kh;         // [B, H, S, 2 D] fp16: K1 | K2 times 2^kk
  f16 *vh;         // [B, H, S, DV] fp16: V times 2^kv
  float *e1, *e2;  // [B, H, S]  E_m = sum_j P_m dP (unscaled)
  float *gnorm, *vnorm, *dlam_row;  // [B, H, S]
  float *amax;     // [B, H, S][4]: the row's largest |Q1|,|Q2|; |K1|,|K2|; |V|; unused
  float *scales;   // [B*H][8]: sg, kappa, omega, kq, kk, kv, unused x2 (exponents of 2)
  float *dlam_bh;  // [B*H] per-(batch, head) sums of dlam_row
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Ws carve(void *base, int B, int S, int H) {
  char *p = static_cast<char *>(base);
  const size_t rows = (size_t)B * H * S;
  Ws w;
  w.gh = (f16 *)p; p += align256(rows * DV * 2);
  w.qh = (f16 *)p; p += align256(rows * 2 * D * 2);
  w.kh = (f16 *)p; p += align256(rows * 2 * D * 2);
  w.vh = (f16 *)p; p += align256(rows * DV * 2);
  w.e1 = (float *)p; p += align256(rows * 4);
  w.e2 = (float *)p; p += align256(rows * 4);
  w.gnorm = (float *)p; p += align256(rows * 4);
  w.vnorm = (float *)p; p += align256(rows * 4);
  w.dlam_row = (float *)p; p += align256(rows * 4);
  w.amax = (float *)p; p += align256(rows * 16);
  w.scales = (float *)p; p += align256((size_t)B * H * 32);
  w.dlam_bh = (float *)p; p += align256((size_t)B * H * 4);
  return w;
}

__host__ __device__ inline size_t ws_bytes(int B, int S, int H) {
  const size_t rows = (size_t)B * H * S;
  return 2 * align256(rows * DV * 2) + 2 * align256(rows * 2 * D * 2) + 5 * align256(rows * 4) +
         align256(rows * 16) + align256((size_t)B * H * 32) + align256((size_t)B * H * 4);
}

__device__ __forceinline__ float exp2i(float e) { return fast_exp2(e); }  // e integral: exact power of 2

// ---------------------------------------------------------------------------
// Row kernels (bwd_pre, bwd_gconv): 16 lanes per (b, h, s) row, 8 channels per
// lane (16-byte bf16 and 32-byte float32 accesses), four rows per wave.  Lanes
// past the last row work on the last row and store nothing (every lane takes
// part in the wave-wide lambda reduction and the row reductions).
constexpr int RPB = NT / kRowLanes;  // rows per workgroup

// g = dL/dO for one row's eight channels (the RMSNorm backward when the norm
// is on): g = a r dy - a r^3 o (sum_c dy o) / dv.  bwd_pre and bwd_gconv both
// form it from dy, the saved O and rstd with this code (explicit fma, fixed
// reduction order), so the two get the same g and it is never stored.
__device__ __forceinline__ void row_grad(const BwdParams &p, int b, int h, int s, const float *dy, const float *o,
                                         float *g) {
#pragma unroll
  for (int i = 0; i < 8; ++i) g[i] = dy[i];
  if (p.norm) {
    const float r = p.rstd[((int64_t)b * p.H + h) * p.S + s];
    const float ar = (1.f - p.lambda_init) * r;
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t = fmaf(dy[i], o[i], t);
    t = row_sum(t);
    const float k = ar * r * r * t * (1.f / DV);
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = fmaf(-k, o[i], ar * dy[i]);
  }
}

// bwd_pre: row norms of g (the gradient reaching the pre-norm output O) and
// V, and the row's largest |Q|, |K|, |V|
// (their fp16 copies are scaled by powers of two chosen from these, vrange.h).
__global__ __launch_bounds__(NT) void bwd_pre_kernel(BwdParams p, Ws w) {
  const int part = threadIdx.x & (kRowLanes - 1);
  const int64_t nrows = (int64_t)p.B * p.H * p.S;
  const int64_t row0 = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 4);  // over [B, H, S]
  const bool ok = row0 < nrows;
  const int64_t row = ok ? row0 : nrows - 1;
  const int s = row % p.S;
  const int bh = row / p.S;
  const int b = bh / p.H, h = bh % p.H;
  const int c = part * 8;
  float dy[8], v[8], o[8], g[8];
  bf16x8_f32(*(const u32x4 *)((const bf16 *)p.dout + b * p.ds_b + (int64_t)s * p.ds_s + h * p.ds_h + c), dy);
  bf16x8_f32(*(const u32x4 *)((const bf16 *)p.v + b * p.vs_b + (int64_t)s * p.vs_s + h * p.vs_h + c), v);
  const int64_t srow = ((int64_t)b * p.S + s) * p.H + h;   // saves are [B, S, H, DV]
  load_f32x8(p.o_pre + srow * DV + c, o);
  row_grad(p, b, h, s, dy, o, g);
  float gn = 0.f, vn = 0.f, vm = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    gn = fmaf(g[i], g[i], gn);
    vn = fmaf(v[i], v[i], vn);
    vm = fmaxf(vm, fabsf(v[i]));
  }
  // Q1 | Q2 and K1 | K2: lanes 0..7 the first (64 channels), 8..15 the second.
  const int qc = (part & 7) * 8;
  float q[8], kk[8];
  bf16x8_f32(*(const u32x4 *)((const bf16 *)(part < 8 ? p.q1 : p.q2) + b * p.qs_b + (int64_t)s * p.qs_s +
                              h * p.qs_h + qc), q);
  bf16x8_f32(*(const u32x4 *)((const bf16 *)(part < 8 ? p.k1 : p.k2) + b * p.ks_b + (int64_t)s * p.ks_s +
                              h * p.ks_h + qc), kk);
  float qm = 0.f, km = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    qm = fmaxf(qm, fabsf(q[i]));
    km = fmaxf(km, fabsf(kk[i]));
  }
  gn = row_sum(gn);
  vn = row_sum(vn);
  qm = row_max(qm);
  km = row_max(km);
  vm = row_max(vm);
  if (ok) {
    if (part == 0) {
      w.gnorm[row] = sqrtf(gn);
      w.vnorm[row] = sqrtf(vn);
      *(f32x4 *)(w.amax + row * 4) = f32x4{qm, km, vm, 0.f};
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_scales: one workgroup of NTS threads per (b, h) (many loads in flight:
// the pass is latency-bound).
constexpr int NTS = 1024, NWS = NTS / 64;

// Fixed-order pairwise sum / maximum of the NWS per-wave values.
__device__ __forceinline__ float tree_sum(const float *v) {
  float t[NWS];
#pragma unroll
  for (int i = 0; i < NWS; ++i) t[i] = v[i];
#pragma unroll
  for (int n = NWS / 2; n > 0; n >>= 1)
#pragma unroll
    for (int i = 0; i < n; ++i) t[i] = t[i] + t[i + n];
  return t[0];
}

__device__ __forceinline__ float tree_max(const float *v) {
  float m = v[0];
#pragma unroll
  for (int i = 1; i < NWS; ++i) m = fmaxf(m, v[i]);
  return m;
}

__global__ __launch_bounds__(NTS) void bwd_scales_kernel(BwdParams p, Ws w) {
  __shared__ float red[5][NWS];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float lam = wave_lambda(p.lq1, p.lk1, p.lq2, p.lk2, p.lambda_dim, p.lambda_fixed, p.lambda_init);
  const int64_t base = (int64_t)bh * p.S;
  float gm = 0.f, vm = 0.f;
  f32x4 am = {0.f, 0.f, 0.f, 0.f};
  for (int s = tid; s < p.S; s += NTS) {
    gm = fmaxf(gm, w.gnorm[base + s]);
    vm = fmaxf(vm, w.vnorm[base + s]);
    const f32x4 a = *(const f32x4 *)(w.amax + (base + s) * 4);
    am = f32x4{fmaxf(am[0], a[0]), fmaxf(am[1], a[1]), fmaxf(am[2], a[2]), 0.f};
  }
  for (int o = 32; o > 0; o >>= 1) {
    gm = fmaxf(gm, __shfl_xor(gm, o));
    vm = fmaxf(vm, __shfl_xor(vm, o));
#pragma unroll
    for (int i = 0; i < 3; ++i) am[i] = fmaxf(am[i], __shfl_xor(am[i], o));
  }
  if (lane == 0) {
    red[0][wave] = gm;
    red[1][wave] = vm;
#pragma unroll
    for (int i = 0; i < 3; ++i) red[2 + i][wave] = am[i];
  }
  __syncthreads();
  if (tid == 0) {
    gm = tree_max(red[0]);
    vm = tree_max(red[1]);
    float ks[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) ks[i] = (float)v_shift_of_max(__float_as_uint(tree_max(red[2 + i])) >> 16);
    const float al = fmaxf(1.f, fabsf(lam));
    const float sg = gm > 0.f ? fminf(fmaxf(floorf(13.f - log2f(gm)), -60.f), 60.f) : 0.f;
    const float x = 2.f * al * gm * vm;  // bound on |dS| before scaling by 2^sg
    // dP' = g' V' carries 2^(sg + kv): dS is scaled by 2^kappa on top of it.
    const float kap = x > 0.f ? fminf(fmaxf(floorf(13.f - log2f(x) - sg), -60.f), 60.f) - ks[2] : 0.f;
    const float om = floorf(13.f - log2f(1.f + fabsf(lam)));
    w.scales[bh * 8 + 0] = sg;
    w.scales[bh * 8 + 1] = kap;
    w.scales[bh * 8 + 2] = om;
    w.scales[bh * 8 + 3] = ks[0];  // Q1, Q2
    w.scales[bh * 8 + 4] = ks[1];  // K1, K2
    w.scales[bh * 8 + 5] = ks[2];  // V
  }
}

// ---------------------------------------------------------------------------
// bwd_gconv: per (b, h, s) row, g' = fp16(g 2^sg) and the row terms
// E_m = g' . A_m (A2 saved by the forward, A1 = O + lambda A2), stored
// unscaled.  Taking E from the same fp16 g' the matrix products use makes it
// equal to sum_j P_m dP' up to float32 rounding, so dS = P (dP - E) stays
// self-consistent where one key dominates a row and dP - E cancels.
__global__ __launch_bounds__(NT) void bwd_gconv_kernel(BwdParams p, Ws w) {
  const int part = threadIdx.x & (kRowLanes - 1);
  const int64_t nrows = (int64_t)p.B * p.H * p.S;
  const int64_t row0 = (int64_t)blockIdx.x * RPB + (threadIdx.x >> 4);  // over [B, H, S]
  const bool ok = row0 < nrows;
  const int64_t row = ok ? row0 : nrows - 1;
  const float lam = wave_lambda(p.lq1, p.lk1, p.lq2, p.lk2, p.lambda_dim, p.lambda_fixed, p.lambda_init);
  const int s = row % p.S;
  const int bh = row / p.S;
  const int b = bh / p.H, h = bh % p.H;
  const int c = part * 8;
  const float sg = w.scales[bh * 8 + 0], f = exp2i(sg);
  float dy[8], g[8], o[8], a2[8];
  bf16x8_f32(*(const u32x4 *)((const bf16 *)p.dout + b * p.ds_b + (int64_t)s * p.ds_s + h * p.ds_h + c), dy);
  const int64_t srow = ((int64_t)b * p.S + s) * p.H + h;   // saves are [B, S, H, DV]
  load_f32x8(p.o_pre + srow * DV + c, o);
  load_f32x8(p.a2 + srow * DV + c, a2);
  row_grad(p, b, h, s, dy, o, g);
  // The row's share -g . A2 of dL/dlambda, from the float32 g (the sum over
  // rows cancels by orders of magnitude; the fp16 g' would not do).
  float ga = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ga = fmaf(g[i], a2[i], ga);
  ga = row_sum(ga);
  f16x8 gh;
#pragma unroll
  for (int i = 0; i < 8; ++i) gh[i] = (f16)(g[i] * f);
  float e1 = 0.f, e2 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float gi = (float)gh[i];
    e2 = fmaf(gi, a2[i], e2);
    e1 = fmaf(gi, fmaf(lam, a2[i], o[i]), e1);
  }
  e1 = row_sum(e1);
  e2 = row_sum(e2);
  if (ok) {
    *(f16x8 *)(w.gh + row * DV + c) = gh;
    // The row's Q1 | Q2 to fp16 times 2^kq (exact) for the key-outer kernel's
    // staging: lanes 0..7 Q1, 8..15 Q2, eight channels each.
    const int qc = (part & 7) * 8;
    const u32x4 raw = *(const u32x4 *)((const bf16 *)(part < 8 ? p.q1 : p.q2) + b * p.qs_b + (int64_t)s * p.qs_s +
                                       h * p.qs_h + qc);
    const VScale sq((int)w.scales[bh * 8 + 3]);
    *(u32x4 *)(w.qh + row * (2 * D) + c) = sq.on ? bf16x8_to_f16x8<true>(raw, sq) : bf16x8_to_f16x8<false>(raw, sq);
    // Its key-side rows for the query-outer kernel's staging: K1 | K2 times
    // 2^kk and V times 2^kv (the same row index: keys and queries are the
    // same S tokens).
    const u32x4 rk = *(const u32x4 *)((const bf16 *)(part < 8 ? p.k1 : p.k2) + b * p.ks_b + (int64_t)s * p.ks_s +
                                      h * p.ks_h + qc);
    const VScale sk((int)w.scales[bh * 8 + 4]);
    *(u32x4 *)(w.kh + row * (2 * D) + c) = sk.on ? bf16x8_to_f16x8<true>(rk, sk) : bf16x8_to_f16x8<false>(rk, sk);
    const u32x4 rv = *(const u32x4 *)((const bf16 *)p.v + b * p.vs_b + (int64_t)s * p.vs_s + h * p.vs_h + c);
    const VScale sv((int)w.scales[bh * 8 + 5]);
    *(u32x4 *)(w.vh + row * DV + c) = sv.on ? bf16x8_to_f16x8<true>(rv, sv) : bf16x8_to_f16x8<false>(rv, sv);
    if (part == 0) {
      const float un = exp2i(-sg);
      w.e1[row] = e1 * un;
      w.e2[row] = e2 * un;
      w.dlam_row[row] = -ga;
    }
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

__device__ __forceinline__ f16x8 pack8h(const float *w) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const f32x2 x = {w[i], w[i + 1]};
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

// Swizzled tiles (no row padding): 16-byte chunk c of row r of a tile with
// 64-half rows (K) is stored at chunk c ^ swz64(r), of a tile with 128-half
// rows (V) at chunk c ^ swz128(r).  The matrix products read a tile two ways:
// one chunk of 16 consecutive rows per 16 lanes (row operands, 16-byte reads)
// and four consecutive chunks of 4 consecutive rows per 32 lanes (transpose
// reads, 8 bytes each); with these permutations both touch each of the 64 LDS
// banks once per 256 bytes, where a plain row padding can serve only one of
// the two (128-half rows padded to 160 put every fourth row of a row-operand
// read on the same banks).  Both depend on r mod 16 only.
__device__ __forceinline__ int swz64(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz128(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Half offset of chunk c of row r in a swizzled tile with W-half rows.  For
// c = c1 | c2 with disjoint bits, swz_off(r, c1 | c2) = swz_off(r, c1) ^ 8 c2:
// each lane keeps one offset per access pattern and forms every read of that
// pattern with one XOR.
template <int W>
__device__ __forceinline__ int swz_off(int r, int c) {
  return r * W + 8 * (c ^ (W == D ? swz64(r) : swz128(r)));
}

// Lane offsets of the two transpose reads of tr_operand (rows 8 (l / 32) +
// (l % 16) / 4 and 4 below, the lane's 8 bytes of chunks 2 ((l / 16) % 2) + 0..1).
struct TrLane {
  int lo, hi;
};

template <int W>
__device__ __forceinline__ TrLane tr_lane(int lane) {
  const int h = lane >> 5, j = lane & 15, half16 = (lane >> 4) & 1;
  const int r = 8 * h + (j >> 2), c = 2 * half16 + ((j & 3) >> 1), w = 4 * (j & 1);
  return TrLane{swz_off<W>(r, c) + w, swz_off<W>(r + 4, c) + w};
}

// tr_operand on a swizzled tile with W-half rows (r0 a multiple of 16, c0 of 32).
template <int W>
__device__ __forceinline__ f16x8 tr_operand_swz(const f16 *tile, const TrLane &t, int r0, int c0) {
  const f16x4 lo = lds_read_tr16(tile + r0 * W + (t.lo ^ c0));
  const f16x4 hi = lds_read_tr16(tile + r0 * W + (t.hi ^ c0));
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------------------
// bwd_dkdv: KV-outer.  Workgroup = 128 keys of one (b, h); wave w owns keys
// kb + 32 w + 0..31 (lane l % 32).  Streams 64-query chunks through three LDS
// buffers: the masked chunks (the diagonal, or every chunk of the last key
// block) one 32-query sub-chunk after another, the rest as a software
// pipeline over sub-chunks (see the loop).
constexpr int KVB = 128, QCH = 64;

struct SmemA {
  f16 q1[QCH * QST];
  f16 q2[QCH * QST];
  f16 g[QCH * GST];
  float lse1[QCH], lse2[QCH], e1[QCH], e2[QCH];
};

// One thread's share of a staged query chunk: four 16-byte chunks of the
// fp16 Q1 | Q2 rows, four of g', and (threads 0..63) one row's statistics as
// loaded.  Nothing is computed from the loaded values until store_chunk, so
// the loads stay in flight while the previous chunk is processed.
struct ChunkRegs {
  u32x4 q[4], g[4];
  float lse1, lse2, e1, e2;
};

// Buffer resources over one (batch, head)'s S rows of 256 bytes (the fp16
// Q1 | Q2 rows, or the fp16 g' rows): rows past the end read as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const f16 *rows, int S) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)rows, 0, (uint32_t)S * 256, 0x00020000);
}

// Thread tid's four 16-byte pieces of the 64 rows starting at q0 (row-major,
// 16 threads per row).
__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t rs, int q0, int tid, u32x4 *v) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
    v[k] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((uint32_t)q0 * 256 + (tid + NT * k) * 16), 0, 0));
}

// Loads the chunk of QCH query rows starting at q0 (rows past the end read as
// zeros; their statistics are read from the last row and masked when stored).
__device__ __forceinline__ void load_chunk(const BwdParams &p, const Ws &w, int64_t statb, int q0, int S, int tid,
                                           ChunkRegs &r) {
  load_rows(row_rsrc(w.qh + statb * (2 * D), S), q0, tid, r.q);
  load_rows(row_rsrc(w.gh + statb * DV, S), q0, tid, r.g);
  if (tid < QCH) {
    const int64_t q = statb + min(q0 + tid, S - 1);
    r.lse1 = p.lse1[q];
    r.lse2 = p.lse2[q];
    r.e1 = w.e1[q];
    r.e2 = w.e2[q];
  }
}

// Per-workgroup constants folded into the staged row statistics, so that the
// score loop forms P1 2^kappa, |lambda| P2 2^kappa and the dS terms with one
// exponential and one or two operations each:
//   lse1' = lse1 log2(e) - kappa,  lse2' = lse2 log2(e) - kappa - log2|lambda|
//   E1' = E1 fE,  E2' = -sigma E2 fE,  sigma = -sign(lambda)
// (lambda = 0 makes lse2' infinite, so P2 and its terms vanish).
struct RowFold {
  float fE, kap, l2lam, sig;
};

__device__ __forceinline__ RowFold row_fold(float lam, float fE, float kap) {
  return RowFold{fE, kap, log2f(fabsf(lam)), lam >= 0.f ? -1.f : 1.f};
}

// Register -> LDS half of the staging; the statistics are folded as above
// and rows past the end masked (infinite lse', so their P terms are zero).
__device__ __forceinline__ void store_chunk(SmemA &sm, const ChunkRegs &r, int tid, int q0, int S,
                                            const RowFold &f) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + NT * k, row = i >> 4, col = (i & 15) * 8;
    f16 *dq = col < D ? sm.q1 + row * QST + col : sm.q2 + row * QST + (col - D);
    *(u32x4 *)dq = r.q[k];
    *(u32x4 *)(sm.g + row * GST + col) = r.g[k];
  }
  if (tid < QCH) {
    const bool ok = q0 + tid < S;
    sm.lse1[tid] = ok ? fmaf(r.lse1, kLog2e, -f.kap) : __builtin_inff();
    sm.lse2[tid] = ok ? fmaf(r.lse2, kLog2e, -(f.kap + f.l2lam)) : __builtin_inff();
    sm.e1[tid] = ok ? r.e1 * f.fE : 0.f;
    sm.e2[tid] = ok ? -f.sig * r.e2 * f.fE : 0.f;
  }
}

// Half of a chunk's staging (part 0: the fp16 Q1 | Q2 rows and the row
// statistics; part 1: the fp16 g' rows), for the pipelined loop, which stages
// the next chunk over two steps so that only half of it is in flight at once.
struct HalfRegs {
  u32x4 v[4];
  float lse1, lse2, e1, e2;
};

__device__ __forceinline__ void store_half(SmemA &sm, const HalfRegs &r, int tid, int q0, int S, int part,
                                           const RowFold &f) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + NT * k, row = i >> 4, col = (i & 15) * 8;
    f16 *dst = part == 1 ? sm.g + row * GST + col
                         : (col < D ? sm.q1 + row * QST + col : sm.q2 + row * QST + (col - D));
    *(u32x4 *)dst = r.v[k];
  }
  if (part == 0 && tid < QCH) {
    const bool ok = q0 + tid < S;
    sm.lse1[tid] = ok ? fmaf(r.lse1, kLog2e, -f.kap) : __builtin_inff();
    sm.lse2[tid] = ok ? fmaf(r.lse2, kLog2e, -(f.kap + f.l2lam)) : __builtin_inff();
    sm.e1[tid] = ok ? r.e1 * f.fE : 0.f;
    sm.e2[tid] = ok ? -f.sig * r.e2 * f.fE : 0.f;
  }
}

// Elementwise part of one 32 x 32 block of the key-outer kernel (lane = key,
// registers = queries qb + row_of_reg(r, h)): the merged dV weight
// (P1 - lambda P2) 2^omega and dS_m 2^kappa for both maps.  Query qb + o is
// masked for this lane's key iff o < lo (lo = my_key - qb under the causal
// mask, 32 for a key past the end, else below 0): one compare per score.
// Rows past the end already have zero probabilities (infinite lse').
template <bool MASK>
__device__ __forceinline__ void dkdv_elem(const SmemA &sm, const f32x16 &s1, const f32x16 &s2, const f32x16 &dp,
                                          int sub, int h, float c, float sig, float fW2, int lo, float *wv,
                                          float *ds1, float *ds2) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qi = sub * 32 + row_of_reg(r, h);
    // The mask selects the exponent (-inf for a masked pair), not the result:
    // a select of the exponential itself was compiled into branches.
    const bool dead = MASK && row_of_reg(r, h) < lo;
    const float a1 = fmaf(s1[r], c, -sm.lse1[qi]), a2 = fmaf(s2[r], c, -sm.lse2[qi]);
    const float p1 = fast_exp2(dead ? -__builtin_inff() : a1);  // P1 2^kappa
    const float p2 = fast_exp2(dead ? -__builtin_inff() : a2);  // |lambda| P2 2^kappa
    wv[r] = fmaf(sig, p2, p1) * fW2;
    ds1[r] = p1 * (dp[r] - sm.e1[qi]);
    ds2[r] = p2 * fmaf(dp[r], sig, sm.e2[qi]);
  }
}

__global__ __launch_bounds__(NT, 1) void bwd_dkdv_kernel(BwdParams p, Ws w) {
  __shared__ SmemA smb[3];
  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave tests become scalar branches
  const float lam = wave_lambda(p.lq1, p.lk1, p.lq2, p.lk2, p.lambda_dim, p.lambda_fixed, p.lambda_init);
  // Workgroup id -> (key block, batch-head): key blocks with the most causal
  // work are dispatched first across all heads, and consecutive ids walk the
  // (batch, head) index so a head's key blocks share one XCD's L2.
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH, b = bh / p.H, hd = bh % p.H;
  const int S = p.S;
  const int kb = (blockIdx.x / BH) * KVB, kw = kb + wave * 32, my_key = kw + ln;
  const float sg = w.scales[bh * 8 + 0], kap = w.scales[bh * 8 + 1], om = w.scales[bh * 8 + 2];
  const float kq = w.scales[bh * 8 + 3], kk = w.scales[bh * 8 + 4], kv = w.scales[bh * 8 + 5];
  const VScale sck((int)kk), scv((int)kv);
  // fp16 Q, K, V are Q 2^kq, K 2^kk, V 2^kv: S' = S 2^(kq + kk), dP' = dP 2^(sg + kv).
  const float c = p.scale * kLog2e * exp2i(-(kq + kk));
  const float fE = exp2i(sg + kv);

  // K1, K2 (B operand of S = Q K^T) and V (B operand of dP = g V^T) for my key, fp16.
  f16x8 kf1[4], kf2[4], vf[8];
  {
    const bool ok = my_key < S;
    const bf16 *k1 = (const bf16 *)p.k1 + b * p.ks_b + (int64_t)my_key * p.ks_s + hd * p.ks_h + 8 * h;
    const bf16 *k2 = (const bf16 *)p.k2 + b * p.ks_b + (int64_t)my_key * p.ks_s + hd * p.ks_h + 8 * h;
    const bf16 *vv = (const bf16 *)p.v + b * p.vs_b + (int64_t)my_key * p.vs_s + hd * p.vs_h + 8 * h;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      kf1[kc] = ok ? to_f16x8(*(const u32x4 *)(k1 + kc * 16), sck) : f16x8{};
      kf2[kc] = ok ? to_f16x8(*(const u32x4 *)(k2 + kc * 16), sck) : f16x8{};
    }
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) vf[kc] = ok ? to_f16x8(*(const u32x4 *)(vv + kc * 16), scv) : f16x8{};
  }

  f32x16 dv[4], dk1[2], dk2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) dv[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < 2; ++i) dk1[i] = dk2[i] = f32x16{};

  const int q_begin = p.causal ? (kb / QCH) * QCH : 0;
  const int prow = row_perm(ln);
  const int64_t statb = (int64_t)bh * S;
  // Query chunks double-buffered in LDS: chunk n + 1 is loaded into
  // registers while chunk n is computed, then stored to the other buffer; one
  // barrier per chunk.
  const RowFold fold = row_fold(lam, fE, kap);
  const float fW2 = exp2i(om - kap);  // wv = (P1 + sigma |lambda| P2) 2^kappa 2^(omega - kappa)
  ChunkRegs nxt;
  if (q_begin < S) {
    load_chunk(p, w, statb, q_begin, S, tid, nxt);
    store_chunk(smb[0], nxt, tid, q_begin, S, fold);
  }
  __syncthreads();
  // One chunk; MASKED applies the key-range and causal masks.  Only the chunks
  // on this workgroup's diagonal (the first KVB / QCH under the causal mask)
  // and, in the workgroup holding the last keys, every chunk need them: two
  // loops, one per form, so the unmasked one carries no mask arithmetic and
  // no branch.
  auto chunk = [&](auto masked, int q0, int it) {
    constexpr bool MASKED = decltype(masked)::value;
    SmemA &sm = smb[it % 3];
    const bool more = q0 + QCH < S;
    if (more) load_chunk(p, w, statb, q0 + QCH, S, tid, nxt);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int qs = q0 + sub * 32;
      if (qs >= S) continue;
      if (p.causal && qs + 31 < kw) continue;  // every query of this sub-chunk precedes my keys
      // S1, S2 = Q K^T and dP' = g' V^T; lane = key, registers = queries.
      f32x16 s1 = {}, s2 = {}, dp = {};
      const f16 *qa1 = sm.q1 + (sub * 32 + prow) * QST + 8 * h;
      const f16 *qa2 = sm.q2 + (sub * 32 + prow) * QST + 8 * h;
      const f16 *ga = sm.g + (sub * 32 + prow) * GST + 8 * h;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        s1 = mfma32(*(const f16x8 *)(qa1 + kc * 16), kf1[kc], s1);
        s2 = mfma32(*(const f16x8 *)(qa2 + kc * 16), kf2[kc], s2);
      }
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) dp = mfma32(*(const f16x8 *)(ga + kc * 16), vf[kc], dp);
      float wv[16], ds1[16], ds2[16];
      const int lo = my_key >= S ? 32 : (p.causal ? my_key - qs : -1);
      dkdv_elem<MASKED>(sm, s1, s2, dp, sub, h, c, fold.sig, fW2, lo, wv, ds1, ds2);
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        const f16x8 wb = pack8h(wv + 8 * kc2), b1 = pack8h(ds1 + 8 * kc2), b2 = pack8h(ds2 + 8 * kc2);
        const int r0 = sub * 32 + kc2 * 16;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) dv[ct] = mfma32(tr_operand(sm.g, GST, r0, ct * 32, lane), wb, dv[ct]);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          dk1[dt] = mfma32(tr_operand(sm.q1, QST, r0, dt * 32, lane), b1, dk1[dt]);
          dk2[dt] = mfma32(tr_operand(sm.q2, QST, r0, dt * 32, lane), b2, dk2[dt]);
        }
      }
    }
    if (more) store_chunk(smb[(it + 1) % 3], nxt, tid, q0 + QCH, S, fold);
    __syncthreads();
  };
  const int n_ch = q_begin < S ? (S - q_begin + QCH - 1) / QCH : 0;
  const int n_mask = kb + KVB > S ? n_ch : (p.causal ? min(n_ch, KVB / QCH) : 0);
  for (int it = 0; it < n_mask; ++it) chunk(std::true_type{}, q_begin + it * QCH, it);

  // The unmasked chunks run as a software pipeline over their 32-query
  // sub-chunks.  Step j: the score products of sub-chunk j; its dP products
  // interleaved with the exponentials (vector ALU); then the dV, dK products
  // of sub-chunk j - 1 interleaved with the rest of j's elementwise part.
  // One matrix instruction, then a share of the vector work, in a fixed order:
  // the single wave on each SIMD issues in order, so that order is what
  // overlaps the two units.  LDS operands are read two instructions ahead,
  // from per-step base addresses with the rest in the instructions' offsets.
  // Chunk n_mask + k (sub-chunks 2k, 2k + 1) is in buffer (n_mask + k) % 3
  // from the end of step 2k - 1 (the second half of its staging, barrier)
  // until step 2k + 2 last reads it.
  const int J = 2 * (n_ch - n_mask);
  if (J > 0) {
    typedef DA_LDS const char lchar;
    const int hq = 8 * h, jj = lane & 15, half16 = (lane >> 4) & 1;
    // Per-lane byte offsets: row-major operand reads (A), transpose reads (C),
    // statistics.
    const uint32_t laQ = (prow * QST + hq) * 2, laG = (prow * GST + hq) * 2;
    const uint32_t lcQ = ((hq + (jj >> 2)) * QST + 16 * half16 + 4 * (jj & 3)) * 2;
    const uint32_t lcG = ((hq + (jj >> 2)) * GST + 16 * half16 + 4 * (jj & 3)) * 2;
    const uint32_t lst = hq * 4;
    constexpr uint32_t OQ1 = offsetof(SmemA, q1), OQ2 = offsetof(SmemA, q2), OG = offsetof(SmemA, g);
    constexpr uint32_t OL1 = offsetof(SmemA, lse1), OL2 = offsetof(SmemA, lse2), OE1 = offsetof(SmemA, e1),
                       OE2 = offsetof(SmemA, e2);
    // Base address of buffer `buf` plus a lane offset, opaque to the compiler
    // so that it keeps the constant parts in the instructions' offsets.
    auto lptr = [&](int buf, uint32_t lane_off) -> lchar * {
      lchar *q = (lchar *)(smb + buf) + lane_off;
      asm volatile("" : "+v"(q));
      return q;
    };
    auto tr8 = [&](lchar *q, uint32_t off, int stride) -> f16x8 {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(q + off));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS i16x4 *)(q + off + 8 * stride));
      const f16x4 a = __builtin_bit_cast(f16x4, lo), b = __builtin_bit_cast(f16x4, hi);
      return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    };
    struct Ops {
      f16x8 w[2], b1[2], b2[2];
    };
    // Operand i (0..15) of the dV/dK products of sub-chunk sub: i = 8 kc2 + k;
    // k < 4: g^T columns 32 k (dV), 4, 5: Q1^T (dK1), 6, 7: Q2^T (dK2).
    auto fetch_c = [&](lchar *pq, lchar *pg, int sub, int i) -> f16x8 {
      const int kc2 = i >> 3, k = i & 7, r0 = sub * 32 + kc2 * 16;
      if (k < 4) return tr8(pg, OG + (r0 * GST + k * 32) * 2, GST);
      if (k < 6) return tr8(pq, OQ1 + (r0 * QST + (k - 4) * 32) * 2, QST);
      return tr8(pq, OQ2 + (r0 * QST + (k - 6) * 32) * 2, QST);
    };
    auto mfma_c = [&](int i, const f16x8 &op, const Ops &o) {
      const int kc2 = i >> 3, k = i & 7;
      if (k < 4) dv[k] = mfma32(op, o.w[kc2], dv[k]);
      else if (k < 6) dk1[k - 4] = mfma32(op, o.b1[kc2], dk1[k - 4]);
      else dk2[k - 6] = mfma32(op, o.b2[kc2], dk2[k - 6]);
    };

    // Staging registers, one per half: each half is loaded right after the
    // previous chunk's same half was stored (two steps before its own store).
    const __amdgpu_buffer_rsrc_t rsq = row_rsrc(w.qh + statb * (2 * D), S), rsg = row_rsrc(w.gh + statb * DV, S);
    auto load_part = [&](int q0, int part, HalfRegs &r) {
      load_rows(part == 0 ? rsq : rsg, q0, tid, r.v);
      if (part == 0 && tid < QCH) {
        const int64_t q = statb + min(q0 + tid, S - 1);
        r.lse1 = p.lse1[q];
        r.lse2 = p.lse2[q];
        r.e1 = w.e1[q];
        r.e2 = w.e2[q];
      }
    };
    HalfRegs hreg[2];
    if (n_mask + 1 < n_ch) {
      load_part(q_begin + (n_mask + 1) * QCH, 0, hreg[0]);
      load_part(q_begin + (n_mask + 1) * QCH, 1, hreg[1]);
    }
    // Exponentials and dP of a sub-chunk, carried from one step to the next
    // (two sets: step j writes set j % 2 and reads the other).
    struct Carry {
      float e1[16], e2[16];  // P1 2^kappa, |lambda| P2 2^kappa
      f32x16 dp;
    };
    Carry cr[2];
    Ops ops;

    // Step j, in two halves of 16 matrix instructions each:
    //   1. the score and dP products of sub-chunk j, with the dV weights and
    //      dS of sub-chunk j - 1 (from its carried exponentials and dP);
    //   2. the dV, dK products of sub-chunk j - 1, with the exponentials of j.
    // Staging: the even step stores part 0 of chunk cb + 1, the odd step
    // part 1 (then a barrier); each then loads the same part of chunk cb + 2.
    auto step = [&](auto has_prev, auto has_cur, auto parity, int j, const Carry &prv, Carry &cur) {
      constexpr bool HP = decltype(has_prev)::value;  // sub-chunk j - 1 exists
      constexpr bool HJ = decltype(has_cur)::value;   // sub-chunk j exists
      constexpr int SUB = decltype(parity)::value;    // j % 2
      constexpr int SUBP = 1 - SUB;                   // (j - 1) % 2
      const int cb = n_mask + (j >> 1);
      lchar *pAq = nullptr, *pAg = nullptr, *pS = nullptr, *pCq = nullptr, *pCg = nullptr, *pSp = nullptr;
      if constexpr (HJ) {
        pAq = lptr(cb % 3, laQ);
        pAg = lptr(cb % 3, laG);
        pS = lptr(cb % 3, lst);
      }
      if constexpr (HP) {
        const int bc = (n_mask + ((j - 1) >> 1)) % 3;
        pCq = lptr(bc, lcQ);
        pCg = lptr(bc, lcG);
        pSp = lptr(bc, lst);
      }
      auto rbyte = [&](int sub, int g) -> uint32_t { return (sub * 32 + ((g & 2) << 3) + (g & 1) * 4) * 4; };
      // Operand i of the score (i < 8: Q1 even, Q2 odd) and dP (i >= 8) products.
      auto fa = [&](int i) -> f16x8 {
        if (i < 8) return *(const DA_LDS f16x8 *)(pAq + ((i & 1) ? OQ2 : OQ1) + (SUB * 32 * QST + (i >> 1) * 16) * 2);
        return *(const DA_LDS f16x8 *)(pAg + OG + (SUB * 32 * GST + (i - 8) * 16) * 2);
      };
      f16x8 oa[16], oc[16];
      f32x4 se[4][2], sl[4][2];  // E1', E2' of j - 1; lse1', lse2' of j (four rows per group)
      auto fetch_e = [&](int g) {
        se[g][0] = *(const DA_LDS f32x4 *)(pSp + OE1 + rbyte(SUBP, g));
        se[g][1] = *(const DA_LDS f32x4 *)(pSp + OE2 + rbyte(SUBP, g));
      };
      auto fetch_l = [&](int g) {
        sl[g][0] = *(const DA_LDS f32x4 *)(pS + OL1 + rbyte(SUB, g));
        sl[g][1] = *(const DA_LDS f32x4 *)(pS + OL2 + rbyte(SUB, g));
      };
      f32x16 s1 = {}, s2 = {};
      if constexpr (HJ) {
        oa[0] = fa(0);
        oa[1] = fa(1);
        cur.dp = f32x16{};
      }
      if constexpr (HP) {
        fetch_e(0);
        fetch_e(1);
      }
      // Half 1.
      float pv[2][3];  // one pair of elementwise results awaiting conversion
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if constexpr (HJ) {
          if (k + 2 < 16) oa[k + 2] = fa(k + 2);
          if (k < 8) {
            if (k & 1) s2 = mfma32(oa[k], kf2[k >> 1], s2);
            else s1 = mfma32(oa[k], kf1[k >> 1], s1);
          } else {
            cur.dp = mfma32(oa[k], vf[k - 8], cur.dp);
          }
          if (k == 12) fetch_l(0);
          if (k == 14) fetch_l(1);
        }
        if constexpr (HP) {
          if ((k & 3) == 0 && k / 4 + 2 < 4) fetch_e(k / 4 + 2);
          if (k >= 14) oc[k - 14] = fetch_c(pCq, pCg, SUBP, k - 14);
          const int r = k;
          const float p1 = prv.e1[r], p2 = prv.e2[r], dpr = prv.dp[r];
          pv[r & 1][0] = fmaf(fold.sig, p2, p1) * fW2;
          pv[r & 1][1] = p1 * (dpr - se[r >> 2][0][r & 3]);
          pv[r & 1][2] = p2 * fmaf(dpr, fold.sig, se[r >> 2][1][r & 3]);
          if (r & 1) {
            const int kc2 = r >> 3, e = r & 7;
            f16x2 a = __builtin_convertvector((f32x2{pv[0][0], pv[1][0]}), f16x2);
            f16x2 b = __builtin_convertvector((f32x2{pv[0][1], pv[1][1]}), f16x2);
            f16x2 d = __builtin_convertvector((f32x2{pv[0][2], pv[1][2]}), f16x2);
            asm volatile("" : "+v"(a), "+v"(b), "+v"(d));  // computed here, not at first use
            ops.w[kc2][e - 1] = a[0];
            ops.w[kc2][e] = a[1];
            ops.b1[kc2][e - 1] = b[0];
            ops.b1[kc2][e] = b[1];
            ops.b2[kc2][e - 1] = d[0];
            ops.b2[kc2][e] = d[1];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // Half 2.
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if constexpr (HP) {
          if (k + 2 < 16) oc[k + 2] = fetch_c(pCq, pCg, SUBP, k + 2);
          mfma_c(k, oc[k], ops);
        }
        if constexpr (HJ) {
          if ((k & 3) == 0 && k / 4 + 2 < 4) fetch_l(k / 4 + 2);
          const int r = k;
          cur.e1[r] = fast_exp2(fmaf(s1[r], c, -sl[r >> 2][0][r & 3]));
          cur.e2[r] = fast_exp2(fmaf(s2[r], c, -sl[r >> 2][1][r & 3]));
          asm volatile("" : "+v"(cur.e1[r]), "+v"(cur.e2[r]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (HJ) {
        if (cb + 1 < n_ch) store_half(smb[(cb + 1) % 3], hreg[SUB], tid, q_begin + (cb + 1) * QCH, S, SUB, fold);
        if constexpr (SUB == 1) __syncthreads();
        if (cb + 2 < n_ch) load_part(q_begin + (cb + 2) * QCH, SUB, hreg[SUB]);
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
    // The last sub-chunk's dV weights and dS, and its dV, dK products.
    step(T{}, F{}, P0{}, J, cr[1], cr[0]);
  }

  // Epilogue: lane = key, registers = channels 8 (r/4) + 4 h + r%4 of each tile.
  if (my_key < S) {
    const float fv = exp2i(-(om + sg));
    const float fk = p.scale * exp2i(-(kap + sg + kv + kq));
    bf16 *dvp = (bf16 *)p.dv + b * p.dvs_b + (int64_t)my_key * p.dvs_s + hd * p.dvs_h;
    bf16 *dk1p = (bf16 *)p.dk1 + b * p.dks_b + (int64_t)my_key * p.dks_s + hd * p.dks_h;
    bf16 *dk2p = (bf16 *)p.dk2 + b * p.dks_b + (int64_t)my_key * p.dks_s + hd * p.dks_h;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int ch = ct * 32 + 8 * g + 4 * h;
        *(bf16x4 *)(dvp + ch) = bf16x4{f2bf(dv[ct][4 * g] * fv), f2bf(dv[ct][4 * g + 1] * fv),
                                       f2bf(dv[ct][4 * g + 2] * fv), f2bf(dv[ct][4 * g + 3] * fv)};
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int ch = dt * 32 + 8 * g + 4 * h;
        *(bf16x4 *)(dk1p + ch) = bf16x4{f2bf(dk1[dt][4 * g] * fk), f2bf(dk1[dt][4 * g + 1] * fk),
                                        f2bf(dk1[dt][4 * g + 2] * fk), f2bf(dk1[dt][4 * g + 3] * fk)};
        *(bf16x4 *)(dk2p + ch) = bf16x4{f2bf(dk2[dt][4 * g] * fk), f2bf(dk2[dt][4 * g + 1] * fk),
                                        f2bf(dk2[dt][4 * g + 2] * fk), f2bf(dk2[dt][4 * g + 3] * fk)};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_dq: query-outer.  Workgroup = 128 queries of one (b, h); wave w owns
// queries q0 + 32 w + 0..31 (lane l % 32).  Streams 64-key tiles of the fp16
// K1, K2, V rows once, forming dS and dQ (E_m comes from bwd_gconv).
constexpr int QB = 128, KT = 64;

struct SmemB {  // swizzled tiles
  f16 k1[KT * D];
  f16 k2[KT * D];
  f16 v[KT * DV];
};

// A key tile is staged global -> registers -> LDS in two halves, each loaded
// while one 32-key sub-tile of the previous tile is computed: the fp16 K1 | K2
// rows, then the fp16 V rows (both formed once per row by bwd_gconv, range
// shifts included; bounded buffer loads, so keys past the end read as zeros).
// Thread tid holds 16-byte pieces tid + NT k (k = 0..3) of the 64 rows of 256
// bytes: row (tid + NT k) / 16, chunk (tid + NT k) % 16.
__device__ __forceinline__ void store_k12(SmemB &sm, const u32x4 (&r)[4], int tid) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + NT * k, row = i >> 4, ch = i & 15;
    *(u32x4 *)(ch < 8 ? sm.k1 + swz_off<D>(row, ch) : sm.k2 + swz_off<D>(row, ch - 8)) = r[k];
  }
}

__device__ __forceinline__ void store_v(SmemB &sm, const u32x4 (&r)[4], int tid) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = tid + NT * k;
    *(u32x4 *)(sm.v + swz_off<DV>(i >> 4, i & 15)) = r[k];
  }
}

// S1^T, S2^T and dP'^T of one 32-key sub-tile (lane = query, registers = keys).
__device__ __forceinline__ void dq_products(const SmemB &sm, int sub, int lk, int lv, const f16x8 *qf1,
                                            const f16x8 *qf2, const f16x8 *gf, f32x16 &s1, f32x16 &s2,
                                            f32x16 &dp) {
  s1 = f32x16{};
  s2 = f32x16{};
  dp = f32x16{};
  // Row krow of each 32-row sub-tile, chunk h + 2 kc: lk = swz_off<D>(krow, h),
  // lv = swz_off<DV>(krow, h) (sub * 32 keeps the row mod 16).
  const f16 *ka1 = sm.k1 + sub * 32 * D;
  const f16 *ka2 = sm.k2 + sub * 32 * D;
  const f16 *va = sm.v + sub * 32 * DV;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    s1 = mfma32(*(const f16x8 *)(ka1 + (lk ^ (16 * kc))), qf1[kc], s1);
    s2 = mfma32(*(const f16x8 *)(ka2 + (lk ^ (16 * kc))), qf2[kc], s2);
  }
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) dp = mfma32(*(const f16x8 *)(va + (lv ^ (16 * kc))), gf[kc], dp);
}

// Elementwise part of one 32 x 32 block of the query-outer kernel (lane =
// query, registers = keys sb + row_of_reg(r, h)): dS_m 2^kappa for both maps
// from the folded row terms L1, L2, E1, E2 (RowFold).  Key sb + o of this
// lane is masked iff o > lim, lim = (last visible key) - sb: one compare per
// score against the register's fixed offset o.
template <bool MASK>
__device__ __forceinline__ void dq_elem(const f32x16 &s1, const f32x16 &s2, const f32x16 &dp, int h, float c,
                                        float L1, float L2, float e1, float e2, float sig, int lim, float *ds1,
                                        float *ds2) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const bool dead = MASK && row_of_reg(r, h) > lim;  // selects the exponent, as in dkdv_elem
    const float p1 = fast_exp2(dead ? -__builtin_inff() : fmaf(s1[r], c, -L1));
    const float p2 = fast_exp2(dead ? -__builtin_inff() : fmaf(s2[r], c, -L2));
    ds1[r] = p1 * (dp[r] - e1);
    ds2[r] = p2 * fmaf(dp[r], sig, e2);
  }
}

__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(BwdParams p, Ws w) {
  __shared__ SmemB smb[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ln = lane & 31, h = lane >> 5;
  const float lam = wave_lambda(p.lq1, p.lk1, p.lq2, p.lk2, p.lambda_dim, p.lambda_fixed, p.lambda_init);
  const int BH = p.B * p.H;
  const int n_qt = (p.S + QB - 1) / QB;
  const int bh = blockIdx.x % BH;
  const int qt = p.causal ? n_qt - 1 - blockIdx.x / BH : blockIdx.x / BH;
  const int b = bh / p.H, hd = bh % p.H;
  const int S = p.S;
  const int q0 = qt * QB, qw = q0 + wave * 32, my_q = qw + ln;
  const float sg = w.scales[bh * 8 + 0], kap = w.scales[bh * 8 + 1];
  const float kq = w.scales[bh * 8 + 3], kk = w.scales[bh * 8 + 4], kv = w.scales[bh * 8 + 5];
  const VScale scq((int)kq);
  // fp16 Q, K, V are Q 2^kq, K 2^kk, V 2^kv: S' = S 2^(kq + kk), dP' = dP 2^(sg + kv).
  const float c = p.scale * kLog2e * exp2i(-(kq + kk));
  const int64_t statb = (int64_t)bh * S;
  const bool qok = my_q < S;

  // B operands: Q1, Q2 (for S^T = K Q^T) and g' (for dP'^T = V g'^T), fp16.
  f16x8 qf1[4], qf2[4], gf[8];
  {
    const bf16 *q1 = (const bf16 *)p.q1 + b * p.qs_b + (int64_t)my_q * p.qs_s + hd * p.qs_h + 8 * h;
    const bf16 *q2 = (const bf16 *)p.q2 + b * p.qs_b + (int64_t)my_q * p.qs_s + hd * p.qs_h + 8 * h;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      qf1[kc] = qok ? to_f16x8(*(const u32x4 *)(q1 + kc * 16), scq) : f16x8{};
      qf2[kc] = qok ? to_f16x8(*(const u32x4 *)(q2 + kc * 16), scq) : f16x8{};
    }
    const f16 *gp = w.gh + (statb + my_q) * DV + 8 * h;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) gf[kc] = qok ? *(const f16x8 *)(gp + kc * 16) : f16x8{};
  }
  // The row statistics folded as in the key-outer kernel (RowFold): the
  // score loop forms P1 2^kappa, |lambda| P2 2^kappa and dS_m 2^kappa.
  const RowFold fold = row_fold(lam, exp2i(sg + kv), kap);
  const float L1 = qok ? fmaf(p.lse1[statb + my_q], kLog2e, -kap) : __builtin_inff();
  const float L2 = qok ? fmaf(p.lse2[statb + my_q], kLog2e, -(kap + fold.l2lam)) : __builtin_inff();

  const int kend = p.causal ? min(S, q0 + QB) : S;
  const int n_kt = (kend + KT - 1) / KT;
  const int krow = row_perm(ln);
  const int lk = swz_off<D>(krow, h), lv = swz_off<DV>(krow, h);
  const TrLane trk = tr_lane<D>(lane);
  const int q_last = qw + 31;

  // Last key this query sees (the masks as one threshold per block).
  const int key_lim = p.causal ? min(my_q, S - 1) : S - 1;
  // E_m' = g' . A_m for this query (scaled like dP'), E2 times -sigma.
  const float e1 = qok ? w.e1[statb + my_q] * fold.fE : 0.f;
  const float e2 = qok ? -fold.sig * w.e2[statb + my_q] * fold.fE : 0.f;

  // ---- dS and dQ
  f32x16 dq1[2], dq2[2];
  dq1[0] = dq1[1] = dq2[0] = dq2[1] = f32x16{};
  // Key tiles double-buffered in LDS; tile kt + 1 is staged in two halves
  // (K1 and K2 during sub-tile 0 of tile kt, V during sub-tile 1), so only
  // one half is held in registers at a time; one barrier per tile.
  const __amdgpu_buffer_rsrc_t rsk = row_rsrc(w.kh + statb * (2 * D), S), rsv = row_rsrc(w.vh + statb * DV, S);
  u32x4 nx[4];
  load_rows(rsk, 0, tid, nx);
  store_k12(smb[0], nx, tid);
  load_rows(rsv, 0, tid, nx);
  store_v(smb[0], nx, tid);
  __syncthreads();
  // One key tile; MASKED applies the causal and key-range masks, which only
  // the tiles from the query tile's start on (causal) and a partial last tile
  // need: two loops, so the interior one carries no mask arithmetic.
  auto tile = [&](auto masked, int kt) {
    constexpr bool MASKED = decltype(masked)::value;
    const SmemB &sm = smb[kt & 1];
    SmemB &sn = smb[(kt + 1) & 1];
    const bool more = kt + 1 < n_kt;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      if (more) {
        load_rows(sub == 0 ? rsk : rsv, (kt + 1) * KT, tid, nx);
      }
      const int sb = kt * KT + sub * 32;
      if (sb < S && !(p.causal && sb > q_last)) {
      f32x16 s1, s2, dp;
      dq_products(sm, sub, lk, lv, qf1, qf2, gf, s1, s2, dp);
      float ds1[16], ds2[16];
      dq_elem<MASKED>(s1, s2, dp, h, c, L1, L2, e1, e2, fold.sig, key_lim - sb, ds1, ds2);
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) {
        const f16x8 b1 = pack8h(ds1 + 8 * kc2), b2 = pack8h(ds2 + 8 * kc2);
        const int r0 = sub * 32 + kc2 * 16;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          dq1[dt] = mfma32(tr_operand_swz<D>(sm.k1, trk, r0, dt * 32), b1, dq1[dt]);
          dq2[dt] = mfma32(tr_operand_swz<D>(sm.k2, trk, r0, dt * 32), b2, dq2[dt]);
        }
      }
      }
      if (more) {
        if (sub == 0) store_k12(sn, nx, tid);
        else store_v(sn, nx, tid);
      }
    }
    __syncthreads();
  };
  const int n_full = min(p.causal ? q0 / KT : n_kt, S / KT);  // tiles no query of the tile needs masked
  int kt = 0;
  for (; kt < n_full; ++kt) tile(std::false_type{}, kt);
  for (; kt < n_kt; ++kt) tile(std::true_type{}, kt);
  if (qok) {
    const float fq = p.scale * exp2i(-(kap + sg + kv + kk));
    bf16 *d1 = (bf16 *)p.dq1 + b * p.dqs_b + (int64_t)my_q * p.dqs_s + hd * p.dqs_h;
    bf16 *d2 = (bf16 *)p.dq2 + b * p.dqs_b + (int64_t)my_q * p.dqs_s + hd * p.dqs_h;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = dt * 32 + 8 * g + 4 * h;
        *(bf16x4 *)(d1 + ch) = bf16x4{f2bf(dq1[dt][4 * g] * fq), f2bf(dq1[dt][4 * g + 1] * fq),
                                      f2bf(dq1[dt][4 * g + 2] * fq), f2bf(dq1[dt][4 * g + 3] * fq)};
        *(bf16x4 *)(d2 + ch) = bf16x4{f2bf(dq2[dt][4 * g] * fq), f2bf(dq2[dt][4 * g + 1] * fq),
                                      f2bf(dq2[dt][4 * g + 2] * fq), f2bf(dq2[dt][4 * g + 3] * fq)};
      }
  }
}

// ---------------------------------------------------------------------------
// bwd_dlsum: one workgroup of NTS threads per (b, h): the (batch, head) sum of
// the rows' dL/dlambda shares, in a fixed order (strided per thread, then the
// wave, then the waves' tree).
__global__ __launch_bounds__(NTS) void bwd_dlsum_kernel(BwdParams p, Ws w) {
  __shared__ float red[NWS];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = (int64_t)bh * p.S;
  float dl = 0.f;
  for (int s = tid; s < p.S; s += NTS) dl += w.dlam_row[base + s];
  for (int o = 32; o > 0; o >>= 1) dl += __shfl_xor(dl, o);
  if (lane == 0) red[wave] = dl;
  __syncthreads();
  if (tid == 0) w.dlam_bh[bh] = tree_sum(red);
}

// ---------------------------------------------------------------------------
// bwd_lambda: one workgroup; dL/dlambda = sum of the (batch, head) sums that
// bwd_dlsum formed, in a fixed order, then the chain rule into the four
// lambda vectors.
__global__ __launch_bounds__(NT) void bwd_lambda_kernel(BwdParams p, Ws w) {
  __shared__ float red[NT / 64];
  __shared__ float dl_sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float s = 0.f;
  for (int i = tid; i < p.B * p.H; i += NT) s += w.dlam_bh[i];
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (tid == 0) {
    dl_sh = (red[0] + red[1]) + (red[2] + red[3]);
    if (p.dlambda) *p.dlambda = dl_sh;
  }
  __syncthreads();
  if (p.lq1 == nullptr || wave != 0) return;
  const float dl = dl_sh;
  float al = 0.f, be = 0.f;
  for (int i = lane; i < p.lambda_dim; i += 64) {
    al = fmaf(p.lq1[i], p.lk1[i], al);
    be = fmaf(p.lq2[i], p.lk2[i], be);
  }
  al = wave_sum(al);
  be = wave_sum(be);
  const float ca = dl * expf(al), cb = -dl * expf(be);
  for (int i = lane; i < p.lambda_dim; i += 64) {
    p.dlq1[i] = ca * p.lk1[i];
    p.dlk1[i] = ca * p.lq1[i];
    p.dlq2[i] = cb * p.lk2[i];
    p.dlk2[i] = cb * p.lq2[i];
  }
}

}  // namespace

size_t bwd_workspace_bytes(int B, int S, int H, int d, int dv) {
  (void)d;
  (void)dv;
  return ws_bytes(B, S, H);
}

hipError_t launch_bwd(const BwdParams &p, hipStream_t st) {
  Ws w = carve(p.workspace, p.B, p.S, p.H);
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  hipLaunchKernelGGL(bwd_pre_kernel, dim3((rows + RPB - 1) / RPB), dim3(NT), 0, st, p, w);
  hipLaunchKernelGGL(bwd_scales_kernel, dim3(p.B * p.H), dim3(NTS), 0, st, p, w);
  hipLaunchKernelGGL(bwd_gconv_kernel, dim3((rows + RPB - 1) / RPB), dim3(NT), 0, st, p, w);
  const int n_qt = (p.S + QB - 1) / QB;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(n_qt * p.B * p.H), dim3(NT), 0, st, p, w);
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((p.S + KVB - 1) / KVB * p.B * p.H), dim3(NT), 0, st, p, w);
  hipLaunchKernelGGL(bwd_dlsum_kernel, dim3(p.B * p.H), dim3(NTS), 0, st, p, w);
  hipLaunchKernelGGL(bwd_lambda_kernel, dim3(1), dim3(NT), 0, st, p, w);
  return hipGetLastError();
}

}  // namespace diffattn
