// Host-side launchers of the libdiffattn kernels (internal to the library).
// Arguments reaching these have been validated by the C ABI layer (api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace diffattn {

// Everything the forward kernels read.  Strides in elements.
struct FwdParams {
  const void *q1, *k1, *q2, *k2, *v;
  int64_t qs_b, qs_s, qs_h, ks_b, ks_s, ks_h, vs_b, vs_s, vs_h, os_b, os_s, os_h;
  void *out;
  int B, S, H;
  int causal, norm;
  const float *lq1, *lk1, *lq2, *lk2;
  int lambda_dim;
  float lambda_fixed, lambda_init;
  float scale;  // softmax scale (> 0)
  float eps;
  float *lambda_out;
  float *lse1, *lse2, *rstd, *o_pre, *a2;  // training saves (all or none)
  const unsigned *vpart;  // V range partials (vrange.hip): the fp8-logit forward
  const _Float16 *v16;    // the one-pass forward's fp16 copy of V and its
  const int *vexp;        // per-256-row-chunk shifts (vrange.hip)
};

struct BwdParams {
  const void *q1, *k1, *q2, *k2, *v, *dout;
  int64_t qs_b, qs_s, qs_h, ks_b, ks_s, ks_h, vs_b, vs_s, vs_h, ds_b, ds_s, ds_h;
  int B, S, H;
  int causal, norm;
  const float *lq1, *lk1, *lq2, *lk2;
  int lambda_dim;
  float lambda_fixed, lambda_init;
  float scale;
  const float *lse1, *lse2, *rstd, *o_pre, *a2;
  void *dq1, *dk1, *dq2, *dk2, *dv;
  int64_t dqs_b, dqs_s, dqs_h, dks_b, dks_s, dks_h, dvs_b, dvs_s, dvs_h;
  float *dlq1, *dlk1, *dlq2, *dlk2, *dlambda;
  void *workspace;
};

struct DecodeParams {
  const void *q, *k, *v;
  int64_t qs_b, qs_h, kvs_b, kvs_s, kvs_h, os_b, os_h;
  const int32_t *seqlens;
  const float *lam;
  int64_t lam_stride_b;
  void *out;
  int B, Hq, Hkv, D, L;
  int splits, chunk;  // keys per split
  float scale;
  float *part_o;   // [B, Hq, splits, D]
  float *part_ml;  // [B, Hq, splits, 2]
};

// DIFF V1 decode step over a K1/K2/V cache (d = 64, dv = 128).
struct V1DecodeParams {
  const void *q1, *q2, *k1, *k2, *v;
  int64_t qs_b, qs_h, ks_b, ks_s, ks_h, vs_b, vs_s, vs_h, os_b, os_h;
  const int32_t *seqlens;
  const float *lq1, *lk1, *lq2, *lk2;
  int lambda_dim;
  float lambda_fixed, lambda_init;
  int norm;
  float eps;
  void *out;
  int B, H, L;
  int splits, chunk;
  float scale;
  float *part_o;   // [B, H, 2, splits, dv]
  float *part_ml;  // [B, H, 2, splits, 2]
};

// DIFF V2 prefill forward: Hq query heads over Hkv KV heads, bf16, D = 128.
struct V2FwdParams {
  const void *q, *k, *v;
  int64_t qs_b, qs_s, qs_h, kvs_b, kvs_s, kvs_h, os_b, os_s, os_h;
  const float *lam;  // sigmoid input per (batch, token, pair)
  int64_t ls_b, ls_s, ls_p;
  void *out;
  int B, S, Hq, Hkv;
  int causal;
  float scale;
  float *lse;            // training saves (all or none): [B, Hq, S] natural-log partition functions,
  float *a_even, *a_odd; // [B, S, Hq/2, D] each head's own output (attn_2p, attn_2p+1)
  // Block-sparse selection (null for dense): per (batch, pair, 128-row query
  // tile), blk_cnt entries of blk_idx (64-key tile indices, ascending).
  const int32_t *blk_idx, *blk_cnt;
  int max_blocks;
  const unsigned *vpart;  // V range partials per (batch, KV head) (vrange.hip)
};

// DIFF V2 prefill backward (bf16, D = 128).
struct V2BwdParams {
  const void *q, *k, *v, *dout;
  int64_t qs_b, qs_s, qs_h, kvs_b, kvs_s, kvs_h, ds_b, ds_s, ds_h;
  const float *lam;
  int64_t ls_b, ls_s, ls_p;
  const float *lse, *a_even, *a_odd;
  void *dq, *dk, *dv;
  int64_t dqs_b, dqs_s, dqs_h, dkvs_b, dkvs_s, dkvs_h;
  float *dlam;  // [B, S, Hq/2]
  int B, S, Hq, Hkv;
  int causal;
  float scale;
  void *workspace;
};

// Range pass over V (vrange.hip): per (batch, head) slice of a bf16
// [B, S, H, C] tensor, the largest magnitude of every 256-row chunk (bf16
// bits) into part[B * H][vrange_chunks(S)].
struct VRangeParams {
  const void *v;
  int64_t vs_b, vs_s, vs_h;
  int B, S, H;
  unsigned *part;
};
constexpr int kVRangeRows = 256;
inline __host__ __device__ int vrange_chunks(int S) { return (S + kVRangeRows - 1) / kVRangeRows; }
inline size_t vrange_bytes(int B, int S, int H) { return ((size_t)B * H * vrange_chunks(S) * 4 + 255) & ~(size_t)255; }
hipError_t launch_vrange(const VRangeParams &p, int channels, hipStream_t st);
// fp16 copy of V for the one-pass forward: v16 [B * H, S, 128], each 256-row
// chunk times 2^kexp[B * H][vrange_chunks(S)] (vrange.hip).
struct VConvParams {
  const void *v;
  int64_t vs_b, vs_s, vs_h;
  int B, S, H;
  _Float16 *v16;
  int *kexp;
};
inline size_t vconv_bytes(int B, int S, int H) {
  return (((size_t)B * H * S * 128 * 2 + 255) & ~(size_t)255) + vrange_bytes(B, S, H);
}
hipError_t launch_vconv(const VConvParams &p, hipStream_t st);

// Reference vector-ALU forward: any supported (d, dv), f32 or bf16.
hipError_t launch_fwd_generic(const FwdParams &p, int dtype, int d, int dv, hipStream_t st);
// Fused bf16 matrix-core forward, d = 64, dv = 128 (one-pass kernel, with or
// without the training saves).  The workspace holds the fp16 copy of V and
// its per-chunk shifts (vrange.hip).
size_t fwd_workspace_bytes(int B, int S, int H);
hipError_t launch_fwd(const FwdParams &p, void *workspace, hipStream_t st);
// The same forward with fp8 e4m3 score operands (per-row power-of-two absmax
// scales); the workspace holds the codes and exponents.
size_t fwd_fp8_workspace_bytes(int B, int S, int H);
hipError_t launch_fwd_fp8(const FwdParams &p, void *workspace, hipStream_t st);

hipError_t launch_fwd_v2(const V2FwdParams &p, hipStream_t st);
size_t v2_bwd_workspace_bytes(int B, int S, int Hq, int Hkv);
hipError_t launch_v2_bwd(const V2BwdParams &p, hipStream_t st);

size_t bwd_workspace_bytes(int B, int S, int H, int d, int dv);
hipError_t launch_bwd(const BwdParams &p, hipStream_t st);

size_t decode_workspace_bytes(int B, int Hq, int D, int splits);
size_t v1_decode_workspace_bytes(int B, int H, int splits);
hipError_t launch_v1_decode(const V1DecodeParams &p, int dtype, hipStream_t st);
int decode_max_chunk();
int decode_auto_splits(int B, int Hkv, int L);
hipError_t launch_decode(const DecodeParams &p, int dtype, hipStream_t st);
// Fixed device scratch of the allocation-free V2 decode: its size, and its
// address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
void *decode_scratch(hipError_t *err);

}  // namespace diffattn
