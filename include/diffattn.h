/*
 * diffattn.h - C ABI of libdiffattn.so: multi-head differential attention on
 * AMD Instinct MI355X (gfx950).
 *
 * Operations (citations name the pages that define them):
 *   - DIFF V1 forward: per head, two softmax maps softmax(s Q1 K1^T) and
 *     softmax(s Q2 K2^T), s = 1/sqrt(d), over one value tensor twice as wide as
 *     the query/key width, combined as (map1 - lambda * map2) V; then per-head
 *     RMSNorm scaled by the fixed multiplier (1 - lambda_init)
 *     [Ultralytics glossary "Differential Transformer", section "How
 *     differential attention works"; esgcw.com.cn write-up, sections on the
 *     differential attention operator and multi-head differential attention].
 *     lambda = exp(<lq1,lk1>) - exp(<lq2,lk2>) + lambda_init, one scalar per
 *     layer shared by all heads; lambda_init = 0.8 - 0.6 exp(-0.3 (l - 1))
 *     [neuralnode.tistory.com "DIFF V2 technical innovations", section "DIFF V1
 *     limits"; esgcw.com.cn write-up, differential attention section].
 *   - DIFF V1 backward: gradients of the forward by the chain rule (the pages
 *     print none; the forward above defines them).
 *   - DIFF V2 decode: 2h query heads over h KV heads; each query head runs
 *     ordinary softmax attention over the KV cache, then heads split into even
 *     and odd along the head axis are combined as attn_even - sigmoid(lam) *
 *     attn_odd; pairs sit inside one grouped-query group so the KV cache is read
 *     once [neuralnode.tistory.com, section "DIFF V2 innovations" items 1, 2, 5;
 *     section "GQA compatibility"].
 *   - DIFF V2 prefill forward: the same operator over whole sequences (causal
 *     or not), with a sigmoid input per token and pair [same sections; item 5
 *     makes lambda per token and per head].
 *   - DIFF V2 prefill backward: its gradients by the chain rule.
 *   - Block-sparse DIFF V2 prefill forward (key blocks selected per head pair).
 *   - DIFF V1 decode: the V1 operator for one new token over a K1/K2/V cache.
 *   - DIFF V1 forward with fp8 e4m3 attention logits (per-row absmax scaling).
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is a device pointer owned by the caller (for example
 *     torch tensor storage).  The library allocates no device memory and keeps
 *     no state beyond a per-thread copy of the last error message.
 *   - Tensors are [batch, seq, head, channel] with the channel dimension
 *     contiguous; the other three strides are passed in elements (int64).
 *   - Calls are asynchronous on the HIP stream passed as `stream`
 *     (hipStream_t; NULL = the default stream) and never synchronise.
 *   - Arguments are validated on the host before any launch; on an error the
 *     function returns a negative status, launches nothing and writes nothing.
 *     diffattn_last_error() then describes the failure.
 *   - No C++ exception crosses this boundary.
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define DIFFATTN_OK 0
#define DIFFATTN_ERR_INVALID_ARGUMENT (-1) /* null pointer, bad size or stride      */
#define DIFFATTN_ERR_UNSUPPORTED (-2)      /* dtype / head-size combination absent  */
#define DIFFATTN_ERR_WORKSPACE (-3)        /* workspace missing or too small        */
#define DIFFATTN_ERR_HIP (-4)              /* HIP runtime or launch failure         */

/* Element types of the activation tensors. */
#define DIFFATTN_F32 0
#define DIFFATTN_BF16 1

/*
 * Forward arguments.
 *   Shapes: q1, k1, q2, k2 [B, S, H, d]; v and out [B, S, H, dv].  Query and
 *   key lengths are equal (S).  Supported: bf16 with d = 64, dv = 128 (the
 *   fused matrix-core kernel); f32 or bf16 with (d, dv) in {(8,16), (16,32),
 *   (32,64), (64,128), (128,256)} through the reference vector kernel.
 *   causal: query i sees keys j <= i.  norm: 1 applies the per-head RMSNorm
 *   times (1 - lambda_init); 0 returns the raw combine (map1 - lambda map2) V.
 *   lambda: from the four device vectors lq1, lk1, lq2, lk2 (float32,
 *   lambda_dim each) when all four are non-NULL, else lambda_fixed.
 *   softmax_scale <= 0 selects 1/sqrt(d).  eps sits inside the RMS root.
 *   lambda_out (optional, device float32[1]) receives the lambda used.
 *   Training saves (all five non-NULL, or all NULL; bf16 fused path only;
 *   o_pre and a2 16-byte aligned, else DIFFATTN_ERR_UNSUPPORTED):
 *     lse1, lse2, rstd: float32 [B, H, S] contiguous - natural-log partition
 *       function of each map's scaled scores, and the RMSNorm reciprocal
 *       root (1 when norm = 0);
 *     o_pre, a2: float32 [B, S, H, dv] contiguous - the un-normalised combine
 *       O = (map1 - lambda map2) V and the second map's output A2 = map2 V.
 *   workspace: device memory of at least diffattn_fwd_workspace_size() bytes,
 *     16-byte aligned (contents on entry do not matter), for the bf16
 *     matrix-core path: a first pass over V writes there an fp16 copy of V
 *     with one power-of-two shift per 256-row chunk, so V may take any finite
 *     bf16 magnitude (B x H x S x 256 bytes and a few bytes per 256 rows,
 *     with or without training saves).  Not read by the vector-kernel paths
 *     (size 0) nor by diffattn_fwd_fp8, which takes its own workspace.
 *   batch = 0 or seqlen = 0 is an empty problem: DIFFATTN_OK, nothing read.
 */
typedef struct diffattn_fwd_args {
  int32_t batch, seqlen, heads, head_dim, v_dim;
  int32_t dtype, causal, norm;
  const void *q1, *k1, *q2, *k2, *v;
  int64_t q_stride[3]; /* batch, seq, head strides of q1 and q2 */
  int64_t k_stride[3]; /* of k1 and k2 */
  int64_t v_stride[3];
  int64_t o_stride[3]; /* of out */
  const float *lq1, *lk1, *lq2, *lk2;
  int32_t lambda_dim;
  float lambda_fixed;
  float lambda_init;
  float softmax_scale;
  float eps;
  void *out;
  float *lambda_out;
  float *lse1, *lse2, *rstd;
  float *o_pre, *a2;
  void *workspace; /* bf16 matrix-core path; see diffattn_fwd_workspace_size */
  size_t workspace_bytes;
} diffattn_fwd_args;

/*
 * Backward arguments: gradients of L = <dout, out> for a forward with the same
 * inputs and flags (bf16, d = 64, dv = 128, causal or not).
 *   Needs the five training saves of that forward (lse1, lse2, rstd, o_pre,
 *   a2), o_pre and a2 16-byte aligned (else DIFFATTN_ERR_UNSUPPORTED).
 *   dout has strides do_stride; outputs dq1, dq2 (strides dq_stride), dk1,
 *   dk2 (dk_stride), dv (dv_stride) in the activation dtype.
 *   With the four lambda vectors given, dlq1, dlk1, dlq2, dlk2 (device
 *   float32[lambda_dim], all four required) receive their gradients; dlambda
 *   (optional, device float32[1]) receives dL/dlambda in either mode.
 *   workspace: device memory of at least diffattn_bwd_workspace_size() bytes,
 *   256-byte aligned; its contents on entry do not matter.
 */
typedef struct diffattn_bwd_args {
  int32_t batch, seqlen, heads, head_dim, v_dim;
  int32_t dtype, causal, norm;
  const void *q1, *k1, *q2, *k2, *v;
  int64_t q_stride[3], k_stride[3], v_stride[3];
  const void *dout;
  int64_t do_stride[3];
  const float *lq1, *lk1, *lq2, *lk2;
  int32_t lambda_dim;
  float lambda_fixed;
  float lambda_init;
  float softmax_scale;
  const float *lse1, *lse2, *rstd, *o_pre, *a2;
  void *dq1, *dk1, *dq2, *dk2, *dv;
  int64_t dq_stride[3], dk_stride[3], dv_stride[3];
  float *dlq1, *dlk1, *dlq2, *dlk2;
  float *dlambda;
  void *workspace;
  size_t workspace_bytes;
} diffattn_bwd_args;

/*
 * DIFF V2 decode arguments (one new query token per sequence).
 *   q [B, Hq, D] (strides q_stride: batch, head); k_cache, v_cache
 *   [B, S_kv, Hkv, D] sharing kv_stride (batch, seq, head).  Query head t
 *   reads KV head t / (Hq / Hkv); Hq / Hkv must be even so that each even/odd
 *   pair shares its KV head.  Supported: bf16 or f32, D in {64, 128}.
 *   seqlens: device int32[B] (NULL = every sequence has kv_len keys); values
 *   are clamped to [0, kv_len]; a length of 0 yields a zero output row.
 *   lam: device float32, element (b, p) at lam[b * lam_stride_b + p] for
 *   p < Hq/2 (lam_stride_b = 0 shares one [Hq/2] vector across the batch).
 *   out [B, Hq/2, D] (strides o_stride: batch, head), in the cache dtype:
 *   out[b, p] = attn[b, 2p] - sigmoid(lam[b, p]) * attn[b, 2p + 1].
 *   softmax_scale <= 0 selects 1/sqrt(D).  num_splits: number of key chunks
 *   each (batch, KV head) is split into (0 = chosen by the library).
 *   workspace: at least diffattn_v2_decode_workspace_size() bytes.
 */
typedef struct diffattn_v2_decode_args {
  int32_t batch, q_heads, kv_heads, head_dim, kv_len;
  int32_t dtype;
  const void *q;
  int64_t q_stride[2];
  const void *k_cache, *v_cache;
  int64_t kv_stride[3];
  const int32_t *seqlens;
  const float *lam;
  int64_t lam_stride_b;
  float softmax_scale;
  void *out;
  int64_t o_stride[2];
  int32_t num_splits;
  void *workspace;
  size_t workspace_bytes;
} diffattn_v2_decode_args;

/*
 * DIFF V2 prefill forward arguments (whole sequences, training or prefill).
 *   q [B, S, Hq, D] (strides q_stride: batch, seq, head); k, v [B, S, Hkv, D]
 *   sharing kv_stride; out [B, S, Hq/2, D] (strides o_stride).  Query head t
 *   reads KV head t / (Hq / Hkv); Hq / Hkv must be even so that each even/odd
 *   pair (2p, 2p + 1) shares its KV head.  Supported: bf16 with D = 128,
 *   16-byte aligned q, k, v, out and strides that are multiples of 8.
 *   lam: device float32, element (b, i, p) at lam[b * lam_stride[0] +
 *   i * lam_stride[1] + p * lam_stride[2]] (strides >= 0; a zero stride
 *   broadcasts, e.g. one value per pair shared by all tokens).
 *   out[b, i, p] = attn_2p[b, i] - sigmoid(lam[b, i, p]) * attn_2p+1[b, i],
 *   where attn_t = softmax(s q_t K^T) V over keys j <= i (causal) or all keys,
 *   in fp32 arithmetic with fp16/bf16 matrix-core operands, rounded to bf16.
 *   softmax_scale <= 0 selects s = 1/sqrt(D).
 *   Training saves (all three non-NULL, or all NULL), float32, contiguous:
 *     lse [B, Hq, S]: natural-log partition function of each query head's
 *       scaled scores;
 *     a_even, a_odd [B, S, Hq/2, D]: each head's own output attn_2p and
 *       attn_2p+1.
 *   workspace: device memory of at least diffattn_v2_fwd_workspace_size()
 *     bytes, 16-byte aligned, contents on entry irrelevant (shared with
 *     diffattn_v2_fwd_sparse): the largest |v| of every 256-row chunk of each
 *     (batch, KV head) slice, from which each workgroup picks the power of two
 *     its fp16 copy of V is scaled by, so V may take any finite bf16 magnitude.
 *   batch = 0 or seqlen = 0 is an empty problem: DIFFATTN_OK, nothing read.
 */
typedef struct diffattn_v2_fwd_args {
  int32_t batch, seqlen, q_heads, kv_heads, head_dim;
  int32_t dtype, causal;
  const void *q, *k, *v;
  int64_t q_stride[3];  /* batch, seq, head */
  int64_t kv_stride[3]; /* of k and v */
  const float *lam;
  int64_t lam_stride[3]; /* batch, token, pair */
  float softmax_scale;
  void *out;
  int64_t o_stride[3];
  float *lse;   /* training saves, all three or none (see above) */
  float *a_even;
  float *a_odd;
  void *workspace; /* see diffattn_v2_fwd_workspace_size */
  size_t workspace_bytes;
} diffattn_v2_fwd_args;

/*
 * DIFF V2 prefill backward arguments: gradients of L = <dout, out> for a
 * diffattn_v2_fwd call with the same inputs and flags that wrote the three
 * training saves (bf16, D = 128).
 *   dout [B, S, Hq/2, D] (strides do_stride).  Outputs: dq [B, S, Hq, D]
 *   (strides dq_stride); dk, dv [B, S, Hkv, D] sharing dkv_stride (summed over
 *   every query head that reads the KV head), all bf16; dlam: device float32
 *   [B, S, Hq/2] contiguous, the gradient for a separate lam value per
 *   (batch, token, pair) (for a broadcast lam, sum it over the broadcast axes).
 *   Every output is fully written; nothing is accumulated into.
 *   workspace: at least diffattn_v2_bwd_workspace_size() bytes, 256-byte
 *   aligned; its contents on entry do not matter.
 */
typedef struct diffattn_v2_bwd_args {
  int32_t batch, seqlen, q_heads, kv_heads, head_dim;
  int32_t dtype, causal;
  const void *q, *k, *v;
  int64_t q_stride[3];
  int64_t kv_stride[3];
  const float *lam;
  int64_t lam_stride[3];
  float softmax_scale;
  const void *dout;
  int64_t do_stride[3];
  const float *lse, *a_even, *a_odd;
  void *dq;
  int64_t dq_stride[3];
  void *dk, *dv;
  int64_t dkv_stride[3];
  float *dlam;
  void *workspace;
  size_t workspace_bytes;
} diffattn_v2_bwd_args;

/*
 * DIFF V1 decode arguments (one new query token per sequence) over a cache of
 * K1, K2 and V [glossary page, section "How differential attention works";
 * news write-up, multi-head section; the V2 page's section "DIFF V1 limits"
 * names this cache layout's decode cost, V read once per map].  V is read
 * once here for both maps.
 *   q1, q2 [B, H, d] sharing q_stride (batch, head); k1_cache, k2_cache
 *   [B, S_kv, H, d] sharing k_stride (batch, seq, head); v_cache
 *   [B, S_kv, H, dv] (v_stride).  Supported: bf16 or f32, d = 64, dv = 128;
 *   caches 16-byte aligned with row strides that keep rows 16-byte aligned.
 *   seqlens: device int32[B] (NULL = every sequence has kv_len keys); values
 *   are clamped to [0, kv_len]; a length of 0 yields a zero output row.
 *   lambda: from the four device vectors lq1, lk1, lq2, lk2 (float32,
 *   lambda_dim each) when all four are non-NULL, else lambda_fixed.
 *   out [B, H, dv] (strides o_stride: batch, head), in the cache dtype:
 *   (map1 - lambda map2) V over the cached keys, then with norm = 1 the
 *   per-head RMSNorm (eps inside the root) times (1 - lambda_init).
 *   softmax_scale <= 0 selects 1/sqrt(d).  num_splits: key chunks per
 *   (batch, head) (0 = chosen by the library).  workspace: at least
 *   diffattn_v1_decode_workspace_size() bytes, 16-byte aligned.
 */
typedef struct diffattn_v1_decode_args {
  int32_t batch, heads, head_dim, v_dim, kv_len;
  int32_t dtype, norm;
  const void *q1, *q2;
  int64_t q_stride[2];
  const void *k1_cache, *k2_cache;
  int64_t k_stride[3];
  const void *v_cache;
  int64_t v_stride[3];
  const int32_t *seqlens;
  const float *lq1, *lk1, *lq2, *lk2;
  int32_t lambda_dim;
  float lambda_fixed;
  float lambda_init;
  float softmax_scale;
  float eps;
  void *out;
  int64_t o_stride[2];
  int32_t num_splits;
  void *workspace;
  size_t workspace_bytes;
} diffattn_v1_decode_args;

/* Forward pass. Returns DIFFATTN_OK or a negative status. */
int diffattn_fwd(const diffattn_fwd_args *args, void *stream);

/* Workspace bytes diffattn_fwd needs for these arguments (0: none needed). */
size_t diffattn_fwd_workspace_size(const diffattn_fwd_args *args);

/*
 * Forward pass with fp8 attention logits: Q1, K1, Q2, K2 are quantised per row
 * (one token of one head) to fp8 e4m3 with a power-of-two absmax scale (e the
 * smallest integer with max|row| 2^-e <= 448, clamped to [-120, 120]; codes
 * rounded to nearest even), and the score products use the dequantised
 * values; everything else is diffattn_fwd [the low-bit attention-logit
 * quantisation and "low-bit FlashAttention" discussed on the V2 page's outlook
 * section and the news write-up].  Same arguments as diffattn_fwd without
 * training saves; supported: bf16 with head_dim 64, v_dim 128.  workspace: at
 * least diffattn_fwd_fp8_workspace_size() bytes, 256-byte aligned (it receives
 * the codes, their exponents and V's range record; args->workspace is not read).
 */
int diffattn_fwd_fp8(const diffattn_fwd_args *args, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes diffattn_fwd_fp8 needs for these arguments (0 if invalid). */
size_t diffattn_fwd_fp8_workspace_size(const diffattn_fwd_args *args);

/* Backward pass. Returns DIFFATTN_OK or a negative status. */
int diffattn_bwd(const diffattn_bwd_args *args, void *stream);

/* Workspace bytes diffattn_bwd needs for these arguments (0 if invalid). */
size_t diffattn_bwd_workspace_size(const diffattn_bwd_args *args);

/* DIFF V2 decode step. Returns DIFFATTN_OK or a negative status. */
int diffattn_v2_decode(const diffattn_v2_decode_args *args, void *stream);

/* Workspace bytes diffattn_v2_decode needs for these arguments (0 if invalid). */
size_t diffattn_v2_decode_workspace_size(const diffattn_v2_decode_args *args);

/*
 * DIFF V2 decode step that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid it).  Same arguments and results as
 * diffattn_v2_decode except that workspace and workspace_bytes are ignored:
 * the split partials go to a fixed scratch array the library holds on each
 * GPU it runs on (DIFFATTN_DECODE_SCRATCH_BYTES, kept until the process ends;
 * the array's address is looked up once per device).  A call whose partials
 * need more than that (diffattn_v2_decode_workspace_size > the limit) returns
 * DIFFATTN_ERR_WORKSPACE without launching.  Every call on one GPU shares that
 * GPU's scratch: calls that overlap in time on one GPU (different streams,
 * different threads) race and must be serialised by the caller.  The scratch
 * needs no clearing (the split kernel writes every partial it reads).
 */
#define DIFFATTN_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int diffattn_v2_decode_noalloc(const diffattn_v2_decode_args *args, void *stream);

/* DIFF V1 decode step. Returns DIFFATTN_OK or a negative status. */
int diffattn_v1_decode(const diffattn_v1_decode_args *args, void *stream);

/* Workspace bytes diffattn_v1_decode needs for these arguments (0 if invalid). */
size_t diffattn_v1_decode_workspace_size(const diffattn_v1_decode_args *args);

/* DIFF V2 prefill forward. Returns DIFFATTN_OK or a negative status. */
int diffattn_v2_fwd(const diffattn_v2_fwd_args *args, void *stream);

/* Workspace bytes diffattn_v2_fwd and diffattn_v2_fwd_sparse need (0 if invalid). */
size_t diffattn_v2_fwd_workspace_size(const diffattn_v2_fwd_args *args);

/*
 * Block-sparse DIFF V2 prefill forward: one key-block selection per even/odd
 * head pair [V2 page, practical considerations: DIFF V2 works with sparse
 * attention frameworks by selecting blocks per head pair inside a GQA group;
 * the glossary's sparse-attention entry: a fixed subset of token pairs is
 * scored and every other weight is zero].  args as for diffattn_v2_fwd
 * without training saves.  block_cnt: device int32 [B, Hq/2, ceil(S / 128)];
 * block_idx: device int32 [B, Hq/2, ceil(S / 128), max_blocks].  For query
 * tile t (rows 128 t .. 128 t + 127) of pair p, the first block_cnt entries
 * of its block_idx row list the 64-key tiles (keys 64 i .. 64 i + 63) the
 * pair attends, ascending; entries out of range, past the query tile (causal)
 * or not above the previous accepted entry are ignored.  Each head's softmax
 * runs over the listed keys (causal mask applied inside them); a row that
 * sees no key is zero.  1 <= max_blocks <= 1024.
 */
int diffattn_v2_fwd_sparse(const diffattn_v2_fwd_args *args, const int32_t *block_idx, const int32_t *block_cnt,
                           int32_t max_blocks, void *stream);

/* DIFF V2 prefill backward. Returns DIFFATTN_OK or a negative status. */
int diffattn_v2_bwd(const diffattn_v2_bwd_args *args, void *stream);

/* Workspace bytes diffattn_v2_bwd needs for these arguments (0 if invalid). */
size_t diffattn_v2_bwd_workspace_size(const diffattn_v2_bwd_args *args);

/* lambda_init for layer index l >= 1: 0.8 - 0.6 exp(-0.3 (l - 1)); NaN for l < 1. */
float diffattn_lambda_init(int layer);

/* Static name of a status code. */
const char *diffattn_status_str(int status);

/* Message describing the last failure on the calling thread ("" if none). */
const char *diffattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
