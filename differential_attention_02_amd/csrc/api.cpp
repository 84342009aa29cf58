// C ABI of libdiffattn (declared in include/diffattn.h): argument validation,
// kernel selection and launch.  Validation runs entirely on the host before
// any HIP call, so a rejected call launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "diffattn.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return DIFFATTN_OK;
  return fail(DIFFATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool strides_ok(const int64_t *s, int n) {
  for (int i = 0; i < n; ++i)
    if (s[i] < 1) return false;
  return true;
}

bool strides_mult(const int64_t *s, int n, int64_t m) {
  for (int i = 0; i < n; ++i)
    if (s[i] % m) return false;
  return true;
}

bool generic_dims(int d, int dv) {
  return (d == 8 && dv == 16) || (d == 16 && dv == 32) || (d == 32 && dv == 64) ||
         (d == 64 && dv == 128) || (d == 128 && dv == 256);
}

// Checks common to forward and backward.  Returns DIFFATTN_OK or an error.
int check_common(int B, int S, int H, int d, int dv, int dtype, const void *q1, const void *k1,
                 const void *q2, const void *k2, const void *v, const int64_t *qs,
                 const int64_t *ks, const int64_t *vs, const float *lq1, const float *lk1,
                 const float *lq2, const float *lk2, int lambda_dim, float lambda_fixed,
                 float lambda_init, float scale) {
  if (B < 0 || S < 0 || H < 1) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0, seqlen >= 0, heads >= 1");
  if (d < 1 || dv < 1) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "head_dim and v_dim must be positive");
  if (dtype != DIFFATTN_F32 && dtype != DIFFATTN_BF16) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (!q1 || !k1 || !q2 || !k2 || !v) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "q1, k1, q2, k2 and v must be non-NULL");
  if (!strides_ok(qs, 3) || !strides_ok(ks, 3) || !strides_ok(vs, 3))
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "strides must be positive");
  const int nvec = (lq1 != nullptr) + (lk1 != nullptr) + (lq2 != nullptr) + (lk2 != nullptr);
  if (nvec != 0 && nvec != 4) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "give all four lambda vectors or none");
  if (nvec == 4 && lambda_dim < 1) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "lambda_dim must be >= 1");
  if (nvec == 0 && !std::isfinite(lambda_fixed)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "lambda_fixed must be finite");
  if (!std::isfinite(lambda_init)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "lambda_init must be finite");
  if (!std::isfinite(scale)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  return DIFFATTN_OK;
}

bool fused_layout_ok(const void *const *ptrs, int np, const int64_t *const *strides, int ns) {
  for (int i = 0; i < np; ++i)
    if (ptrs[i] && !aligned16(ptrs[i])) return false;
  for (int i = 0; i < ns; ++i)
    if (!strides_mult(strides[i], 3, 8)) return false;
  return true;
}

}  // namespace

extern "C" {

const char *diffattn_status_str(int status) {
  switch (status) {
    case DIFFATTN_OK: return "ok";
    case DIFFATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DIFFATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case DIFFATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case DIFFATTN_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char *diffattn_last_error(void) { return g_last_error.c_str(); }

float diffattn_lambda_init(int layer) {
  if (layer < 1) return NAN;
  return 0.8f - 0.6f * expf(-0.3f * (float)(layer - 1));
}

int diffattn_fwd(const diffattn_fwd_args *a, void *stream) {
  g_last_error.clear();
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0 || a->seqlen < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0, seqlen >= 0");
  if (a->batch == 0 || a->seqlen == 0) return DIFFATTN_OK;  // empty problem: nothing to read or write
  int rc = check_common(a->batch, a->seqlen, a->heads, a->head_dim, a->v_dim, a->dtype, a->q1, a->k1,
                        a->q2, a->k2, a->v, a->q_stride, a->k_stride, a->v_stride, a->lq1, a->lk1,
                        a->lq2, a->lk2, a->lambda_dim, a->lambda_fixed, a->lambda_init,
                        a->softmax_scale);
  if (rc) return rc;
  if (!a->out) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "out must be non-NULL");
  if (!strides_ok(a->o_stride, 3)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "out strides must be positive");
  if (!(a->eps >= 0.f) || !std::isfinite(a->eps)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  const int nsave = (a->lse1 != nullptr) + (a->lse2 != nullptr) + (a->rstd != nullptr) +
                    (a->o_pre != nullptr) + (a->a2 != nullptr);
  if (nsave != 0 && nsave != 5) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "give all five training saves or none");
  const bool fused = a->dtype == DIFFATTN_BF16 && a->head_dim == 64 && a->v_dim == 128;
  if (!fused && !generic_dims(a->head_dim, a->v_dim))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "(head_dim, v_dim) = (%d, %d) not instantiated", a->head_dim, a->v_dim);
  if (nsave && !fused) return fail(DIFFATTN_ERR_UNSUPPORTED, "training saves need bf16 with head_dim 64, v_dim 128");
  if (nsave && !(aligned16(a->o_pre) && aligned16(a->a2)))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "training saves o_pre and a2 must be 16-byte aligned");
  if (fused) {
    const void *ptrs[] = {a->q1, a->k1, a->q2, a->k2, a->v, a->out};
    const int64_t *str[] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride};
    if (!fused_layout_ok(ptrs, 6, str, 4))
      return fail(DIFFATTN_ERR_UNSUPPORTED, "bf16 fused path needs 16-byte aligned pointers and strides that are multiples of 8");
    // Key tiles are addressed with 32-bit byte offsets inside one (batch, head) slice.
    const int64_t span = (int64_t)a->seqlen * (a->k_stride[1] > a->v_stride[1] ? a->k_stride[1] : a->v_stride[1]) * 2;
    if (span >= ((int64_t)1 << 31))
      return fail(DIFFATTN_ERR_UNSUPPORTED, "bf16 fused path needs seqlen x key-row stride below 2^30 elements");
    const size_t need = diffattn::fwd_workspace_bytes(a->batch, a->seqlen, a->heads);
    if (!a->workspace || a->workspace_bytes < need)
      return fail(DIFFATTN_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", need, a->workspace_bytes);
    if (!aligned16(a->workspace)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  }

  diffattn::FwdParams p{};
  p.q1 = a->q1; p.k1 = a->k1; p.q2 = a->q2; p.k2 = a->k2; p.v = a->v;
  p.qs_b = a->q_stride[0]; p.qs_s = a->q_stride[1]; p.qs_h = a->q_stride[2];
  p.ks_b = a->k_stride[0]; p.ks_s = a->k_stride[1]; p.ks_h = a->k_stride[2];
  p.vs_b = a->v_stride[0]; p.vs_s = a->v_stride[1]; p.vs_h = a->v_stride[2];
  p.os_b = a->o_stride[0]; p.os_s = a->o_stride[1]; p.os_h = a->o_stride[2];
  p.out = a->out;
  p.B = a->batch; p.S = a->seqlen; p.H = a->heads;
  p.causal = a->causal != 0; p.norm = a->norm != 0;
  p.lq1 = a->lq1; p.lk1 = a->lk1; p.lq2 = a->lq2; p.lk2 = a->lk2;
  p.lambda_dim = a->lambda_dim; p.lambda_fixed = a->lambda_fixed; p.lambda_init = a->lambda_init;
  p.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.f / std::sqrt((float)a->head_dim);
  p.eps = a->eps;
  p.lambda_out = a->lambda_out;
  p.lse1 = a->lse1; p.lse2 = a->lse2; p.rstd = a->rstd; p.o_pre = a->o_pre; p.a2 = a->a2;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fused) return hip_status(diffattn::launch_fwd(p, a->workspace, st), "fused forward launch");
  return hip_status(diffattn::launch_fwd_generic(p, a->dtype, a->head_dim, a->v_dim, st), "forward launch");
}

size_t diffattn_fwd_workspace_size(const diffattn_fwd_args *a) {
  if (!a || a->batch <= 0 || a->seqlen <= 0 || a->heads < 1) return 0;
  const bool fused = a->dtype == DIFFATTN_BF16 && a->head_dim == 64 && a->v_dim == 128;
  return fused ? diffattn::fwd_workspace_bytes(a->batch, a->seqlen, a->heads) : 0;
}

static int check_fwd_fp8(const diffattn_fwd_args *a) {
  int rc = check_common(a->batch, a->seqlen, a->heads, a->head_dim, a->v_dim, a->dtype, a->q1, a->k1,
                        a->q2, a->k2, a->v, a->q_stride, a->k_stride, a->v_stride, a->lq1, a->lk1,
                        a->lq2, a->lk2, a->lambda_dim, a->lambda_fixed, a->lambda_init, a->softmax_scale);
  if (rc) return rc;
  if (!a->out) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "out must be non-NULL");
  if (!strides_ok(a->o_stride, 3)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "out strides must be positive");
  if (!(a->eps >= 0.f) || !std::isfinite(a->eps)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (a->lse1 || a->lse2 || a->rstd || a->o_pre || a->a2)
    return fail(DIFFATTN_ERR_UNSUPPORTED, "the fp8-logit forward has no training saves");
  if (a->dtype != DIFFATTN_BF16 || a->head_dim != 64 || a->v_dim != 128)
    return fail(DIFFATTN_ERR_UNSUPPORTED, "the fp8-logit forward is built for bf16 with head_dim 64, v_dim 128");
  const void *ptrs[] = {a->q1, a->k1, a->q2, a->k2, a->v, a->out};
  const int64_t *str[] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride};
  if (!fused_layout_ok(ptrs, 6, str, 4))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "fp8-logit forward needs 16-byte aligned pointers and strides that are multiples of 8");
  const int64_t vspan = (int64_t)a->seqlen * a->v_stride[1] * 2;
  const int64_t cspan = (int64_t)a->batch * a->heads * a->seqlen * 64;
  if (vspan >= ((int64_t)1 << 31) || cspan >= ((int64_t)1 << 31))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "fp8-logit forward needs V and code slices below 2^31 bytes");
  return DIFFATTN_OK;
}

size_t diffattn_fwd_fp8_workspace_size(const diffattn_fwd_args *a) {
  std::string keep = g_last_error;
  const int rc = (!a || a->batch <= 0 || a->seqlen <= 0) ? DIFFATTN_ERR_INVALID_ARGUMENT : check_fwd_fp8(a);
  g_last_error = keep;
  if (rc) return 0;
  return diffattn::fwd_fp8_workspace_bytes(a->batch, a->seqlen, a->heads);
}

int diffattn_fwd_fp8(const diffattn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream) {
  g_last_error.clear();
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0 || a->seqlen < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0, seqlen >= 0");
  if (a->batch == 0 || a->seqlen == 0) return DIFFATTN_OK;
  int rc = check_fwd_fp8(a);
  if (rc) return rc;
  const size_t need = diffattn::fwd_fp8_workspace_bytes(a->batch, a->seqlen, a->heads);
  if (!workspace || workspace_bytes < need)
    return fail(DIFFATTN_ERR_WORKSPACE, "fp8-logit forward needs %zu workspace bytes, got %zu", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  diffattn::FwdParams p{};
  p.q1 = a->q1; p.k1 = a->k1; p.q2 = a->q2; p.k2 = a->k2; p.v = a->v;
  p.qs_b = a->q_stride[0]; p.qs_s = a->q_stride[1]; p.qs_h = a->q_stride[2];
  p.ks_b = a->k_stride[0]; p.ks_s = a->k_stride[1]; p.ks_h = a->k_stride[2];
  p.vs_b = a->v_stride[0]; p.vs_s = a->v_stride[1]; p.vs_h = a->v_stride[2];
  p.os_b = a->o_stride[0]; p.os_s = a->o_stride[1]; p.os_h = a->o_stride[2];
  p.out = a->out;
  p.B = a->batch; p.S = a->seqlen; p.H = a->heads;
  p.causal = a->causal != 0; p.norm = a->norm != 0;
  p.lq1 = a->lq1; p.lk1 = a->lk1; p.lq2 = a->lq2; p.lk2 = a->lk2;
  p.lambda_dim = a->lambda_dim; p.lambda_fixed = a->lambda_fixed; p.lambda_init = a->lambda_init;
  p.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.f / std::sqrt((float)a->head_dim);
  p.eps = a->eps;
  p.lambda_out = a->lambda_out;
  return hip_status(diffattn::launch_fwd_fp8(p, workspace, static_cast<hipStream_t>(stream)), "fp8-logit forward launch");
}

static int check_bwd(const diffattn_bwd_args *a) {
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  int rc = check_common(a->batch, a->seqlen, a->heads, a->head_dim, a->v_dim, a->dtype, a->q1, a->k1,
                        a->q2, a->k2, a->v, a->q_stride, a->k_stride, a->v_stride, a->lq1, a->lk1,
                        a->lq2, a->lk2, a->lambda_dim, a->lambda_fixed, a->lambda_init,
                        a->softmax_scale);
  if (rc) return rc;
  if (!a->dout) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "dout must be non-NULL");
  if (!a->lse1 || !a->lse2 || !a->rstd || !a->o_pre || !a->a2)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "backward needs the five forward saves");
  if (!(aligned16(a->o_pre) && aligned16(a->a2)))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "forward saves o_pre and a2 must be 16-byte aligned");
  if (!a->dq1 || !a->dk1 || !a->dq2 || !a->dk2 || !a->dv)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "dq1, dk1, dq2, dk2 and dv must be non-NULL");
  if (!strides_ok(a->do_stride, 3) || !strides_ok(a->dq_stride, 3) || !strides_ok(a->dk_stride, 3) ||
      !strides_ok(a->dv_stride, 3))
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "strides must be positive");
  const int ng = (a->dlq1 != nullptr) + (a->dlk1 != nullptr) + (a->dlq2 != nullptr) + (a->dlk2 != nullptr);
  if (a->lq1 && ng != 4) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "lambda vectors given: dlq1, dlk1, dlq2, dlk2 are required");
  if (!a->lq1 && ng != 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "lambda vector gradients need the lambda vectors");
  if (!(a->dtype == DIFFATTN_BF16 && a->head_dim == 64 && a->v_dim == 128))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "backward is built for bf16 with head_dim 64, v_dim 128");
  const void *ptrs[] = {a->q1, a->k1, a->q2, a->k2, a->v, a->dout, a->dq1, a->dk1, a->dq2, a->dk2, a->dv};
  const int64_t *str[] = {a->q_stride, a->k_stride, a->v_stride, a->do_stride, a->dq_stride, a->dk_stride, a->dv_stride};
  if (!fused_layout_ok(ptrs, 11, str, 7))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "backward needs 16-byte aligned pointers and strides that are multiples of 8");
  // Key tiles are addressed with 32-bit byte offsets inside one (batch, head) slice.
  const int64_t span = (int64_t)a->seqlen * (a->k_stride[1] > a->v_stride[1] ? a->k_stride[1] : a->v_stride[1]) * 2;
  if (span >= ((int64_t)1 << 31))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "backward needs seqlen x key-row stride below 2^30 elements");
  return DIFFATTN_OK;
}

size_t diffattn_bwd_workspace_size(const diffattn_bwd_args *a) {
  std::string keep = g_last_error;
  const int rc = check_bwd(a);
  g_last_error = keep;
  if (rc) return 0;
  return diffattn::bwd_workspace_bytes(a->batch, a->seqlen, a->heads, a->head_dim, a->v_dim);
}

int diffattn_bwd(const diffattn_bwd_args *a, void *stream) {
  g_last_error.clear();
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0 || a->seqlen < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0, seqlen >= 0");
  if (a->batch == 0 || a->seqlen == 0) return DIFFATTN_OK;
  int rc = check_bwd(a);
  if (rc) return rc;
  const size_t need = diffattn::bwd_workspace_bytes(a->batch, a->seqlen, a->heads, a->head_dim, a->v_dim);
  if (need && (!a->workspace || a->workspace_bytes < need))
    return fail(DIFFATTN_ERR_WORKSPACE, "backward needs %zu workspace bytes, got %zu", need, a->workspace_bytes);
  if (a->workspace && (reinterpret_cast<uintptr_t>(a->workspace) & 255u))
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");

  diffattn::BwdParams p{};
  p.q1 = a->q1; p.k1 = a->k1; p.q2 = a->q2; p.k2 = a->k2; p.v = a->v; p.dout = a->dout;
  p.qs_b = a->q_stride[0]; p.qs_s = a->q_stride[1]; p.qs_h = a->q_stride[2];
  p.ks_b = a->k_stride[0]; p.ks_s = a->k_stride[1]; p.ks_h = a->k_stride[2];
  p.vs_b = a->v_stride[0]; p.vs_s = a->v_stride[1]; p.vs_h = a->v_stride[2];
  p.ds_b = a->do_stride[0]; p.ds_s = a->do_stride[1]; p.ds_h = a->do_stride[2];
  p.B = a->batch; p.S = a->seqlen; p.H = a->heads;
  p.causal = a->causal != 0; p.norm = a->norm != 0;
  p.lq1 = a->lq1; p.lk1 = a->lk1; p.lq2 = a->lq2; p.lk2 = a->lk2;
  p.lambda_dim = a->lambda_dim; p.lambda_fixed = a->lambda_fixed; p.lambda_init = a->lambda_init;
  p.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.f / std::sqrt((float)a->head_dim);
  p.lse1 = a->lse1; p.lse2 = a->lse2; p.rstd = a->rstd; p.o_pre = a->o_pre; p.a2 = a->a2;
  p.dq1 = a->dq1; p.dk1 = a->dk1; p.dq2 = a->dq2; p.dk2 = a->dk2; p.dv = a->dv;
  p.dqs_b = a->dq_stride[0]; p.dqs_s = a->dq_stride[1]; p.dqs_h = a->dq_stride[2];
  p.dks_b = a->dk_stride[0]; p.dks_s = a->dk_stride[1]; p.dks_h = a->dk_stride[2];
  p.dvs_b = a->dv_stride[0]; p.dvs_s = a->dv_stride[1]; p.dvs_h = a->dv_stride[2];
  p.dlq1 = a->dlq1; p.dlk1 = a->dlk1; p.dlq2 = a->dlq2; p.dlk2 = a->dlk2; p.dlambda = a->dlambda;
  p.workspace = a->workspace;
  return hip_status(diffattn::launch_bwd(p, static_cast<hipStream_t>(stream)), "backward launch");
}

// Checks shared by the V2 prefill forward and backward (shapes, pointers of
// the forward inputs, strides, layout and offset range).
static int check_v2_common(int B, int S, int Hq, int Hkv, int D, int dtype, const void *q, const void *k,
                           const void *v, const float *lam, const int64_t *qs, const int64_t *kvs,
                           const int64_t *ls, float scale) {
  if (B < 0 || S < 0 || Hq < 2 || Hkv < 1)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0, seqlen >= 0, q_heads >= 2, kv_heads >= 1");
  if (Hq % Hkv || (Hq / Hkv) % 2)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                "q_heads / kv_heads must be an even integer so each even/odd pair shares a KV head");
  if (dtype != DIFFATTN_F32 && dtype != DIFFATTN_BF16) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (!q || !k || !v || !lam) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "q, k, v and lam must be non-NULL");
  if (!strides_ok(qs, 3) || !strides_ok(kvs, 3)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "strides must be positive");
  if (ls[0] < 0 || ls[1] < 0 || ls[2] < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "lam strides must be >= 0");
  if (!std::isfinite(scale)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (dtype != DIFFATTN_BF16 || D != 128)
    return fail(DIFFATTN_ERR_UNSUPPORTED, "V2 prefill is built for bf16 with head_dim 128");
  // Key tiles are addressed with 32-bit byte offsets inside one (batch, KV head)
  // slice, including the two tiles a workgroup may prefetch past the end.
  if (((int64_t)S + 128) * kvs[1] * 2 >= ((int64_t)1 << 31))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "V2 prefill needs (seqlen + 128) x key-row stride below 2^30 elements");
  return DIFFATTN_OK;
}

static int check_v2_workspace(const diffattn_v2_fwd_args *a) {
  const size_t need = diffattn::vrange_bytes(a->batch, a->seqlen, a->kv_heads);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(DIFFATTN_ERR_WORKSPACE, "V2 prefill needs %zu workspace bytes, got %zu", need, a->workspace_bytes);
  if (!aligned16(a->workspace)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  return DIFFATTN_OK;
}

size_t diffattn_v2_fwd_workspace_size(const diffattn_v2_fwd_args *a) {
  if (!a || a->batch <= 0 || a->seqlen <= 0 || a->kv_heads < 1) return 0;
  return diffattn::vrange_bytes(a->batch, a->seqlen, a->kv_heads);
}

int diffattn_v2_fwd(const diffattn_v2_fwd_args *a, void *stream) {
  g_last_error.clear();
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch == 0 || a->seqlen == 0) {
    if (a->batch < 0 || a->seqlen < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0, seqlen >= 0");
    return DIFFATTN_OK;
  }
  int rc = check_v2_common(a->batch, a->seqlen, a->q_heads, a->kv_heads, a->head_dim, a->dtype, a->q, a->k, a->v,
                           a->lam, a->q_stride, a->kv_stride, a->lam_stride, a->softmax_scale);
  if (rc) return rc;
  if (!a->out) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "out must be non-NULL");
  if (!strides_ok(a->o_stride, 3)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "strides must be positive");
  const int nsave = (a->lse != nullptr) + (a->a_even != nullptr) + (a->a_odd != nullptr);
  if (nsave != 0 && nsave != 3) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "give all three training saves or none");
  {
    const void *ptrs[] = {a->q, a->k, a->v, a->out, a->a_even, a->a_odd};
    const int64_t *str[] = {a->q_stride, a->kv_stride, a->o_stride};
    if (!fused_layout_ok(ptrs, 6, str, 3))
      return fail(DIFFATTN_ERR_UNSUPPORTED, "V2 prefill needs 16-byte aligned pointers and strides that are multiples of 8");
  }
  if ((rc = check_v2_workspace(a))) return rc;
  diffattn::V2FwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v;
  p.qs_b = a->q_stride[0]; p.qs_s = a->q_stride[1]; p.qs_h = a->q_stride[2];
  p.kvs_b = a->kv_stride[0]; p.kvs_s = a->kv_stride[1]; p.kvs_h = a->kv_stride[2];
  p.os_b = a->o_stride[0]; p.os_s = a->o_stride[1]; p.os_h = a->o_stride[2];
  p.lam = a->lam; p.ls_b = a->lam_stride[0]; p.ls_s = a->lam_stride[1]; p.ls_p = a->lam_stride[2];
  p.out = a->out;
  p.B = a->batch; p.S = a->seqlen; p.Hq = a->q_heads; p.Hkv = a->kv_heads;
  p.causal = a->causal != 0;
  p.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.f / std::sqrt((float)a->head_dim);
  p.lse = a->lse; p.a_even = a->a_even; p.a_odd = a->a_odd;
  p.vpart = static_cast<const unsigned *>(a->workspace);
  return hip_status(diffattn::launch_fwd_v2(p, static_cast<hipStream_t>(stream)), "V2 prefill launch");
}

int diffattn_v2_fwd_sparse(const diffattn_v2_fwd_args *a, const int32_t *block_idx, const int32_t *block_cnt,
                           int32_t max_blocks, void *stream) {
  g_last_error.clear();
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch == 0 || a->seqlen == 0) {
    if (a->batch < 0 || a->seqlen < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0, seqlen >= 0");
    return DIFFATTN_OK;
  }
  int rc = check_v2_common(a->batch, a->seqlen, a->q_heads, a->kv_heads, a->head_dim, a->dtype, a->q, a->k, a->v,
                           a->lam, a->q_stride, a->kv_stride, a->lam_stride, a->softmax_scale);
  if (rc) return rc;
  if (!a->out) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "out must be non-NULL");
  if (!strides_ok(a->o_stride, 3)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "strides must be positive");
  if (a->lse || a->a_even || a->a_odd)
    return fail(DIFFATTN_ERR_UNSUPPORTED, "the block-sparse forward has no training saves");
  if (!block_idx || !block_cnt) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "block_idx and block_cnt must be non-NULL");
  if (max_blocks < 1 || max_blocks > 1024) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "max_blocks must be in [1, 1024]");
  {
    const void *ptrs[] = {a->q, a->k, a->v, a->out};
    const int64_t *str[] = {a->q_stride, a->kv_stride, a->o_stride};
    if (!fused_layout_ok(ptrs, 4, str, 3))
      return fail(DIFFATTN_ERR_UNSUPPORTED, "V2 prefill needs 16-byte aligned pointers and strides that are multiples of 8");
  }
  if ((rc = check_v2_workspace(a))) return rc;
  diffattn::V2FwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v;
  p.qs_b = a->q_stride[0]; p.qs_s = a->q_stride[1]; p.qs_h = a->q_stride[2];
  p.kvs_b = a->kv_stride[0]; p.kvs_s = a->kv_stride[1]; p.kvs_h = a->kv_stride[2];
  p.os_b = a->o_stride[0]; p.os_s = a->o_stride[1]; p.os_h = a->o_stride[2];
  p.lam = a->lam; p.ls_b = a->lam_stride[0]; p.ls_s = a->lam_stride[1]; p.ls_p = a->lam_stride[2];
  p.out = a->out;
  p.B = a->batch; p.S = a->seqlen; p.Hq = a->q_heads; p.Hkv = a->kv_heads;
  p.causal = a->causal != 0;
  p.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.f / std::sqrt((float)a->head_dim);
  p.blk_idx = block_idx; p.blk_cnt = block_cnt; p.max_blocks = max_blocks;
  p.vpart = static_cast<const unsigned *>(a->workspace);
  return hip_status(diffattn::launch_fwd_v2(p, static_cast<hipStream_t>(stream)), "block-sparse V2 prefill launch");
}

static int check_v2_bwd(const diffattn_v2_bwd_args *a) {
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  int rc = check_v2_common(a->batch, a->seqlen, a->q_heads, a->kv_heads, a->head_dim, a->dtype, a->q, a->k, a->v,
                           a->lam, a->q_stride, a->kv_stride, a->lam_stride, a->softmax_scale);
  if (rc) return rc;
  if (!a->dout) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "dout must be non-NULL");
  if (!a->lse || !a->a_even || !a->a_odd)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "backward needs the forward's three training saves");
  if (!a->dq || !a->dk || !a->dv || !a->dlam)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "dq, dk, dv and dlam must be non-NULL");
  if (!strides_ok(a->do_stride, 3) || !strides_ok(a->dq_stride, 3) || !strides_ok(a->dkv_stride, 3))
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "strides must be positive");
  const void *ptrs[] = {a->q, a->k, a->v, a->dout, a->dq, a->dk, a->dv, a->a_even, a->a_odd};
  const int64_t *str[] = {a->q_stride, a->kv_stride, a->do_stride, a->dq_stride, a->dkv_stride};
  if (!fused_layout_ok(ptrs, 9, str, 5))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "V2 backward needs 16-byte aligned pointers and strides that are multiples of 8");
  return DIFFATTN_OK;
}

size_t diffattn_v2_bwd_workspace_size(const diffattn_v2_bwd_args *a) {
  std::string keep = g_last_error;
  const int rc = (a && (a->batch == 0 || a->seqlen == 0)) ? DIFFATTN_OK : check_v2_bwd(a);
  g_last_error = keep;
  if (rc || a->batch <= 0 || a->seqlen <= 0) return 0;
  return diffattn::v2_bwd_workspace_bytes(a->batch, a->seqlen, a->q_heads, a->kv_heads);
}

int diffattn_v2_bwd(const diffattn_v2_bwd_args *a, void *stream) {
  g_last_error.clear();
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0 || a->seqlen < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0, seqlen >= 0");
  if (a->batch == 0 || a->seqlen == 0) return DIFFATTN_OK;
  int rc = check_v2_bwd(a);
  if (rc) return rc;
  const size_t need = diffattn::v2_bwd_workspace_bytes(a->batch, a->seqlen, a->q_heads, a->kv_heads);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(DIFFATTN_ERR_WORKSPACE, "V2 backward needs %zu workspace bytes, got %zu", need, a->workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  diffattn::V2BwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.dout = a->dout;
  p.qs_b = a->q_stride[0]; p.qs_s = a->q_stride[1]; p.qs_h = a->q_stride[2];
  p.kvs_b = a->kv_stride[0]; p.kvs_s = a->kv_stride[1]; p.kvs_h = a->kv_stride[2];
  p.ds_b = a->do_stride[0]; p.ds_s = a->do_stride[1]; p.ds_h = a->do_stride[2];
  p.lam = a->lam; p.ls_b = a->lam_stride[0]; p.ls_s = a->lam_stride[1]; p.ls_p = a->lam_stride[2];
  p.lse = a->lse; p.a_even = a->a_even; p.a_odd = a->a_odd;
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  p.dqs_b = a->dq_stride[0]; p.dqs_s = a->dq_stride[1]; p.dqs_h = a->dq_stride[2];
  p.dkvs_b = a->dkv_stride[0]; p.dkvs_s = a->dkv_stride[1]; p.dkvs_h = a->dkv_stride[2];
  p.dlam = a->dlam;
  p.B = a->batch; p.S = a->seqlen; p.Hq = a->q_heads; p.Hkv = a->kv_heads;
  p.causal = a->causal != 0;
  p.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.f / std::sqrt((float)a->head_dim);
  p.workspace = a->workspace;
  return hip_status(diffattn::launch_v2_bwd(p, static_cast<hipStream_t>(stream)), "V2 backward launch");
}

static int check_v1_decode(const diffattn_v1_decode_args *a, int *splits_out) {
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0 || a->heads < 1 || a->kv_len < 0)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0, heads >= 1, kv_len >= 0");
  if (a->dtype != DIFFATTN_F32 && a->dtype != DIFFATTN_BF16) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", a->dtype);
  if (a->head_dim != 64 || a->v_dim != 128)
    return fail(DIFFATTN_ERR_UNSUPPORTED, "V1 decode is built for head_dim 64, v_dim 128");
  if (!a->q1 || !a->q2 || !a->k1_cache || !a->k2_cache || !a->v_cache || !a->out)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "q1, q2, k1_cache, k2_cache, v_cache and out must be non-NULL");
  if (a->q_stride[0] < 1 || a->q_stride[1] < 1 || a->o_stride[0] < 1 || a->o_stride[1] < 1 ||
      !strides_ok(a->k_stride, 3) || !strides_ok(a->v_stride, 3))
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "strides must be positive");
  const int nvec = (a->lq1 != nullptr) + (a->lk1 != nullptr) + (a->lq2 != nullptr) + (a->lk2 != nullptr);
  if (nvec != 0 && nvec != 4) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "give all four lambda vectors or none");
  if (nvec == 4 && a->lambda_dim < 1) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "lambda_dim must be >= 1");
  if (nvec == 0 && !std::isfinite(a->lambda_fixed)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "lambda_fixed must be finite");
  if (!std::isfinite(a->lambda_init)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "lambda_init must be finite");
  if (!std::isfinite(a->softmax_scale)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (!(a->eps >= 0.f) || !std::isfinite(a->eps)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  const int64_t vec = a->dtype == DIFFATTN_BF16 ? 8 : 4;
  if (!aligned16(a->k1_cache) || !aligned16(a->k2_cache) || !aligned16(a->v_cache) ||
      !strides_mult(a->k_stride, 3, vec) || !strides_mult(a->v_stride, 3, vec))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "caches need 16-byte aligned rows");
  if (a->num_splits < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "num_splits must be >= 0");
  int splits = a->num_splits ? a->num_splits : diffattn::decode_auto_splits(a->batch, a->heads, a->kv_len);
  if (splits < 1) splits = 1;
  const int chunk = (a->kv_len + splits - 1) / splits;
  if (chunk > diffattn::decode_max_chunk())
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "num_splits %d leaves %d keys per split (max %d)", splits, chunk,
                diffattn::decode_max_chunk());
  *splits_out = splits;
  return DIFFATTN_OK;
}

size_t diffattn_v1_decode_workspace_size(const diffattn_v1_decode_args *a) {
  std::string keep = g_last_error;
  int splits = 0;
  const int rc = check_v1_decode(a, &splits);
  g_last_error = keep;
  if (rc) return 0;
  return diffattn::v1_decode_workspace_bytes(a->batch, a->heads, splits);
}

int diffattn_v1_decode(const diffattn_v1_decode_args *a, void *stream) {
  g_last_error.clear();
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0");
  if (a->batch == 0) return DIFFATTN_OK;
  int splits = 0;
  int rc = check_v1_decode(a, &splits);
  if (rc) return rc;
  const size_t need = diffattn::v1_decode_workspace_bytes(a->batch, a->heads, splits);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(DIFFATTN_ERR_WORKSPACE, "V1 decode needs %zu workspace bytes, got %zu", need, a->workspace_bytes);
  if (!aligned16(a->workspace)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  diffattn::V1DecodeParams p{};
  p.q1 = a->q1; p.q2 = a->q2; p.k1 = a->k1_cache; p.k2 = a->k2_cache; p.v = a->v_cache;
  p.qs_b = a->q_stride[0]; p.qs_h = a->q_stride[1];
  p.ks_b = a->k_stride[0]; p.ks_s = a->k_stride[1]; p.ks_h = a->k_stride[2];
  p.vs_b = a->v_stride[0]; p.vs_s = a->v_stride[1]; p.vs_h = a->v_stride[2];
  p.os_b = a->o_stride[0]; p.os_h = a->o_stride[1];
  p.seqlens = a->seqlens;
  p.lq1 = a->lq1; p.lk1 = a->lk1; p.lq2 = a->lq2; p.lk2 = a->lk2;
  p.lambda_dim = a->lambda_dim; p.lambda_fixed = a->lambda_fixed; p.lambda_init = a->lambda_init;
  p.norm = a->norm != 0; p.eps = a->eps;
  p.out = a->out;
  p.B = a->batch; p.H = a->heads; p.L = a->kv_len;
  p.splits = splits;
  p.chunk = (a->kv_len + splits - 1) / splits;
  if (p.chunk < 1) p.chunk = 1;
  p.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.f / std::sqrt((float)a->head_dim);
  p.part_o = static_cast<float *>(a->workspace);
  p.part_ml = p.part_o + (size_t)a->batch * a->heads * 2 * splits * a->v_dim;
  return hip_status(diffattn::launch_v1_decode(p, a->dtype, static_cast<hipStream_t>(stream)), "V1 decode launch");
}

static int check_decode(const diffattn_v2_decode_args *a, int *splits_out) {
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0 || a->q_heads < 2 || a->kv_heads < 1 || a->kv_len < 0)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0, q_heads >= 2, kv_heads >= 1, kv_len >= 0");
  if (a->q_heads % a->kv_heads || (a->q_heads / a->kv_heads) % 2)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT,
                "q_heads / kv_heads must be an even integer so each even/odd pair shares a KV head");
  if (a->dtype != DIFFATTN_F32 && a->dtype != DIFFATTN_BF16) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "unknown dtype %d", a->dtype);
  if (a->head_dim != 64 && a->head_dim != 128) return fail(DIFFATTN_ERR_UNSUPPORTED, "decode head_dim must be 64 or 128");
  if (!a->q || !a->k_cache || !a->v_cache || !a->lam || !a->out)
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "q, k_cache, v_cache, lam and out must be non-NULL");
  if (a->q_stride[0] < 1 || a->q_stride[1] < 1 || a->o_stride[0] < 1 || a->o_stride[1] < 1 || !strides_ok(a->kv_stride, 3))
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "strides must be positive");
  if (a->lam_stride_b < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "lam_stride_b must be >= 0");
  const int64_t vec = a->dtype == DIFFATTN_BF16 ? 8 : 4;
  if (!aligned16(a->k_cache) || !aligned16(a->v_cache) || !strides_mult(a->kv_stride, 3, vec))
    return fail(DIFFATTN_ERR_UNSUPPORTED, "KV caches need 16-byte aligned rows");
  if (!std::isfinite(a->softmax_scale)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (a->num_splits < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "num_splits must be >= 0");
  int splits = a->num_splits ? a->num_splits : diffattn::decode_auto_splits(a->batch, a->kv_heads, a->kv_len);
  if (splits < 1) splits = 1;
  const int chunk = (a->kv_len + splits - 1) / splits;
  if (chunk > diffattn::decode_max_chunk())
    return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "num_splits %d leaves %d keys per split (max %d)", splits, chunk,
                diffattn::decode_max_chunk());
  *splits_out = splits;
  return DIFFATTN_OK;
}

size_t diffattn_v2_decode_workspace_size(const diffattn_v2_decode_args *a) {
  std::string keep = g_last_error;
  int splits = 0;
  const int rc = check_decode(a, &splits);
  g_last_error = keep;
  if (rc) return 0;
  return diffattn::decode_workspace_bytes(a->batch, a->q_heads, a->head_dim, splits);
}

static_assert(diffattn::kDecodeScratchBytes == DIFFATTN_DECODE_SCRATCH_BYTES, "scratch size and its header constant");

// Launches a validated decode with its partials in `ws` (need bytes).
static int run_decode(const diffattn_v2_decode_args *a, int splits, void *ws, void *stream) {
  diffattn::DecodeParams p{};
  p.q = a->q; p.k = a->k_cache; p.v = a->v_cache;
  p.qs_b = a->q_stride[0]; p.qs_h = a->q_stride[1];
  p.kvs_b = a->kv_stride[0]; p.kvs_s = a->kv_stride[1]; p.kvs_h = a->kv_stride[2];
  p.os_b = a->o_stride[0]; p.os_h = a->o_stride[1];
  p.seqlens = a->seqlens; p.lam = a->lam; p.lam_stride_b = a->lam_stride_b;
  p.out = a->out;
  p.B = a->batch; p.Hq = a->q_heads; p.Hkv = a->kv_heads; p.D = a->head_dim; p.L = a->kv_len;
  p.splits = splits;
  p.chunk = (a->kv_len + splits - 1) / splits;
  if (p.chunk < 1) p.chunk = 1;
  p.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.f / std::sqrt((float)a->head_dim);
  p.part_o = static_cast<float *>(ws);
  p.part_ml = p.part_o + (size_t)a->batch * a->q_heads * splits * a->head_dim;
  return hip_status(diffattn::launch_decode(p, a->dtype, static_cast<hipStream_t>(stream)), "decode launch");
}

int diffattn_v2_decode(const diffattn_v2_decode_args *a, void *stream) {
  g_last_error.clear();
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0");
  if (a->batch == 0) return DIFFATTN_OK;
  int splits = 0;
  int rc = check_decode(a, &splits);
  if (rc) return rc;
  const size_t need = diffattn::decode_workspace_bytes(a->batch, a->q_heads, a->head_dim, splits);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(DIFFATTN_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need, a->workspace_bytes);
  if (!aligned16(a->workspace)) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  return run_decode(a, splits, a->workspace, stream);
}

int diffattn_v2_decode_noalloc(const diffattn_v2_decode_args *a, void *stream) {
  g_last_error.clear();
  if (!a) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0) return fail(DIFFATTN_ERR_INVALID_ARGUMENT, "need batch >= 0");
  if (a->batch == 0) return DIFFATTN_OK;
  int splits = 0;
  int rc = check_decode(a, &splits);
  if (rc) return rc;
  const size_t need = diffattn::decode_workspace_bytes(a->batch, a->q_heads, a->head_dim, splits);
  if (need > diffattn::kDecodeScratchBytes)
    return fail(DIFFATTN_ERR_WORKSPACE,
                "decode needs %zu scratch bytes; the fixed scratch holds %zu (use diffattn_v2_decode with a "
                "workspace, or fewer splits)", need, diffattn::kDecodeScratchBytes);
  hipError_t e = hipSuccess;
  void *ws = diffattn::decode_scratch(&e);
  if (!ws) return fail(DIFFATTN_ERR_HIP, "decode scratch lookup failed: %s", hipGetErrorString(e));
  return run_decode(a, splits, ws, stream);
}

}  // extern "C"
