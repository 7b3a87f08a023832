// C-ABI entry points: argument validation, workspace layout, launch.
// The maths lives in adaflash_kernels.hip; see include/adaflash.h for the
// contract of every entry point.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/adaflash.h"
#include "adaflash_internal.h"

namespace adaflash {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, const char* detail = "") {
  std::snprintf(g_err, sizeof(g_err), fmt, detail);
  return code;
}

bool sizes_ok(int B, int k, int V) {
  if (B < 0 || k < 1 || k > kMaxK || V < 1 || V > kMaxV) return false;
  if ((long long)B * (k + 1) >= (1LL << 24)) return false;
  return true;
}

}  // namespace

}  // namespace adaflash

using namespace adaflash;

extern "C" {

int adaflash_version(void) { return 100; }

int adaflash_timing_enable(int max_records) {
  if (max_records < 0 || max_records > (1 << 20)) return fail(ADAFLASH_E_INVALID, "max_records out of range%s");
  if (timing_enable(max_records) != 0) return fail(ADAFLASH_E_HIP, "hipEventCreate failed%s");
  return ADAFLASH_OK;
}

int adaflash_timing_every(int n) {
  if (timing_every(n) != 0) return fail(ADAFLASH_E_INVALID, "n must be at least 1%s");
  return ADAFLASH_OK;
}

int adaflash_timing_read(float* ms, int cap) {
  if (cap < 0 || (cap > 0 && !ms)) return fail(ADAFLASH_E_INVALID, "bad output buffer%s");
  const int n = timing_read(ms, cap);
  if (n < 0) return fail(ADAFLASH_E_HIP, "event query failed%s");
  return n;
}

const char* adaflash_last_error(void) { return g_err; }

size_t adaflash_workspace_bytes(int B, int k, int V) {
  if (!sizes_ok(B, k, V)) return 0;
  return workspace_layout(B, k, V, nullptr, nullptr);
}

static int common_checks(adaflash_dtype dtype, const void* target, const void* draft, int B, int k,
                         int V, int32_t* row_offsets, void* workspace, size_t workspace_bytes,
                         bool need_draft) {
  if (dtype != ADAFLASH_F32 && dtype != ADAFLASH_BF16) return fail(ADAFLASH_E_INVALID, "invalid dtype%s");
  if (!sizes_ok(B, k, V))
    return fail(ADAFLASH_E_INVALID,
                "invalid sizes%s: need B >= 0, 1 <= k <= 64, 1 <= V <= 2^20, B*(k+1) < 2^24");
  if (!row_offsets) return fail(ADAFLASH_E_INVALID, "row_offsets must not be NULL%s");
  if (B > 0 && !target) return fail(ADAFLASH_E_INVALID, "target_logits must not be NULL%s");
  if (B > 0 && need_draft && !draft) return fail(ADAFLASH_E_INVALID, "draft_logits must not be NULL%s");
  const size_t need = workspace_layout(B, k, V, nullptr, nullptr);
  if (!workspace || workspace_bytes < need)
    return fail(ADAFLASH_E_WORKSPACE, "workspace missing or smaller than adaflash_workspace_bytes()%s");
  return ADAFLASH_OK;
}

static int run(LaunchArgs& a, void* workspace) {
  workspace_layout(a.B, a.k, a.V, (char*)workspace, &a.ws);
  const hipError_t e = launch(a);
  if (e != hipSuccess) return fail(ADAFLASH_E_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return ADAFLASH_OK;
}

}  // extern "C"

namespace adaflash {
int fail_with(int code, const char* msg) { return fail(code, "%s", msg); }

int verify_impl(int packed, int dtype_code, const void* target_logits, const void* draft_logits,
                const int32_t* draft_tokens, const int32_t* verify_len, const float* uniforms,
                int B, int k, int V, float T, int32_t* accept_len, int32_t* out_tokens,
                float* margins, float clip_c, float lambda, int32_t* row_offsets,
                float* loss_ce, float* loss_rkl, void* grad_draft, int32_t* status_flags,
                void* workspace, size_t workspace_bytes, void* stream) {
  const adaflash_dtype dtype = (adaflash_dtype)dtype_code;
  const bool opd = loss_ce || loss_rkl || grad_draft;
  if (!(T >= 0.f) || std::isinf(T)) return fail(ADAFLASH_E_INVALID, "T must be finite and >= 0%s");
  const bool need_draft = T > 0.f || opd;
  int rc = common_checks(dtype, target_logits, draft_logits, B, k, V, row_offsets, workspace,
                         workspace_bytes, need_draft);
  if (rc != ADAFLASH_OK) return rc;
  if (B > 0 && (!draft_tokens || !verify_len || !accept_len || !out_tokens))
    return fail(ADAFLASH_E_INVALID, "draft_tokens, verify_len, accept_len and out_tokens must not be NULL%s");
  if (B > 0 && T > 0.f && !uniforms) return fail(ADAFLASH_E_INVALID, "uniforms must not be NULL when T > 0%s");
  if (opd && !(clip_c > 0.f)) return fail(ADAFLASH_E_INVALID, "clip_c must be > 0%s");
  if (opd && !(lambda >= 0.f) ) return fail(ADAFLASH_E_INVALID, "lambda must be >= 0%s");
  if (opd && (std::isinf(lambda))) return fail(ADAFLASH_E_INVALID, "lambda must be finite%s");

  LaunchArgs a{};
  a.bf16 = dtype == ADAFLASH_BF16;
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = draft_tokens;
  a.verify_len = verify_len;
  a.uniforms = uniforms;
  a.B = B;
  a.k = k;
  a.V = V;
  a.T = T;
  a.verify = 1;
  a.packed = packed;
  a.opd = opd ? 1 : 0;
  a.clip_c = clip_c;
  a.lambda = lambda;
  a.accept_len = accept_len;
  a.out_tokens = out_tokens;
  a.margins = margins;
  a.row_offsets = row_offsets;
  a.loss_ce = loss_ce;
  a.loss_rkl = loss_rkl;
  a.grad = grad_draft;
  a.status = status_flags;
  a.stream = (hipStream_t)stream;
  return run(a, workspace);
}

}  // namespace adaflash

extern "C" {

static int opd_impl(int packed, adaflash_dtype dtype, const void* target_logits,
                    const void* draft_logits, const int32_t* verify_len, int B, int k,
                    int V, float clip_c, float lambda, int32_t* row_offsets,
                    float* loss_ce, float* loss_rkl, void* grad_draft,
                    int32_t* status_flags, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int rc = common_checks(dtype, target_logits, draft_logits, B, k, V, row_offsets, workspace,
                         workspace_bytes, true);
  if (rc != ADAFLASH_OK) return rc;
  if (!(clip_c > 0.f)) return fail(ADAFLASH_E_INVALID, "clip_c must be > 0%s");
  if (!(lambda >= 0.f) || std::isinf(lambda)) return fail(ADAFLASH_E_INVALID, "lambda must be finite and >= 0%s");

  LaunchArgs a{};
  a.bf16 = dtype == ADAFLASH_BF16;
  a.target = target_logits;
  a.draft = draft_logits;
  a.verify_len = verify_len;
  a.B = B;
  a.k = k;
  a.V = V;
  a.T = 1.f;
  a.verify = 0;
  a.packed = packed;
  a.opd = 1;
  a.clip_c = clip_c;
  a.lambda = lambda;
  a.row_offsets = row_offsets;
  a.loss_ce = loss_ce;
  a.loss_rkl = loss_rkl;
  a.grad = grad_draft;
  a.status = status_flags;
  a.stream = (hipStream_t)stream;
  return run(a, workspace);
}

int adaflash_verify(adaflash_dtype dtype, const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const int32_t* verify_len, const float* uniforms,
                    int B, int k, int V, float T, int32_t* accept_len, int32_t* out_tokens,
                    float* margins, float clip_c, float lambda, int32_t* row_offsets,
                    float* loss_ce, float* loss_rkl, void* grad_draft, int32_t* status_flags,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return verify_impl(0, dtype, target_logits, draft_logits, draft_tokens, verify_len, uniforms, B, k, V, T,
                     accept_len, out_tokens, margins, clip_c, lambda, row_offsets, loss_ce, loss_rkl, grad_draft,
                     status_flags, workspace, workspace_bytes, stream);
}

int adaflash_verify_packed(adaflash_dtype dtype, const void* target_logits, const void* draft_logits,
                           const int32_t* draft_tokens, const int32_t* verify_len, const float* uniforms,
                           int B, int k, int V, float T, int32_t* accept_len, int32_t* out_tokens,
                           float* margins, float clip_c, float lambda, int32_t* row_offsets,
                           float* loss_ce, float* loss_rkl, void* grad_draft, int32_t* status_flags,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return verify_impl(1, dtype, target_logits, draft_logits, draft_tokens, verify_len, uniforms, B, k, V, T,
                     accept_len, out_tokens, margins, clip_c, lambda, row_offsets, loss_ce, loss_rkl, grad_draft,
                     status_flags, workspace, workspace_bytes, stream);
}

int adaflash_opd_loss_fwd_bwd(adaflash_dtype dtype, const void* target_logits,
                              const void* draft_logits, const int32_t* verify_len, int B, int k,
                              int V, float clip_c, float lambda, int32_t* row_offsets,
                              float* loss_ce, float* loss_rkl, void* grad_draft,
                              int32_t* status_flags, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return opd_impl(0, dtype, target_logits, draft_logits, verify_len, B, k, V, clip_c, lambda, row_offsets,
                  loss_ce, loss_rkl, grad_draft, status_flags, workspace, workspace_bytes, stream);
}

int adaflash_opd_loss_fwd_bwd_packed(adaflash_dtype dtype, const void* target_logits,
                                     const void* draft_logits, const int32_t* verify_len, int B, int k,
                                     int V, float clip_c, float lambda, int32_t* row_offsets,
                                     float* loss_ce, float* loss_rkl, void* grad_draft,
                                     int32_t* status_flags, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return opd_impl(1, dtype, target_logits, draft_logits, verify_len, B, k, V, clip_c, lambda, row_offsets,
                  loss_ce, loss_rkl, grad_draft, status_flags, workspace, workspace_bytes, stream);
}

int adaflash_loss_variant_fwd_bwd(adaflash_dtype dtype, const void* target_logits, const void* draft_logits,
                                  const int32_t* verify_len, int B, int k, int V, int variant, float p1, float p2,
                                  int32_t* row_offsets, float* loss, void* grad_draft, int32_t* status_flags,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  int rc = common_checks(dtype, target_logits, draft_logits, B, k, V, row_offsets, workspace, workspace_bytes,
                         true);
  if (rc != ADAFLASH_OK) return rc;
  LaunchArgs a{};
  const float inf = std::numeric_limits<float>::infinity();
  switch (variant) {
    case ADAFLASH_LOSS_RKL:
      a.a_ce = 0.f, a.lambda = 1.f, a.clip_c = inf;
      break;
    case ADAFLASH_LOSS_RKL_CLIP:
      if (!(p1 > 0.f) || std::isinf(p1)) return fail(ADAFLASH_E_INVALID, "delta must be finite and > 0%s");
      a.a_ce = 0.f, a.lambda = 1.f, a.clip_c = p1;
      break;
    case ADAFLASH_LOSS_MIXTURE:
      if (!(p1 >= 0.f && p1 <= 1.f)) return fail(ADAFLASH_E_INVALID, "alpha must be in [0, 1]%s");
      if (!(p2 > 0.f) || std::isinf(p2)) return fail(ADAFLASH_E_INVALID, "delta must be finite and > 0%s");
      a.a_ce = p1, a.lambda = 1.f - p1, a.clip_c = p2;
      break;
    case ADAFLASH_LOSS_FKL:
      a.a_ce = 0.f, a.lambda = 0.f, a.clip_c = inf, a.fkl = 1;
      break;
    case ADAFLASH_LOSS_WCE:
      if (!(p1 > 0.f) || std::isinf(p1)) return fail(ADAFLASH_E_INVALID, "position decay must be finite and > 0%s");
      a.a_ce = 1.f, a.lambda = 0.f, a.clip_c = inf, a.wdecay = p1;
      break;
    default:
      return fail(ADAFLASH_E_INVALID, "unknown loss variant%s");
  }
  a.bf16 = dtype == ADAFLASH_BF16;
  a.target = target_logits;
  a.draft = draft_logits;
  a.verify_len = verify_len;
  a.B = B;
  a.k = k;
  a.V = V;
  a.T = 1.f;
  a.verify = 0;
  a.opd = 1;
  a.row_offsets = row_offsets;
  a.loss_var = loss;
  a.grad = grad_draft;
  a.status = status_flags;
  a.stream = (hipStream_t)stream;
  return run(a, workspace);
}

size_t adaflash_length_head_workspace_bytes(int B, int k, int H, int Hp) {
  if (B < 0 || k < 1 || k > 64 || H < 16 || H > 65536 || H % 16 != 0 || Hp < 1 || Hp > 8192) return 0;
  if ((long long)B * k >= (1LL << 24)) return 0;
  const size_t n = lh_workspace_layout(B, k, H, Hp, nullptr, nullptr);
  return n > 256 ? n : 256;  // (an empty batch still gets a valid, nonzero size)
}

static int lh_checks(const void* h, const void* W1, const float* b1, const float* w2, float b2, int B, int k,
                     int H, int Hp, void* workspace, size_t workspace_bytes) {
  if (B < 0 || k < 1 || k > 64 || H < 16 || H > 65536 || H % 16 != 0 || Hp < 1 || Hp > 8192 ||
      (long long)B * k >= (1LL << 24))
    return fail(ADAFLASH_E_INVALID,
                "invalid sizes%s: need B >= 0, 1 <= k <= 64, 16 <= H <= 65536 with H %% 16 == 0, "
                "1 <= H' <= 8192, B*k < 2^24");
  if (B > 0 && (!h || !W1 || !b1 || !w2))
    return fail(ADAFLASH_E_INVALID, "hidden, W1, b1 and w2 must not be NULL%s");
  if (((uintptr_t)h & 15) || ((uintptr_t)W1 & 15))
    return fail(ADAFLASH_E_INVALID, "hidden and W1 must be 16-byte aligned%s");
  if (!std::isfinite(b2)) return fail(ADAFLASH_E_INVALID, "b2 must be finite%s");
  const size_t need = lh_workspace_layout(B, k, H, Hp, nullptr, nullptr);
  if (B > 0 && (!workspace || workspace_bytes < need))
    return fail(ADAFLASH_E_WORKSPACE, "workspace missing or smaller than adaflash_length_head_workspace_bytes()%s");
  return ADAFLASH_OK;
}

static int lh_forward(const void* hidden, const void* W1, const float* b1, const float* w2, float b2, int B, int k,
                      int H, int Hp, float gamma, float* a_hat, int32_t* k_hat, float* z1_cache, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int rc = lh_checks(hidden, W1, b1, w2, b2, B, k, H, Hp, workspace, workspace_bytes);
  if (rc != ADAFLASH_OK) return rc;
  if (!(gamma > 0.f) || std::isinf(gamma)) return fail(ADAFLASH_E_INVALID, "gamma must be finite and > 0%s");
  if (B > 0 && !a_hat && !k_hat) return fail(ADAFLASH_E_INVALID, "a_hat and k_hat are both NULL%s");
  LhArgs a{};
  a.h = (const uint16_t*)hidden;
  a.W1 = (const uint16_t*)W1;
  a.b1 = b1;
  a.w2 = w2;
  a.b2 = b2;
  a.gamma = gamma;
  a.B = B;
  a.k = k;
  a.H = H;
  a.Hp = Hp;
  a.a_hat = a_hat;
  a.k_hat = k_hat;
  a.z1_out = z1_cache;
  a.stream = (hipStream_t)stream;
  lh_workspace_layout(B, k, H, Hp, (char*)workspace, &a.ws);
  const hipError_t e = lh_launch(a);
  if (e != hipSuccess) return fail(ADAFLASH_E_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return ADAFLASH_OK;
}

static int lh_backward(const void* hidden, const void* W1, const float* b1, const float* w2, float b2, int B,
                       int k, int H, int Hp, const int32_t* accept_len, const int32_t* verify_len, float* loss,
                       float* dW1, float* db1, float* dw2, float* db2, const float* z1_cache, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int rc = lh_checks(hidden, W1, b1, w2, b2, B, k, H, Hp, workspace, workspace_bytes);
  if (rc != ADAFLASH_OK) return rc;
  if (!dW1 || !db1 || !dw2 || !db2) return fail(ADAFLASH_E_INVALID, "dW1, db1, dw2 and db2 must not be NULL%s");
  if (B > 0 && (!accept_len || !verify_len || !loss))
    return fail(ADAFLASH_E_INVALID, "accept_len, verify_len and loss must not be NULL%s");
  LhArgs a{};
  a.h = (const uint16_t*)hidden;
  a.W1 = (const uint16_t*)W1;
  a.b1 = b1;
  a.w2 = w2;
  a.b2 = b2;
  a.gamma = 1.f;
  a.B = B;
  a.k = k;
  a.H = H;
  a.Hp = Hp;
  a.accept_len = accept_len;
  a.verify_len = verify_len;
  a.loss = loss;
  a.dW1 = dW1;
  a.db1 = db1;
  a.dw2 = dw2;
  a.db2 = db2;
  a.z1_in = z1_cache;
  a.stream = (hipStream_t)stream;
  lh_workspace_layout(B, k, H, Hp, (char*)workspace, &a.ws);
  const hipError_t e = lh_launch(a);
  if (e != hipSuccess) return fail(ADAFLASH_E_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return ADAFLASH_OK;
}

int adaflash_length_head_forward(const void* hidden, const void* W1, const float* b1, const float* w2, float b2,
                                 int B, int k, int H, int Hp, float gamma, float* a_hat, int32_t* k_hat,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return lh_forward(hidden, W1, b1, w2, b2, B, k, H, Hp, gamma, a_hat, k_hat, nullptr, workspace, workspace_bytes,
                    stream);
}

int adaflash_length_head_forward_cached(const void* hidden, const void* W1, const float* b1, const float* w2,
                                        float b2, int B, int k, int H, int Hp, float gamma, float* a_hat,
                                        int32_t* k_hat, float* z1_cache, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (B > 0 && !z1_cache) return fail(ADAFLASH_E_INVALID, "z1_cache must not be NULL%s");
  return lh_forward(hidden, W1, b1, w2, b2, B, k, H, Hp, gamma, a_hat, k_hat, z1_cache, workspace,
                    workspace_bytes, stream);
}

int adaflash_length_head_backward(const void* hidden, const void* W1, const float* b1, const float* w2, float b2,
                                  int B, int k, int H, int Hp, const int32_t* accept_len,
                                  const int32_t* verify_len, float* loss, float* dW1, float* db1, float* dw2,
                                  float* db2, void* workspace, size_t workspace_bytes, void* stream) {
  return lh_backward(hidden, W1, b1, w2, b2, B, k, H, Hp, accept_len, verify_len, loss, dW1, db1, dw2, db2, nullptr,
                     workspace, workspace_bytes, stream);
}

int adaflash_length_head_backward_cached(const void* hidden, const void* W1, const float* b1, const float* w2,
                                         float b2, int B, int k, int H, int Hp, const int32_t* accept_len,
                                         const int32_t* verify_len, float* loss, float* dW1, float* db1,
                                         float* dw2, float* db2, const float* z1_cache, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (B > 0 && !z1_cache) return fail(ADAFLASH_E_INVALID, "z1_cache must not be NULL%s");
  return lh_backward(hidden, W1, b1, w2, b2, B, k, H, Hp, accept_len, verify_len, loss, dW1, db1, dw2, db2,
                     z1_cache, workspace, workspace_bytes, stream);
}

}  // extern "C"
