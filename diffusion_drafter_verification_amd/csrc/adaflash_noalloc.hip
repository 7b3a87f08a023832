// adaflash_verify_noalloc: adaflash_verify for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  Its workspace is a fixed device array of this library, one
// per GPU, instead of a caller buffer.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/adaflash.h"
#include "adaflash_internal.h"

namespace adaflash {
namespace {

// The workspace of the no-allocation entry point: each GPU the library runs
// on holds one copy until the process ends.  In host code `scratch` is only a
// stand-in for the symbol; its device address on the current device comes
// from hipGetSymbolAddress and is kept per device.
constexpr size_t kScratchBytes = ADAFLASH_NOALLOC_WORKSPACE_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up once per device).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail_with(ADAFLASH_E_HIP, "no current HIP device for the no-allocation workspace");
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return fail_with(ADAFLASH_E_HIP, "hipGetSymbolAddress of the workspace array failed");
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ADAFLASH_OK;
}

}  // namespace
}  // namespace adaflash

using namespace adaflash;

extern "C" {

int adaflash_verify_noalloc(adaflash_dtype dtype, const void* target_logits, const void* draft_logits,
                            const int32_t* draft_tokens, const int32_t* verify_len, const float* uniforms, int B,
                            int k, int V, float T, int32_t* accept_len, int32_t* out_tokens, float* margins,
                            float clip_c, float lambda, int32_t* row_offsets, float* loss_ce, float* loss_rkl,
                            void* grad_draft, int32_t* status_flags, void* stream) {
  const size_t need = adaflash_workspace_bytes(B, k, V);
  if (need == 0)
    return fail_with(ADAFLASH_E_INVALID,
                     "invalid sizes: need B >= 0, 1 <= k <= 64, 1 <= V <= 2^20, B*(k+1) < 2^24");
  if (need > kScratchBytes)
    return fail_with(ADAFLASH_E_UNSUPPORTED,
                     "batch too large for the no-allocation workspace (adaflash_workspace_bytes(B, k, V) must not "
                     "exceed ADAFLASH_NOALLOC_WORKSPACE_BYTES); use adaflash_verify with a workspace");
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != ADAFLASH_OK) return rc;
  return verify_impl(0, dtype, target_logits, draft_logits, draft_tokens, verify_len, uniforms, B, k, V, T,
                     accept_len, out_tokens, margins, clip_c, lambda, row_offsets, loss_ce, loss_rkl, grad_draft,
                     status_flags, ws, kScratchBytes, stream);
}

}  // extern "C"
