// pa_decode_noalloc: pa_decode for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The stream kernel's scratch -- per-sequence records and
// the partial outputs of sequences shared by several waves -- lives in a
// file-scope device array instead of a caller workspace.  The kernels and the
// plan are pa_decode's; only where the scratch lives differs.
//
// Each GPU the library runs on holds its own copy of the array (loaded with
// the code object, kept until the process ends).  In host code the array's
// name is not a device address: its address on the current device comes from
// hipGetSymbolAddress, taken once per device and cached.  Every call on one
// GPU shares that GPU's array, so calls that overlap on one GPU (two streams,
// or two host threads) race on it; calls ordered on one stream do not.  The
// decode scratch needs no initialisation (each call writes every record and
// partial it later reads), so nothing is cleared between calls.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "pa_internal.h"

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (set up on the first
// call on each device, with that device current).
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return pa::fail(PA_EHIP, "pa_decode_noalloc: no current device");
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return pa::fail(PA_EHIP, std::string("pa_decode_noalloc: hipGetSymbolAddress failed: ") +
                                     hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                                 const int32_t* context_lens_host, int32_t num_seqs, int32_t num_kv_heads,
                                 int32_t gqa_ratio, int32_t head_dim, int32_t block_size, int64_t num_pages,
                                 float scale, pa_dtype dtype, int32_t split_pages, void* stream) {
  pa::clear_error();
  if (num_seqs == 0) return PA_OK;
  void* ws = nullptr;
  int rc = scratch_ptr(&ws);
  if (rc) return rc;
  rc = pa::decode_call(out, lse_out, q, k_pool, v_pool, nullptr, nullptr, false, block_tables, max_blocks,
                       context_lens, context_lens_host, num_seqs, num_kv_heads, gqa_ratio, head_dim, block_size,
                       num_pages, scale, dtype, split_pages, ws, kScratchBytes, stream, 0, 1, "pa_decode_noalloc",
                       /*plan_sized=*/true);
  if (rc == PA_EWORKSPACE)
    return pa::fail(PA_EWORKSPACE, "pa_decode_noalloc: the batch's plan needs more than the " +
                                       std::to_string(kScratchBytes >> 20) + " MiB scratch maximum (" +
                                       pa_last_error() + ")");
  return rc;
}
