// KV append for gfx950 (MI355X): this step's new K/V rows into the paged
// cache, through the block tables (the cache model of the SwiftLLM page,
// section 3.1: a sequence's rows live in fixed-size blocks named by its
// table, handed out as it grows).
//
// One wave per new token.  The wave finds the token's segment in the
// device copy of cu_q_lens (a two-level ballot search: one load per lane
// over a coarse grid of the offsets, then one over the chosen stretch),
// its row pos = context_lens[s] - q_len + i and the page holding that row,
// then copies the token's rows of every kv-head, K and V, in 16-byte
// pieces: the reads are the token's contiguous [Hkv, D] rows (1 KB per
// instruction), the writes one contiguous row per (page, kv-head).  Pure
// data movement, bound by HBM: 2 x (read + write) x Hkv x D x element
// bytes per token.
#include <hip/hip_runtime.h>

#include <string>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kTokensPerBlock = 4;  // one wave each

// The segment holding token t: the largest s < S with cu[s] <= t (cu is
// non-decreasing with cu[0] = 0 <= t, and t < cu[S]); empty segments are
// passed over because the next segment starts at the same offset.
__device__ __forceinline__ int segment_of(const int32_t* __restrict__ cu, int S, int t) {
  const int lane = lane_id();
  const int per = (S + 63) >> 6;
  const int ic = lane * per;
  const unsigned long long bc = __ballot(ic < S && cu[ic] <= t);  // lane 0 always set
  const int lo = (63 - __clzll(bc)) * per;
  const int hi = min(lo + per, S);
  int ans = lo;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const unsigned long long b = __ballot(i < hi && cu[i] <= t);
    if (b == 0ull) break;
    ans = base + 63 - __clzll(b);
    if (ans < min(base + 64, hi) - 1) break;  // the set lanes are a prefix: the last one is found
  }
  return ans;
}

__global__ __launch_bounds__(64 * kTokensPerBlock) void kv_append_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ ctx, int S, int T, int Hkv, int row_bytes,
    int num_pages) {
  const int lane = lane_id();
  const int t = static_cast<int>(blockIdx.x) * kTokensPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  const int s = __builtin_amdgcn_readfirstlane(segment_of(cu, S, t));
  const int c0 = cu[s];
  const int n = cu[s + 1] - c0;
  const int pos = ctx[s] - n + (t - c0);
  // (Device copies that disagree with the validated host copies must not
  // move a write out of the table row or the pool.)
  if (pos < 0 || pos >= static_cast<int64_t>(max_blocks) * kBlockSize) return;
  const int pid = block_tables[static_cast<int64_t>(s) * max_blocks + (pos / kBlockSize)];
  if (pid < 0 || pid >= num_pages) return;
  const int slot = pos % kBlockSize;
  const int cpr = row_bytes / 16;  // 16-byte pieces per row
  const int nch = Hkv * cpr;       // pieces per token and pool
  const int64_t src = static_cast<int64_t>(t) * Hkv * row_bytes;
  const int64_t page = static_cast<int64_t>(pid) * Hkv;
  // Two pieces of K and two of V in flight per lane before the stores.
  for (int c = lane; c < nch; c += 128) {
    const int c1 = c + 64;
    const bool two = c1 < nch;
    const uint4 k0 = *reinterpret_cast<const uint4*>(k_new + src + static_cast<int64_t>(c) * 16);
    const uint4 v0 = *reinterpret_cast<const uint4*>(v_new + src + static_cast<int64_t>(c) * 16);
    uint4 k1 = make_uint4(0u, 0u, 0u, 0u), v1 = k1;
    if (two) {
      k1 = *reinterpret_cast<const uint4*>(k_new + src + static_cast<int64_t>(c1) * 16);
      v1 = *reinterpret_cast<const uint4*>(v_new + src + static_cast<int64_t>(c1) * 16);
    }
    const int g0 = c / cpr;
    const int64_t d0 = ((page + g0) * kBlockSize + slot) * row_bytes + static_cast<int64_t>(c - g0 * cpr) * 16;
    *reinterpret_cast<uint4*>(k_pool + d0) = k0;
    *reinterpret_cast<uint4*>(v_pool + d0) = v0;
    if (two) {
      const int g1 = c1 / cpr;
      const int64_t d1 = ((page + g1) * kBlockSize + slot) * row_bytes + static_cast<int64_t>(c1 - g1 * cpr) * 16;
      *reinterpret_cast<uint4*>(k_pool + d1) = k1;
      *reinterpret_cast<uint4*>(v_pool + d1) = v1;
    }
  }
}

}  // namespace

int launch_append(const AppendLaunch& a) {
  if (a.num_tokens > 0x7fffffffLL - kTokensPerBlock) return fail(PA_EUNSUPPORTED, "pa_kv_append: too many tokens");
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const unsigned blocks = static_cast<unsigned>((a.num_tokens + kTokensPerBlock - 1) / kTokensPerBlock);
  profile_before(a.stream);
  hipLaunchKernelGGL(kv_append_kernel, dim3(blocks), dim3(64 * kTokensPerBlock), 0, st,
                     static_cast<char*>(a.k_pool), static_cast<char*>(a.v_pool), static_cast<const char*>(a.k_new),
                     static_cast<const char*>(a.v_new), a.block_tables, a.max_blocks, a.cu_q_lens, a.context_lens,
                     a.num_segments, static_cast<int>(a.num_tokens), a.num_kv_heads, a.row_bytes,
                     static_cast<int>(a.num_pages));
  profile_after(a.stream);
  if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_kv_append: launch failed");
  return PA_OK;
}

}  // namespace pa
