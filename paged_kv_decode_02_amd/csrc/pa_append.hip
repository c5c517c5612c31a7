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

// max over the 16 lanes of a DPP row (each lane gets it)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppRor4>(v));
  return fmaxf(v, dpp<kDppRor8>(v));
}

// KV append into an fp8 cache: one wave per new token; its 2 x Hkv rows (K
// and V of every kv-head) are each quantised on their own -- scale =
// max(max |x|, 1e-10) / 448, codes = e4m3(clamp(x / scale, -448, 448)), all
// float32 with correctly rounded division (the token-group FP8 recipe of the
// tokenspeed deep-dive, section 6-4, with a group = one row) -- and written
// with their scale to the row's page and slot.  Four rows at a time: lanes
// 16 r .. 16 r + 15 take row r, lane c of them elements c * EPL .. +EPL.
template <typename TN, int D>
__global__ __launch_bounds__(64 * kTokensPerBlock) void kv_append_fp8_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, float* __restrict__ k_scales,
    float* __restrict__ v_scales, const TN* __restrict__ k_new, const TN* __restrict__ v_new,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ ctx, int S, int T, int Hkv, int num_pages) {
  constexpr int EPL = D / 16;  // elements per lane: 8 (D = 128) or 4 (D = 64)
  const int lane = lane_id();
  const int t = static_cast<int>(blockIdx.x) * kTokensPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  const int s = __builtin_amdgcn_readfirstlane(segment_of(cu, S, t));
  const int c0 = cu[s];
  const int n = cu[s + 1] - c0;
  const int pos = ctx[s] - n + (t - c0);
  if (pos < 0 || pos >= static_cast<int64_t>(max_blocks) * kBlockSize) return;
  const int pid = block_tables[static_cast<int64_t>(s) * max_blocks + (pos / kBlockSize)];
  if (pid < 0 || pid >= num_pages) return;
  const int slot = pos % kBlockSize;
  const int r = lane >> 4;  // row of the four this lane works on
  const int c = lane & 15;  // its piece of the row
  for (int r0 = 0; r0 < 2 * Hkv; r0 += 4) {
    const int ri = r0 + r;  // rows 0 .. Hkv-1: K of kv-head ri; Hkv .. 2 Hkv-1: V
    const bool live = ri < 2 * Hkv;
    const int kv = live && ri >= Hkv ? 1 : 0;
    const int g = live ? ri - kv * Hkv : 0;
    const TN* nw = kv ? v_new : k_new;
    const int64_t src = (static_cast<int64_t>(t) * Hkv + g) * D + c * EPL;
    float x[EPL];
    if constexpr (sizeof(TN) == 2) {
      uint32_t w[EPL / 2];
      if constexpr (EPL == 8) {
        const uint4 u = *reinterpret_cast<const uint4*>(nw + src);
        w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(nw + src);
        w[0] = u.x; w[1] = u.y;
      }
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) {
        x[2 * e] = bf16_lo(w[e]);
        x[2 * e + 1] = bf16_hi(w[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const float4 f = *reinterpret_cast<const float4*>(nw + src + e);
        x[e] = f.x; x[e + 1] = f.y; x[e + 2] = f.z; x[e + 3] = f.w;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = row16_max(amax);
    const float scale = fmaxf(amax, 1e-10f) / 448.0f;
    // x / scale, correctly rounded, by a product and a rare fallback: with
    // the correctly rounded reciprocal, q = x * (1 / scale) lies within 2
    // float32 ulps of the quotient, so it falls on the same side of every
    // rounding midpoint of the e4m3 grid unless it lies within a few ulps of
    // one (a normal value whose 20 mantissa bits below the 3 kept ones are
    // near 0x80000) or is below 2^-6 (the subnormal grid); only those
    // elements take the division.
    const float rcp = 1.0f / scale;
    float y[EPL];
    bool slow[EPL];
    bool any = false;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      y[e] = x[e] * rcp;
      const uint32_t b = __float_as_uint(y[e]) & 0x7fffffffu;
      const int d = static_cast<int>(b & 0xfffffu) - 0x80000;
      slow[e] = b < 0x3c800000u || (d >= -4 && d <= 4);
      any = any || slow[e];
    }
    if (__ballot(any) != 0ull) {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        if (slow[e]) y[e] = x[e] / scale;
    }
    // codes, four per word: v_cvt_pk_fp8_f32 rounds to the nearest e4m3fn
    // value, ties to even, subnormals included (values are in range after
    // the clamp)
    uint32_t code[EPL / 4];
#pragma unroll
    for (int e4 = 0; e4 < EPL / 4; ++e4) {
      float z[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = fminf(fmaxf(y[4 * e4 + e], -448.0f), 448.0f);
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(z[0], z[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(z[2], z[3], word, true);
      code[e4] = static_cast<uint32_t>(word);
    }
    if (live) {
      const int64_t row = (static_cast<int64_t>(pid) * Hkv + g) * kBlockSize + slot;
      uint8_t* dst = (kv ? v_pool : k_pool) + row * D + c * EPL;
      if constexpr (EPL == 8)
        *reinterpret_cast<uint2*>(dst) = make_uint2(code[0], code[1]);
      else
        *reinterpret_cast<uint32_t*>(dst) = code[0];
      if (c == 0) (kv ? v_scales : k_scales)[row] = scale;
    }
  }
}

}  // namespace

int launch_append_fp8(const AppendFp8Launch& a) {
  if (a.num_tokens > 0x7fffffffLL - kTokensPerBlock)
    return fail(PA_EUNSUPPORTED, "pa_kv_append_fp8: too many tokens");
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const unsigned blocks = static_cast<unsigned>((a.num_tokens + kTokensPerBlock - 1) / kTokensPerBlock);
  profile_before(a.stream);
#define PA_APPEND_FP8(TN, D)                                                                                         \
  hipLaunchKernelGGL((kv_append_fp8_kernel<TN, D>), dim3(blocks), dim3(64 * kTokensPerBlock), 0, st,                  \
                     static_cast<uint8_t*>(a.k_pool), static_cast<uint8_t*>(a.v_pool), a.k_scales, a.v_scales,      \
                     static_cast<const TN*>(a.k_new), static_cast<const TN*>(a.v_new), a.block_tables, a.max_blocks, \
                     a.cu_q_lens, a.context_lens, a.num_segments, static_cast<int>(a.num_tokens), a.num_kv_heads,   \
                     static_cast<int>(a.num_pages))
  if (a.new_dtype == PA_BF16 && a.head_dim == 128) PA_APPEND_FP8(uint16_t, 128);
  else if (a.new_dtype == PA_BF16 && a.head_dim == 64) PA_APPEND_FP8(uint16_t, 64);
  else if (a.new_dtype == PA_F32 && a.head_dim == 128) PA_APPEND_FP8(float, 128);
  else if (a.new_dtype == PA_F32 && a.head_dim == 64) PA_APPEND_FP8(float, 64);
  else return fail(PA_EUNSUPPORTED, "pa_kv_append_fp8: head_dim must be 64 or 128");
#undef PA_APPEND_FP8
  profile_after(a.stream);
  if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_kv_append_fp8: launch failed");
  return PA_OK;
}

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
