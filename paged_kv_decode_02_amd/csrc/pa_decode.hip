// Split-KV paged decode attention for gfx950 (MI355X).
//
// Work item = (sequence s, split j, kv-head g): one wave walks the pages
// [j*C, min((j+1)*C, pages_s)) of sequence s through its block table and
// computes, for the G q-heads that share kv-head g, the split's softmax
// partial (normalised output + log2-sum-exp).  A sequence with a single
// split writes its final output directly; otherwise a second kernel merges
// the partials by their log-sum-exp (TokenSpeed deep-dive, sections 7 and
// 7.1: split-KV partial output + LSE into a workspace, reduced by a second
// kernel).  Page walk, GQA head packing (one K/V pass serves all G heads
// of a kv-head, the analog of fold_sq_factor in section 7.2) and the
// per-step gather follow the PagedAttention cache of the SwiftLLM page,
// section 3.1.
//
// Per iteration a wave consumes one batch of 4 pages = 64 rows:
//  * K: the 4 (page, kv-head) tiles are read with coalesced 16-byte loads
//    (each instruction covers 1 KB contiguous), written to LDS with an XOR
//    swizzle, and read back transposed so that lane t holds row t.  Scores
//    are then lane-local dot products (bf16 pairs: v_dot2_f32_bf16) against
//    q, which is wave-uniform and read through the scalar cache.
//  * V: row-per-instruction dword loads (256 B contiguous per instruction
//    at D=128 bf16), so lane l holds columns (2l, 2l+1) of every row and
//    P.V needs no cross-lane reduction; the 64 probabilities of each head
//    are broadcast through LDS.
//  * Online softmax per head in the exp2 domain; masked rows are selected
//    out (never multiplied by zero) so NaN poison in unused rows cannot
//    leak.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

template <typename T, int D>
struct Geom {
  static constexpr int EB = sizeof(T);              // element bytes
  static constexpr int RD = D * EB / 4;             // dwords per row
  static constexpr int NCH = RD / 4;                // 16-byte chunks per row
  static constexpr int TILE = 16 * RD * 4;          // bytes of one (page, kv-head) tile
  static constexpr int NKI = 4 * TILE / 1024;       // 1 KB staging loads per batch
  static constexpr int VH = 64 / RD;                // row halves the V loads split into
  static constexpr int VT = 64 / VH;                // V rows each lane holds per batch
  static constexpr int EPD = 4 / EB;                // elements per dword
  static_assert(RD == 32 || RD == 64, "row must be 128 or 256 bytes");
};

// Pointer into the constant address space: loads through it are scalar.
typedef __attribute__((address_space(4))) const uint32_t ConstU32;
typedef __attribute__((address_space(3))) void* LdsPtr;

template <int EPD>
__device__ __forceinline__ void unpack(uint32_t w, float (&v)[EPD]) {
  if constexpr (EPD == 2) {
    v[0] = bf16_lo(w);
    v[1] = bf16_hi(w);
  } else {
    v[0] = __uint_as_float(w);
  }
}

// Physical page ids of table entries [pb, pb+4), clamped into the pool;
// entries at or past p_hi repeat the last valid one (its tile is then
// re-read from cache and its rows are masked out).
__device__ __forceinline__ void load_page_ids(const int32_t* __restrict__ bt, int pb, int p_hi, int num_pages,
                                              int (&pid)[4]) {
  if (pb + 4 <= p_hi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) pid[i] = bt[pb + i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) pid[i] = bt[min(pb + i, p_hi - 1)];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) pid[i] = min(max(pid[i], 0), num_pages - 1);
}

template <typename T, int D, int G>
__global__ __launch_bounds__(64) void split_decode_kernel(
    T* __restrict__ out, float* __restrict__ lse_out, const T* __restrict__ q, const T* __restrict__ k_pool,
    const T* __restrict__ v_pool, const int32_t* __restrict__ block_tables, const int32_t* __restrict__ ctx,
    int max_blocks, int S, int Hkv, int num_pages, float scale_log2, int C, int cap, float* __restrict__ part_o,
    float* __restrict__ part_lse) {
  using Gm = Geom<T, D>;
  constexpr int RD = Gm::RD, NCH = Gm::NCH, TILE = Gm::TILE, NKI = Gm::NKI, VH = Gm::VH, VT = Gm::VT,
                EPD = Gm::EPD;
  __shared__ uint4 k_lds[64 * NCH];
  __shared__ __align__(16) float p_lds[G * 64];

  const int lane = lane_id();
  const int kvh = blockIdx.y;
  const int Hq = Hkv * G;
  const char* kbytes = reinterpret_cast<const char*>(k_pool);
  const char* vbytes = reinterpret_cast<const char*>(v_pool);

  // Normally the grid has one wave per item; if the device lengths imply
  // more items than the host planned, waves take the extra ones in turn.
  for (int x = blockIdx.x, total = 0x7fffffff; x < total; x += gridDim.x) {
    ItemLoc loc;
    if (!locate_item(ctx, nullptr, S, max_blocks, C, x, loc)) return;
    // The lookup is wave-uniform; say so, so that everything derived from it
    // lives in scalar registers and branches on it are scalar branches.
    total = __builtin_amdgcn_readfirstlane(loc.total);
    const int s = __builtin_amdgcn_readfirstlane(loc.s);
    const int split_j = __builtin_amdgcn_readfirstlane(loc.j);
    const int split_n = __builtin_amdgcn_readfirstlane(loc.ns);
    const int L = ctx[s];
    const int64_t pg = (static_cast<int64_t>(L) + 15) >> 4;
    const int pages = static_cast<int>(pg < max_blocks ? pg : max_blocks);
    const int p_lo = split_j * C;
    const int p_hi = min(p_lo + C, pages);
    const int t_hi = min(p_hi * 16, L);
    const int32_t* bt = block_tables + static_cast<int64_t>(s) * max_blocks;
    const uint4* qh = reinterpret_cast<const uint4*>(q + (static_cast<int64_t>(s) * Hq + kvh * G) * D);

    float m[G], l[G], acc[G][EPD];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPD; ++e) acc[h][e] = 0.f;
    }

    // Page ids of the first batch; later batches' ids are fetched one batch
    // ahead, while the current batch computes.
    int pid[4];
    load_page_ids(bt, p_lo, p_hi, num_pages, pid);
    // Per-lane byte offsets of the K loads inside a page tile: instruction i
    // covers rows 4(i%per_tile)..+3 of tile i/per_tile (see below).
    constexpr int per_tile = TILE / 1024;
    uint32_t koff[per_tile];
#pragma unroll
    for (int r = 0; r < per_tile; ++r) {
      const int slot = r * 64 + lane;   // slot inside the tile's rows
      const int row = slot / NCH;       // row inside the tile (0..15)
      const int ch = (slot % NCH) ^ (row % NCH);
      koff[r] = row * (RD * 4) + ch * 16;
    }
    const uint32_t voff = ((VH == 2) ? (lane >> 5) * 32 * (RD * 4) : 0) + (lane % RD) * 4;

    for (int pb = p_lo; pb < p_hi; pb += 4) {
      const char* ktile[4];
      const char* vtile[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = (static_cast<int64_t>(pid[i]) * Hkv + kvh) * TILE;
        ktile[i] = kbytes + t;
        vtile[i] = vbytes + t;
      }
      // K: straight from HBM into LDS with 16-byte loads (global_load_lds),
      // each instruction covering 1 KB contiguous of one page tile.  Lane l
      // of instruction i fills LDS slot 64*i + l with the chunk the XOR
      // swizzle assigns to that slot, so the transposed read below (lane t
      // takes row t) is free of bank conflicts.
#pragma unroll
      for (int i = 0; i < NKI; ++i) {
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(ktile[i / per_tile] + koff[i % per_tile]),
                                         (LdsPtr)(&k_lds[i * 64]), 16, 0, 0);
      }
      // V: one row (or two half-rows) per instruction, one dword per lane.
      uint32_t vr[VT];
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        // VH == 2: lanes 32..63 read row t + 32, which lives two pages on.
        const char* base = (VH == 2) ? ((lane >> 5) ? vtile[(t / 16 + 2) & 3] - 32 * (RD * 4) : vtile[t / 16])
                                     : vtile[t / 16];
        vr[t] = *reinterpret_cast<const uint32_t*>(base + voff + (t % 16) * (RD * 4));
      }
      // Next batch's page ids (scalar loads) while this batch is in flight.
      int pid_next[4];
      if (pb + 4 < p_hi) load_page_ids(bt, pb + 4, p_hi, num_pages, pid_next);
      // Keep every load of the batch ahead of any use, so the whole batch is
      // in flight at once.
      __builtin_amdgcn_sched_barrier(0);
      const int nvalid = t_hi - pb * 16;  // rows of this batch that exist (1..64)
      if (nvalid < 64) {
#pragma unroll
        for (int t = 0; t < VT; ++t) {
          const int row = (VH == 2) ? t + (lane >> 5) * 32 : t;
          if (row >= nvalid) vr[t] = 0u;
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      uint4 kr[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) kr[c] = k_lds[lane * NCH + (c ^ (lane % NCH))];

      // Scores: lane = row.  q is wave-uniform: it is re-read from the
      // scalar cache each batch, one head at a time (the empty asm keeps the
      // compiler from hoisting all G*D values into scalar registers, which
      // would spill), and used as the scalar operand of v_dot2.
      float sc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sc[h] = 0.f;
        ConstU32* qrow = (ConstU32*)(uintptr_t)(qh + h * NCH);
        asm volatile("" : "+s"(qrow));
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          uint4 qv;
          qv.x = qrow[4 * c];
          qv.y = qrow[4 * c + 1];
          qv.z = qrow[4 * c + 2];
          qv.w = qrow[4 * c + 3];
          if constexpr (EPD == 2) {
            sc[h] = dot2_bf16(kr[c].x, qv.x, sc[h]);
            sc[h] = dot2_bf16(kr[c].y, qv.y, sc[h]);
            sc[h] = dot2_bf16(kr[c].z, qv.z, sc[h]);
            sc[h] = dot2_bf16(kr[c].w, qv.w, sc[h]);
          } else {
            sc[h] = fmaf(__uint_as_float(kr[c].x), __uint_as_float(qv.x), sc[h]);
            sc[h] = fmaf(__uint_as_float(kr[c].y), __uint_as_float(qv.y), sc[h]);
            sc[h] = fmaf(__uint_as_float(kr[c].z), __uint_as_float(qv.z), sc[h]);
            sc[h] = fmaf(__uint_as_float(kr[c].w), __uint_as_float(qv.w), sc[h]);
          }
        }
      }
      const bool valid = lane < nvalid;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float s2 = valid ? sc[h] * scale_log2 : -INFINITY;
        const float mn = fmaxf(m[h], wave_max(s2));
        const float alpha = fast_exp2(m[h] - mn);
        const float p = fast_exp2(s2 - mn);
        l[h] = l[h] * alpha + p;
#pragma unroll
        for (int e = 0; e < EPD; ++e) acc[h][e] *= alpha;
        m[h] = mn;
        p_lds[h * 64 + lane] = p;
      }
      __syncthreads();
      // P.V: lane owns one dword column of V; rows are uniform per step.
      const int rbase = (VH == 2) ? (lane >> 5) * 32 : 0;
#pragma unroll
      for (int t4 = 0; t4 < VT / 4; ++t4) {
        float4 p4[G];
#pragma unroll
        for (int h = 0; h < G; ++h) p4[h] = *reinterpret_cast<const float4*>(&p_lds[h * 64 + rbase + t4 * 4]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float v[EPD];
          unpack<EPD>(vr[t4 * 4 + u], v);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float p = u == 0 ? p4[h].x : u == 1 ? p4[h].y : u == 2 ? p4[h].z : p4[h].w;
#pragma unroll
            for (int e = 0; e < EPD; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pid[i] = pid_next[i];
    }

    // Finish the split.
    const int dw = lane % RD;
    const bool writer = (VH == 1) || (lane < 32);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float lt = wave_sum(l[h]);
      const float inv = 1.0f / lt;
      float o[EPD];
#pragma unroll
      for (int e = 0; e < EPD; ++e) {
        float a = acc[h][e];
        if constexpr (VH == 2) a += __shfl_xor(a, 32, 64);
        o[e] = a * inv;
      }
      const float lse2 = m[h] + fast_log2(lt);
      const int hq = kvh * G + h;
      if (split_n == 1) {
        const int64_t row = static_cast<int64_t>(s) * Hq + hq;
        if (writer) {
          if constexpr (EPD == 2) {
            const uint32_t packed = bf16_bits_rne(o[0]) | (bf16_bits_rne(o[1]) << 16);
            reinterpret_cast<uint32_t*>(out)[row * RD + dw] = packed;
          } else {
            reinterpret_cast<float*>(out)[row * D + dw] = o[0];
          }
        }
        if (lse_out && lane == 0) lse_out[row] = lse2 * kLn2;
      } else if (x < cap) {
        const int64_t r = (static_cast<int64_t>(x) * Hkv + kvh) * G + h;
        if (writer) {
#pragma unroll
          for (int e = 0; e < EPD; ++e) part_o[r * D + dw * EPD + e] = o[e];
        }
        if (lane == 0) part_lse[r] = lse2;
      }
    }
  }
}

// Merge the split partials of one (sequence, kv-head): out = sum_j a_j o_j /
// sum_j a_j with a_j = 2^(lse_j - max lse), lse = max + log2(sum a_j).
template <typename T, int D, int G>
__global__ __launch_bounds__(64) void merge_kernel(T* __restrict__ out, float* __restrict__ lse_out,
                                                   const int32_t* __restrict__ ctx, int max_blocks, int S, int Hkv,
                                                   int C, int cap, const float* __restrict__ part_o,
                                                   const float* __restrict__ part_lse) {
  constexpr int EPL = D / 64;  // output elements per lane
  const int lane = lane_id();
  const int s = blockIdx.x;
  const int kvh = blockIdx.y;
  const int Hq = Hkv * G;
  int base, ns;
  sequence_items(ctx, nullptr, S, max_blocks, C, s, base, ns);
  if (ns <= 1 || base + ns > cap) return;
  for (int h = 0; h < G; ++h) {
    const int64_t r0 = (static_cast<int64_t>(base) * Hkv + kvh) * G + h;
    const int64_t stride = static_cast<int64_t>(Hkv) * G;
    float M = -INFINITY;
    for (int j = lane; j < ns; j += 64) M = fmaxf(M, part_lse[r0 + j * stride]);
    M = wave_max(M);
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
    float wsum = 0.f;
    for (int j = 0; j < ns; ++j) {
      const int64_t r = r0 + j * stride;
      const float a = fast_exp2(part_lse[r] - M);
      wsum += a;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(a, part_o[r * D + lane * EPL + e], o[e]);
    }
    const float inv = 1.0f / wsum;
    const int64_t row = static_cast<int64_t>(s) * Hq + kvh * G + h;
    if constexpr (sizeof(T) == 2) {
      if constexpr (EPL == 2) {
        reinterpret_cast<uint32_t*>(out)[row * (D / 2) + lane] =
            bf16_bits_rne(o[0] * inv) | (bf16_bits_rne(o[1] * inv) << 16);
      } else {
        reinterpret_cast<uint16_t*>(out)[row * D + lane] = static_cast<uint16_t>(bf16_bits_rne(o[0] * inv));
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) reinterpret_cast<float*>(out)[row * D + lane * EPL + e] = o[e] * inv;
    }
    if (lse_out && lane == 0) lse_out[row] = (M + fast_log2(wsum)) * kLn2;
  }
}

template <typename T, int D, int G>
int launch_typed(const DecodeLaunch& a) {
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const float scale_log2 = a.scale * kLog2e;
  const int gx = static_cast<int>(std::min<int64_t>(a.items, 0x7fffffff));
  profile_before(a.stream);
  hipLaunchKernelGGL((split_decode_kernel<T, D, G>), dim3(gx, a.num_kv_heads), dim3(64), 0, st,
                     static_cast<T*>(a.out), a.lse_out, static_cast<const T*>(a.q), static_cast<const T*>(a.k_pool),
                     static_cast<const T*>(a.v_pool), a.block_tables, a.context_lens, a.max_blocks, a.num_seqs,
                     a.num_kv_heads, static_cast<int>(a.num_pages), scale_log2, a.split_pages,
                     static_cast<int>(a.capacity), a.part_o, a.part_lse);
  profile_after(a.stream);
  if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_decode: split kernel launch failed");
  if (a.any_multi) {
    hipLaunchKernelGGL((merge_kernel<T, D, G>), dim3(a.num_seqs, a.num_kv_heads), dim3(64), 0, st,
                       static_cast<T*>(a.out), a.lse_out, a.context_lens, a.max_blocks, a.num_seqs, a.num_kv_heads,
                       a.split_pages, static_cast<int>(a.capacity), a.part_o, a.part_lse);
    if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_decode: merge kernel launch failed");
  }
  return PA_OK;
}

template <typename T, int D>
int launch_g(const DecodeLaunch& a) {
  switch (a.gqa) {
    case 1: return launch_typed<T, D, 1>(a);
    case 2: return launch_typed<T, D, 2>(a);
    case 4: return launch_typed<T, D, 4>(a);
    case 8: return launch_typed<T, D, 8>(a);
    case 16: return launch_typed<T, D, 16>(a);
  }
  return fail(PA_EUNSUPPORTED, "pa_decode: gqa_ratio not built");
}

// Profiling ring (thread-local).
struct ProfileRing {
  std::vector<hipEvent_t> ev;  // begin/end pairs
  size_t next = 0;
};
thread_local ProfileRing g_prof;

}  // namespace

bool decode_supported(pa_dtype dtype, int32_t head_dim, int32_t gqa) {
  const bool g_ok = gqa == 1 || gqa == 2 || gqa == 4 || gqa == 8 || gqa == 16;
  if (!g_ok) return false;
  if (dtype == PA_BF16) return head_dim == 64 || head_dim == 128;
  if (dtype == PA_F32) return head_dim == 64;
  return false;
}

int launch_decode(const DecodeLaunch& a) {
  if (a.dtype == PA_BF16) {
    if (a.head_dim == 128) return launch_g<uint16_t, 128>(a);
    if (a.head_dim == 64) return launch_g<uint16_t, 64>(a);
  } else if (a.dtype == PA_F32) {
    if (a.head_dim == 64) return launch_g<float, 64>(a);
  }
  return fail(PA_EUNSUPPORTED, "pa_decode: shape not built");
}

void profile_before(void* stream) {
  if (g_prof.ev.empty() || g_prof.next + 2 > g_prof.ev.size()) return;
  (void)hipEventRecord(g_prof.ev[g_prof.next], static_cast<hipStream_t>(stream));
}

void profile_after(void* stream) {
  if (g_prof.ev.empty() || g_prof.next + 2 > g_prof.ev.size()) return;
  (void)hipEventRecord(g_prof.ev[g_prof.next + 1], static_cast<hipStream_t>(stream));
  g_prof.next += 2;
}

}  // namespace pa

using namespace pa;

extern "C" int pa_profile_enable(int32_t num_pairs) {
  clear_error();
  if (num_pairs < 0) return fail(PA_EINVAL, "pa_profile_enable: negative count");
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.next = 0;
  for (int32_t i = 0; i < 2 * num_pairs; ++i) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return fail(PA_EHIP, "pa_profile_enable: hipEventCreate failed");
    g_prof.ev.push_back(e);
  }
  return PA_OK;
}

extern "C" int pa_profile_collect(float* ms_out, int32_t cap) {
  clear_error();
  if (cap < 0 || (cap > 0 && !ms_out)) return fail(PA_EINVAL, "pa_profile_collect: bad output buffer");
  int32_t n = 0;
  for (size_t i = 0; i + 1 < g_prof.next && n < cap; i += 2) {
    if (hipEventSynchronize(g_prof.ev[i + 1]) != hipSuccess)
      return fail(PA_EHIP, "pa_profile_collect: hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_prof.ev[i], g_prof.ev[i + 1]) != hipSuccess)
      return fail(PA_EHIP, "pa_profile_collect: hipEventElapsedTime failed");
    ms_out[n++] = ms;
  }
  g_prof.next = 0;
  return n;
}
