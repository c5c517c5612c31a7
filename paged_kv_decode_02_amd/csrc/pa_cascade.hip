// Shared-prefix (cascade / Hydragen) decode for gfx950 (MI355X).
//
// A group is a contiguous range of sequences whose block tables start with
// the same prefix pages (shared blocks, SwiftLLM page section 3.1).  The
// Tokasaurus page ("dynamic prefix identification") describes attending to
// the shared prefix once for the whole group: the group's queries against
// the prefix keys form one dense product.  Attention over prefix + suffix is
// then the log-sum-exp merge of attention over each part.
//
// Three launches on the caller's stream:
//  1. prefix_kernel (MFMA): per (group, row chunk, key split, kv-head) a
//     workgroup of 8 waves takes up to 256 query rows -- (member, q-head)
//     pairs of the kv-head, folded into one tile dimension the way
//     TokenSpeed's fold_sq_factor folds query tokens (TokenSpeed deep-dive
//     section 7.2) -- against one split of the prefix keys, FlashAttention
//     style: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16,
//     online softmax in between.  Writes one partial (o, log2-sum-exp) per
//     (member, head, split) and each member's first suffix page.
//  2. stream_decode_kernel in cascade mode over the suffix pages only.
//  3. cascade_merge_kernel: per (sequence, kv-head), the prefix splits and
//     the suffix partial(s) merged by log-sum-exp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __attribute__((address_space(3))) void* LdsPtr;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPrefixRows = 256;   // query rows per workgroup (8 waves x 32)
constexpr int kKeyTile = 64;       // keys per LDS tile (4 pages)
constexpr int kVtStride = 72;      // bf16 per row of the transposed V tile (64 + 8 pad)

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// MFMA 16x16x32 operand layout (wave64): A (16 x 32): lane l holds row l%16,
// k = 8*(l/16) .. +8; B (32 x 16): lane l holds column l%16, the same k;
// C (16 x 16): lane l holds column l%16, rows 4*(l/16) .. +4.
template <int G>
__global__ __launch_bounds__(512) void prefix_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ group_off,
    const int32_t* __restrict__ prefix_lens, int RC, int nks, int kps, int Hkv, int num_pages, float scale_log2,
    int32_t* __restrict__ begin_pages, float* __restrict__ pre_o, float* __restrict__ pre_lse) {
  constexpr int D = 128;
  constexpr int TILE = 16 * D * 2;  // bytes of one (page, kv-head) tile
  __shared__ uint4 k_lds[kKeyTile * 16];             // [key][16 chunks], chunk XOR-swizzled by key
  __shared__ uint16_t vt_lds[D * kVtStride];        // V^T: [d][key]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  int bx = blockIdx.x;
  const int ks = bx % nks;
  bx /= nks;
  const int rc = bx % RC;
  const int g = bx / RC;
  const int kvh = blockIdx.y;
  const int Hq = Hkv * G;
  const int off0 = group_off[g];
  const int n_g = group_off[g + 1] - off0;
  const int P = prefix_lens[g];  // prefix tokens (whole pages)
  if (kvh == 0 && rc == 0 && ks == 0)
    for (int i = tid; i < n_g; i += 512) begin_pages[off0 + i] = P / 16;
  const int R = n_g * G;
  const int k_lo = ks * kps;
  const int k_hi = min(P, k_lo + kps);
  if (k_lo >= k_hi || rc * kPrefixRows >= R || n_g <= 0) return;  // uniform over the workgroup

  const int row0 = rc * kPrefixRows + wv * 32;  // first of this wave's 32 query rows
  const int col = lane & 15;
  const int lg = lane >> 4;
  // Q^T operand (B of S^T = K Q^T): row r = row0 + 16 rb + col, d = 32 c + 8 lg.
  u32x4 qb[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = row0 + rb * 16 + col;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (r < R) {
        const int64_t qi = (static_cast<int64_t>(off0 + r / G) * Hq + kvh * G + r % G) * D + c * 32 + lg * 8;
        qb[rb][c] = *reinterpret_cast<const u32x4*>(q + qi);
      } else {
        qb[rb][c] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  const int32_t* bt = block_tables + static_cast<int64_t>(off0) * max_blocks;
  const char* kbytes = reinterpret_cast<const char*>(k_pool);
  const char* vbytes = reinterpret_cast<const char*>(v_pool);

  f32x4 o[8][2];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};

  for (int kt = k_lo; kt < k_hi; kt += kKeyTile) {
    const int nk = min(kKeyTile, k_hi - kt);  // keys of this tile that exist (whole pages)
    int pid[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pi = kt / 16 + min(j, nk / 16 - 1);
      pid[j] = min(max(bt[pi], 0), num_pages - 1);
    }
    // K tile -> LDS: slot (i*8 + wave)*64 + lane holds key slot/16, chunk
    // (slot%16) ^ (key%16).
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int slot = (i * 8 + wv) * 64 + lane;
      const int key = slot >> 4;
      const int ch = (slot & 15) ^ (key & 15);
      const char* src = kbytes + (static_cast<int64_t>(pid[key >> 4]) * Hkv + kvh) * TILE + (key & 15) * (D * 2) + ch * 16;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (LdsPtr)(&k_lds[(i * 8 + wv) * 64]), 16,
                                       0, 0);
    }
    // V tile -> registers -> transposed into LDS.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = i * 512 + tid;
      const int key = u >> 4;
      const int dc = u & 15;
      const char* src = vbytes + (static_cast<int64_t>(pid[key >> 4]) * Hkv + kvh) * TILE + (key & 15) * (D * 2) + dc * 16;
      const u32x4 v = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt_lds[(dc * 8 + 2 * e) * kVtStride + key] = static_cast<uint16_t>(v[e] & 0xffffu);
        vt_lds[(dc * 8 + 2 * e + 1) * kVtStride + key] = static_cast<uint16_t>(v[e] >> 16);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // S^T = K Q^T: s[kb][rb] holds keys 16 kb + 4 lg + i, query row 16 rb + col.
    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = kb * 16 + col;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cc = c * 4 + lg;
        const u32x4 a = *reinterpret_cast<const u32x4*>(&k_lds[key * 16 + (cc ^ (key & 15))]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) s[kb][rb] = mfma16x16x32(a, qb[rb][c], s[kb][rb]);
      }
    }
    // Online softmax per query row (column of S^T); the 64 keys of a row are
    // spread over this lane's 16 values and the lanes l^16, l^32, l^48.
    u32x4 pb[2][2];  // P^T operand: [rb][key half]
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb * 16 + lg * 4 + i;
          const float x = key < nk ? s[kb][rb][i] * scale_log2 : -INFINITY;
          s[kb][rb][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = max_xor32(max_xor16(mx));
      const float mn = fmaxf(m[rb], mx);
      const float alpha = fast_exp2(m[rb] - mn);
      m[rb] = mn;
      float ps = 0.f;
      uint32_t pw[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = fast_exp2(s[kb][rb][i] - mn);
          ps += p[i];
        }
        pw[kb][0] = bf16_bits_rne(p[0]) | (bf16_bits_rne(p[1]) << 16);
        pw[kb][1] = bf16_bits_rne(p[2]) | (bf16_bits_rne(p[3]) << 16);
      }
      lsum[rb] = lsum[rb] * alpha + ps;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db][rb] *= alpha;
      // k slots 8 lg .. 8 lg + 7 of key half hf = keys 32 hf + 4 lg + [0, 4)
      // and 32 hf + 16 + 4 lg + [0, 4): the same order the V^T operand uses.
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        pb[rb][hf] = u32x4{pw[2 * hf][0], pw[2 * hf][1], pw[2 * hf + 1][0], pw[2 * hf + 1][1]};
    }
    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = db * 16 + col;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(&vt_lds[d * kVtStride + hf * 32 + lg * 4]);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(&vt_lds[d * kVtStride + hf * 32 + 16 + lg * 4]);
        const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) o[db][rb] = mfma16x16x32(a, pb[rb][hf], o[db][rb]);
      }
    }
    __syncthreads();
  }

  // Partials: o / l per query row, log2-sum-exp.
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float lt = add_xor32(add_xor16(lsum[rb]));
    const int r = row0 + rb * 16 + col;
    if (r < R) {
      const int sq = off0 + r / G;
      const int h = r % G;
      const int64_t pr = ((static_cast<int64_t>(sq) * Hkv + kvh) * nks + ks) * G + h;
      const float inv = 1.0f / lt;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const f32x4 v = o[db][rb] * inv;
        *reinterpret_cast<f32x4*>(pre_o + pr * D + db * 16 + lg * 4) = v;
      }
      if (lg == 0) pre_lse[pr] = m[rb] + fast_log2(lt);
    }
  }
}

// Final merge per (sequence, kv-head): the prefix splits of the sequence's
// group (from begin_pages: the prefix length) and its suffix, which is one
// partial (seq_part) when a single wave covered it and one partial per wave
// otherwise.
template <typename T, int D, int G>
__global__ __launch_bounds__(64) void cascade_merge_kernel(
    T* __restrict__ out, float* __restrict__ lse_out, int S, int Hkv, int W, int nks, int kps,
    const int32_t* __restrict__ begin_pages, const float* __restrict__ pre_o, const float* __restrict__ pre_lse,
    const float* __restrict__ seq_part, const int32_t* __restrict__ seq_info, const float* __restrict__ part_o,
    const float* __restrict__ part_lse) {
  constexpr int EPL = D / 64;
  const int lane = lane_id();
  const int s = blockIdx.x;
  const int kvh = blockIdx.y;
  const int Hq = Hkv * G;
  const int np = min(nks, (begin_pages[s] * 16 + kps - 1) / kps);  // prefix splits with keys
  const int w0 = seq_info[4 * s + 0];
  const int w1 = seq_info[4 * s + 1];
  const int slot0 = seq_info[4 * s + 2];
  const bool shared = w1 > w0;
  if (shared && (w0 < 0 || w1 >= W || slot0 < 0 || slot0 > 1)) return;
  const int ns = shared ? (w1 - w0 + 1) : 1;
  const int n = np + ns;
  // Partial j: prefix split j < np, else suffix part j - np.
  auto lse_at = [&](int j, int h) -> float {
    if (j < np) return pre_lse[((static_cast<int64_t>(s) * Hkv + kvh) * nks + j) * G + h];
    const int k = j - np;
    if (!shared) return seq_part[static_cast<int64_t>(S) * Hq * D + static_cast<int64_t>(s) * Hq + kvh * G + h];
    return part_lse[((static_cast<int64_t>(w0 + k) * Hkv + kvh) * 2 + (k == 0 ? slot0 : 0)) * G + h];
  };
  auto o_at = [&](int j, int h) -> const float* {
    if (j < np) return pre_o + (((static_cast<int64_t>(s) * Hkv + kvh) * nks + j) * G + h) * D;
    const int k = j - np;
    if (!shared) return seq_part + (static_cast<int64_t>(s) * Hq + kvh * G + h) * D;
    return part_o + (((static_cast<int64_t>(w0 + k) * Hkv + kvh) * 2 + (k == 0 ? slot0 : 0)) * G + h) * D;
  };
#pragma unroll 1
  for (int h = 0; h < G; ++h) {
    float M = -INFINITY;
    for (int j = lane; j < n; j += 64) M = fmaxf(M, lse_at(j, h));
    M = wave_max(M);
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    float wsum = 0.f;
    for (int j = 0; j < n; ++j) {
      const float a = fast_exp2(lse_at(j, h) - M);
      wsum += a;
      const float* src = o_at(j, h) + lane * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(a, src[e], acc[e]);
    }
    const float inv = 1.0f / wsum;
    const int64_t row = static_cast<int64_t>(s) * Hq + kvh * G + h;
    if constexpr (sizeof(T) == 2) {
      if constexpr (EPL == 2) {
        reinterpret_cast<uint32_t*>(out)[row * (D / 2) + lane] =
            bf16_bits_rne(acc[0] * inv) | (bf16_bits_rne(acc[1] * inv) << 16);
      } else {
        reinterpret_cast<uint16_t*>(out)[row * D + lane] = static_cast<uint16_t>(bf16_bits_rne(acc[0] * inv));
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) reinterpret_cast<float*>(out)[row * D + lane * EPL + e] = acc[e] * inv;
    }
    if (lse_out && lane == 0) lse_out[row] = (M + fast_log2(wsum)) * kLn2;
  }
}

template <int G>
int launch_cascade_g(const CascadeLaunch& c) {
  const DecodeLaunch& a = c.base;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  char* ws = static_cast<char*>(c.workspace);
  const CascadeLayout& L = c.layout;
  int32_t* begin_pages = reinterpret_cast<int32_t*>(ws + L.begin_offset);
  float* seq_part = reinterpret_cast<float*>(ws + L.seq_part_offset);
  float* pre_o = reinterpret_cast<float*>(ws + L.pre_o_offset);
  float* pre_lse = reinterpret_cast<float*>(ws + L.pre_lse_offset);
  const float scale_log2 = a.scale * kLog2e;
  profile_before(a.stream);
  hipLaunchKernelGGL((prefix_kernel<G>), dim3(c.num_groups * c.row_chunks * c.nks, a.num_kv_heads), dim3(512), 0,
                     st, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_pool),
                     static_cast<const uint16_t*>(a.v_pool), a.block_tables, a.max_blocks, c.group_offsets,
                     c.prefix_lens, c.row_chunks, c.nks, c.kps, a.num_kv_heads, static_cast<int>(a.num_pages),
                     scale_log2, begin_pages, pre_o, pre_lse);
  profile_after(a.stream);
  if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_prefix_cascade: prefix kernel launch failed");
  // Suffix: the stream decode kernel over the pages after each prefix.
  DecodeLaunch sfx = a;
  sfx.workspace = ws + L.stream_offset;
  sfx.workspace_bytes = c.workspace_bytes - L.stream_offset;
  sfx.total_pages = c.suffix_pages;
  StreamPlan plan;
  int rc = launch_stream(sfx, begin_pages, seq_part, /*merge=*/false, &plan);
  if (rc) return rc;
  char* sws = static_cast<char*>(sfx.workspace);
  hipLaunchKernelGGL((cascade_merge_kernel<uint16_t, 128, G>), dim3(a.num_seqs, a.num_kv_heads), dim3(64), 0, st,
                     static_cast<uint16_t*>(a.out), a.lse_out, a.num_seqs, a.num_kv_heads,
                     static_cast<int>(plan.waves), c.nks, c.kps, begin_pages, pre_o, pre_lse, seq_part,
                     reinterpret_cast<const int32_t*>(sws + plan.layout.info_offset),
                     reinterpret_cast<const float*>(sws + plan.layout.o_offset),
                     reinterpret_cast<const float*>(sws + plan.layout.lse_offset));
  if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_prefix_cascade: merge kernel launch failed");
  return PA_OK;
}

}  // namespace

bool cascade_supported(pa_dtype dtype, int32_t head_dim, int32_t gqa) {
  return dtype == PA_BF16 && head_dim == 128 && (gqa == 1 || gqa == 2 || gqa == 4 || gqa == 8 || gqa == 16);
}

int launch_cascade(const CascadeLaunch& c) {
  switch (c.base.gqa) {
    case 1: return launch_cascade_g<1>(c);
    case 2: return launch_cascade_g<2>(c);
    case 4: return launch_cascade_g<4>(c);
    case 8: return launch_cascade_g<8>(c);
    case 16: return launch_cascade_g<16>(c);
  }
  return fail(PA_EUNSUPPORTED, "pa_prefix_cascade: gqa_ratio not built");
}

}  // namespace pa
