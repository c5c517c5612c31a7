// MFMA tile kernels for gfx950 (MI355X): the dense parts of paged attention.
//
// Shared-prefix (cascade / Hydragen) decode.  A group is a contiguous range
// of sequences whose block tables start with the same prefix pages (shared
// blocks, SwiftLLM page section 3.1).  The Tokasaurus page ("dynamic prefix
// identification") describes attending to the shared prefix once for the
// whole group: the group's queries against the prefix keys form one dense
// product.  Attention over prefix + suffix is then the log-sum-exp merge of
// attention over each part.  Three launches on the caller's stream:
//  1. tile_kernel<G, false> (MFMA): per (group, row block, key split,
//     kv-head) a workgroup of 8 waves takes up to 128 query rows --
//     (member, q-head) pairs of the kv-head, folded into one tile dimension
//     the way TokenSpeed's fold_sq_factor folds query tokens (TokenSpeed
//     deep-dive section 7.2) -- against one split of the prefix keys,
//     FlashAttention style: S^T = K Q^T and O^T += V^T P^T on
//     v_mfma_f32_16x16x32_bf16, online softmax in between.  Writes one
//     partial (o, log2-sum-exp) per (member, head, split) and each member's
//     first suffix page.
//  2. The stream kernel (stream_mfma_kernel for 4 or more q-heads per
//     kv-head, stream_decode_kernel otherwise) over the suffix pages only.
//  3. cascade_merge_kernel: per (sequence, kv-head), the prefix splits and
//     the suffix partial(s) merged by log-sum-exp.
//
// Mixed batch (SARATHI-style piggybacking of decode tokens on prefill
// chunks, SwiftLLM page section 3.3; chunked prefill, TokenSpeed deep-dive
// section 5.1): prefill chunks (n > 1 new tokens, causal inside the chunk)
// and decode tokens in one call.
//  1. tile_kernel<G, true>: per (chunk, row block, key split, kv-head) the
//     chunk's (token, q-head) rows against its own keys, causal mask by
//     select; marks the chunks as "no decode pages" for step 2.
//  2. The stream kernel (+ its merge) over the decode segments.
//  3. chunk_merge_kernel: per (chunk token, kv-head), the key splits.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kRows = kPrefixRowsPerBlock;  // query rows per workgroup: 4 row groups of 32
constexpr int kKeyTile = 64;                  // keys per LDS tile (4 pages); each wave takes 32 of them
constexpr int kPidWindow = 256;               // page ids per LDS window (64 tiles)

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that leaves global loads in flight: __syncthreads()
// also waits for every outstanding vector memory access (vmcnt(0)), which
// would drain the tile prefetch at each barrier.  LDS accesses are waited
// for (lgkmcnt(0)); the DMA'd tiles are waited for explicitly by vmcnt.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// MFMA 16x16x32 operand layout (wave64): A (16 x 32): lane l holds row l%16,
// k = 8*(l/16) .. +8; B (32 x 16): lane l holds column l%16, the same k;
// C (16 x 16): lane l holds column l%16, rows 4*(l/16) .. +4.
//
// One workgroup = 8 waves = up to 128 query rows of one kv-head against the
// keys [k_lo, k_hi) of one block-table row, in tiles of 64 keys that stream
// through four LDS buffers (three tiles in flight while one is used).  Wave
// (row group rg, key half kh) takes query rows 32 rg .. +32 against keys
// 32 kh .. +32 of every tile, so two waves share each SIMD and every K/V byte
// in LDS is read by four waves; at the end the two key halves of a row group
// are merged through LDS.
//  PREFIX: unit = a group; rows are (member, q-head) pairs; keys are the
//          shared prefix, read through the first member's table; every row
//          sees every key.
//  CHUNK:  unit = a prefill chunk (segment with more than one query token);
//          rows are (token, q-head) pairs; keys are the segment's own rows;
//          token i sees keys t <= L - n + i (causal inside the chunk).
// Work items (unit, kv-head, key split) are numbered w; the row blocks of
// one item sit on consecutive slots of one XCD (workgroup i runs on XCD
// i % 8), so they fetch the same K/V tiles through the same L2.
// Output: one partial (normalised o, log2-sum-exp) per (row, key split);
// a row that sees no key of the split gets o = 0, lse = -inf.
template <int G, bool CHUNK>
__global__ __launch_bounds__(512) void tile_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ group_off, const int32_t* __restrict__ prefix_lens,
    ChunkList chunks, int S, int RC, int nks, int kps, int Hkv, int n_items, int num_pages, float scale_log2,
    int32_t* __restrict__ begin_pages, int32_t* __restrict__ seq_info, float* __restrict__ pre_o,
    float* __restrict__ pre_lse) {
  constexpr int D = 128;
  constexpr int TILE = 16 * D * 2;  // bytes of one (page, kv-head) tile
  // Four buffers each of K and V: [key][16 chunks of 16 bytes], the chunk
  // index XOR-swizzled by key % 16 so that column reads spread over the
  // banks.  The tiles arrive by DMA (dma16), waited for explicitly.
  // (Four arrays each, named statically in a loop unrolled by four.)
  __shared__ uint4 k_lds0[kKeyTile * 16], k_lds1[kKeyTile * 16], k_lds2[kKeyTile * 16], k_lds3[kKeyTile * 16];
  __shared__ uint4 v_lds0[kKeyTile * 16], v_lds1[kKeyTile * 16], v_lds2[kKeyTile * 16], v_lds3[kKeyTile * 16];
  // Page ids of the key range, in windows of kPidWindow pages (64 tiles),
  // two windows resident: reading an id from LDS is one short broadcast
  // read, where a scalar load from the table would put a cache round trip
  // in front of every tile's DMA.
  __shared__ int32_t pid_lds[2][kPidWindow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // (wave-uniform: scalar from here on)
  const int rg = wv & 3;   // row group
  const int kh = wv >> 2;  // key half
  const int Hq = Hkv * G;

  // Per-sequence set-up for the launches that follow (mixed batches: each
  // chunk's "no decode pages" mark and the "not shared" record the decode
  // merge reads).
  if constexpr (CHUNK) {
    if (blockIdx.x == 0) {
      for (int s = tid; s < S; s += 512) {
        const bool chunk = cu_q[s + 1] - cu_q[s] > 1;
        const int64_t pg = (static_cast<int64_t>(ctx[s]) + 15) >> 4;
        begin_pages[s] = chunk ? static_cast<int>(pg < max_blocks ? pg : max_blocks) : 0;
        if (chunk) {
          seq_info[4 * s + 0] = 0;
          seq_info[4 * s + 1] = 0;
          seq_info[4 * s + 2] = 0;
          seq_info[4 * s + 3] = 0;
        }
      }
    }
  }

  // Workgroup -> (item w, row block rc): slot j of XCD x holds row block
  // j % RC of item (j / RC) * 8 + x.
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int w = (slot / RC) * 8 + xcd;
  const int rc = slot % RC;
  if (w >= n_items) return;
  // Item w -> (unit u, kv-head, key split ks of nsplit, kpsplit keys each).
  // Chunks: items are numbered chunk by chunk in launch order (the chunks
  // with the longest splits first), each chunk's (kv-head, split) pairs
  // together; prefix groups: (group, kv-head, split) in order.
  int u, kvh, ks, nsplit, kpsplit;
  if constexpr (CHUNK) {
    int j = 0;
    while (chunks.item_end[j] <= w) ++j;  // w < n_items = item_end[n - 1]
    u = chunks.ord[j];
    const int local = w - (j > 0 ? chunks.item_end[j - 1] : 0);
    nsplit = chunks.nks[u];
    kpsplit = chunks.kps[u];
    ks = local % nsplit;
    kvh = local / nsplit;
  } else {
    nsplit = nks;
    kpsplit = kps;
    ks = w % nks;
    kvh = (w / nks) % Hkv;
    u = w / (nks * Hkv);
  }

  // rec_base: partial record (token or member, kv-head, split) of the
  // unit's first row.
  int seg, n_rows, k_lo, k_hi, L = 0, n_tok = 1, q_base;
  int64_t rec_base;
  if constexpr (CHUNK) {
    seg = chunks.seg[u];
    n_tok = cu_q[seg + 1] - cu_q[seg];
    L = ctx[seg];
    n_rows = n_tok * G;
    q_base = cu_q[seg];
    rec_base = chunks.rec[u];
    const int r_end = min(n_rows, (rc + 1) * kRows);
    const int i_max = (r_end - 1) / G;
    const int k_end = min(L, L - n_tok + i_max + 1);
    k_lo = ks * kpsplit;
    k_hi = min(k_end, k_lo + kpsplit);
  } else {
    const int off0 = group_off[u];
    const int n_g = group_off[u + 1] - off0;
    const int P = prefix_lens[u];  // prefix tokens (whole pages)
    if (kvh == 0 && rc == 0 && ks == 0)
      for (int i = tid; i < n_g; i += 512) begin_pages[off0 + i] = P / 16;
    seg = off0;
    n_rows = n_g * G;
    q_base = off0;
    rec_base = static_cast<int64_t>(off0) * Hkv * nks;
    k_lo = ks * kps;
    k_hi = min(P, k_lo + kps);
  }
  if (k_lo >= k_hi || rc * kRows >= n_rows) return;  // uniform over the workgroup

  const int row0 = rc * kRows + rg * 32;  // first of this wave's 32 query rows
  const int col = lane & 15;
  const int lg = lane >> 4;
  // Q^T operand (B of S^T = K Q^T): row r = row0 + 16 rb + col, d = 32 c + 8 lg.
  u32x4 qb[2][4];
  int vis[2];  // CHUNK: last visible key of the lane's query row
  // CHUNK: last key every row of this wave sees (uniform).
  const int vis_lo = CHUNK ? L - n_tok + min(row0, n_rows - 1) / G : 0x7fffffff;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = row0 + rb * 16 + col;
    vis[rb] = CHUNK ? L - n_tok + min(r, n_rows - 1) / G : 0x7fffffff;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (r < n_rows) {
        const int64_t qi = (static_cast<int64_t>(q_base + r / G) * Hq + kvh * G + r % G) * D + c * 32 + lg * 8;
        qb[rb][c] = *reinterpret_cast<const u32x4*>(q + qi);
      } else {
        qb[rb][c] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // Wait for the q rows here, before any tile DMA is in flight: the
  // compiler does not see the (inline-assembly) DMAs, and left to itself it
  // would wait for q -- with vmcnt(0), draining the tile pipeline -- at the
  // first MFMA of every tile.
  asm volatile("" ::"v"(qb[0][0]), "v"(qb[0][1]), "v"(qb[0][2]), "v"(qb[0][3]), "v"(qb[1][0]), "v"(qb[1][1]),
               "v"(qb[1][2]), "v"(qb[1][3]));
  const int32_t* bt = block_tables + static_cast<int64_t>(seg) * max_blocks;
  const char* kbytes = reinterpret_cast<const char*>(k_pool);
  const char* vbytes = reinterpret_cast<const char*>(v_pool);

  // O^T accumulators, and the float32 row sums of P over this lane's keys
  // (the lanes l ^ 16, l ^ 32, l ^ 48 hold the rest of the row's keys; the
  // sums are reduced over them at the end).  As in the decode kernels, the
  // normaliser sums the float32 probabilities while P.V takes them rounded
  // to bf16.
  f32x4 o[8][2];
  float lsum[2] = {0.f, 0.f};
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m[2] = {-INFINITY, -INFINITY};

  // K or V of tile t (keys k_lo + 64 t ..) -> an LDS buffer, by DMA: slot
  // (i*8 + wave)*64 + lane of a buffer holds key slot/16, chunk
  // (slot%16) ^ (key%16).  Keys past the tile's end (past the split or the
  // sequence) load the last valid key's row: finite values whose
  // probability is 0.
  const int nt = (k_hi - k_lo + kKeyTile - 1) / kKeyTile;
  // Lane offsets of a whole tile's DMA inside its page tile: slot
  // (i*8 + wave)*64 + lane -> key row % 16 and the swizzled chunk.
  uint32_t dma_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int sl = (i * 8 + wv) * 64 + lane;
    const int key = sl >> 4;
    dma_off[i] = (key & 15) * (D * 2) + ((sl & 15) ^ (key & 15)) * 16;
  }
  // Window w of page ids: pages k_lo/16 + 256 w .. +256 of the table row
  // (entries past the row read its last entry), one dword DMA per wave
  // from waves 0..3.
  const int pg0 = k_lo / 16;
  auto issue_pids = [&](int w) {
    if (wv < 4) {
      const int p = min(pg0 + w * kPidWindow + wv * 64 + lane, max_blocks - 1);
      dma4(bt + p, lds_offset(&pid_lds[w & 1][wv * 64]));
    }
  };
  // Two DMA loads per wave: this wave's share of tile t of the pool at
  // `pool` into buffer `dst`.  Page ids come from the LDS window (uniform).
  auto issue_half = [&](int t, const char* pool, uint4* dst) {
    const int kt = k_lo + t * kKeyTile;
    const int nk = min(kKeyTile, k_hi - kt);
    const int npg = (nk + 15) / 16;
    const int32_t* pw = &pid_lds[(t / (kPidWindow / 4)) & 1][(t * 4) % kPidWindow];
    int pid[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pid[j] = __builtin_amdgcn_readfirstlane(min(max(pw[min(j, npg - 1)], 0), num_pages - 1));
    if (nk == kKeyTile) {
      // Whole tile: DMA instruction i of this wave covers keys
      // 4 (8 i + wave) .. +4, all in page 2 i + wave / 4; the page's tile
      // base is scalar, the lane's row and chunk a fixed offset.
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t tb = (static_cast<int64_t>(pid[2 * i + wv / 4]) * Hkv + kvh) * TILE;
        dma16_sbase(pool + tb, dma_off[i], lds_offset(&dst[(i * 8 + wv) * 64]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int sl = (i * 8 + wv) * 64 + lane;
        const int key = sl >> 4;
        const int ch = (sl & 15) ^ (key & 15);
        const int kc = min(key, nk - 1);
        const int64_t off = (static_cast<int64_t>(pid[kc >> 4]) * Hkv + kvh) * TILE + (kc & 15) * (D * 2) + ch * 16;
        dma16(pool + off, lds_offset(&dst[(i * 8 + wv) * 64]));
      }
    }
  };
  // Per-lane byte offsets of the transposed V reads inside a buffer: lane
  // (group lg, j) reads row key0 + j/4, columns d0 + 4(j%4) .. +3, with
  // key0 = 32 kh + 4 lg (+16) and d0 = 16 db.
  const int tr_r = col >> 2;
  const int tr_c = col & 3;

  // Tile t's K and V into buffers kw, vw.
  auto issue_tile = [&](int t, uint4* kw, uint4* vw) {
    issue_half(t, kbytes, kw);
    issue_half(t, vbytes, vw);
  };

  // The first page-id window, then tiles 0..2 in flight before the first
  // is used.
  issue_pids(0);
  wait_vmcnt<0>();
  lds_barrier();
  if (nt > kPidWindow / 4) issue_pids(1);
  issue_tile(0, k_lds0, v_lds0);
  if (nt > 1) issue_tile(1, k_lds1, v_lds1);
  if (nt > 2) issue_tile(2, k_lds2, v_lds2);

  // One tile: wait for its DMA (each wave issued 4 loads per tile; tiles
  // t+1 and t+2 may stay in flight), start tile t+3 into the buffer freed by
  // tile t-1, compute.  Returns whether another tile follows.
  auto tile = [&](int t, const uint4* kb_lds, const uint4* vb_lds4, uint4* k_next, uint4* v_next) -> bool {
    const int kt = k_lo + t * kKeyTile;
    const int nk = min(kKeyTile, k_hi - kt);  // keys of this tile that exist
    const int ahead = min(2, nt - 1 - t);
    if (ahead >= 2)
      wait_vmcnt<8>();
    else if (ahead == 1)
      wait_vmcnt<4>();
    else
      wait_vmcnt<0>();
    // Every wave's part of this tile has landed, and every wave is done
    // with the buffer tile t-1 used.
    lds_barrier();
    if (t + 3 < nt) issue_tile(t + 3, k_next, v_next);
    // Page-id window w + 1 into the buffer window w - 1 used: its last
    // tile's DMA went out three tiles before window w began.  (Its loads,
    // issued after this tile's, are waited for by the tile waits that
    // follow, long before the first of its ids is read.)
    if (t % (kPidWindow / 4) == 0 && t > 0 && (t / (kPidWindow / 4) + 1) * (kPidWindow / 4) < nt)
      issue_pids(t / (kPidWindow / 4) + 1);
    const char* vb_lds = reinterpret_cast<const char*>(vb_lds4);

    // S^T = K Q^T: s[kb][rb] holds keys 32 kh + 16 kb + 4 lg + i, query
    // row 16 rb + col.
    f32x4 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kh * 32 + kb * 16 + col;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int cc = c * 4 + lg;
        const u32x4 a = *(LdsU4*)(&kb_lds[key * 16 + (cc ^ (key & 15))]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) s[kb][rb] = mfma16x16x32(a, qb[rb][c], s[kb][rb]);
      }
    }
    // Online softmax per query row (column of S^T); the 32 keys of a row in
    // this wave's half are spread over this lane's 8 values and the lanes
    // l^16, l^32, l^48.  Keys are masked (by select) only in tiles that need
    // it: the last, partial tile of a split, and chunk tiles that cross the
    // causal diagonal of this wave's rows.
    const bool need_mask = nk < kh * 32 + 32 || (CHUNK && kt + kh * 32 + 31 > vis_lo);
    if (need_mask) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kh * 32 + kb * 16 + lg * 4 + i;
            const bool ok = key < nk && (!CHUNK || kt + key <= vis[rb]);
            s[kb][rb][i] = ok ? s[kb][rb][i] : -INFINITY;
          }
    }
    float mx[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float x = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x = fmaxf(x, s[kb][rb][i]);
      mx[rb] = max_xor32(max_xor16(x)) * scale_log2;  // scale > 0 keeps the order
    }
    // Lazy rescaling: probabilities are taken against the running reference
    // m, which moves (and o, the row sums are rescaled) only when a row's
    // maximum exceeds it by more than 2^8 -- so p <= 256, and the rescale, a
    // wave-wide branch, is rare after the first tiles.
    if (__ballot(mx[0] > m[0] + 8.f || mx[1] > m[1] + 8.f) != 0ull) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float mn = fmaxf(m[rb], mx[rb]);
        // m = -inf (nothing visible yet): o and the sums are 0, any factor will do
        const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m[rb] - mn);
        m[rb] = mn;
        lsum[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][rb] *= alpha;
      }
    }
    u32x4 pb[2];  // P^T operand per row block
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      // A row with no visible key so far keeps m = -inf: its p are all 0.
      const float nref = m[rb] == -INFINITY ? 0.f : -m[rb];
      uint32_t pw[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = fast_exp2(fmaf(s[kb][rb][i], scale_log2, nref));
          lsum[rb] += p[i];
        }
        pw[kb][0] = bf16x2_rne(p[0], p[1]);
        pw[kb][1] = bf16x2_rne(p[2], p[3]);
      }
      // k slots 8 lg .. 8 lg + 7 = keys 32 kh + 4 lg + [0, 4) and
      // 32 kh + 16 + 4 lg + [0, 4): the same order the V^T operand uses.
      pb[rb] = u32x4{pw[0][0], pw[0][1], pw[1][0], pw[1][1]};
    }
    // O^T += V^T P^T; the V^T operand (d = 16 db + col, keys as above) comes
    // from two transposed reads of 4 keys each.
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      u32x2 part[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = kh * 32 + e * 16 + lg * 4 + tr_r;
        const int ch = (db * 2 + (tr_c >> 1)) ^ (row & 15);
        part[e] = lds_read_tr16(vb_lds + row * (D * 2) + ch * 16 + (tr_c & 1) * 8);
      }
      const u32x4 a = u32x4{part[0].x, part[0].y, part[1].x, part[1].y};
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) o[db][rb] = mfma16x16x32(a, pb[rb], o[db][rb]);
    }
    return t + 1 < nt;
  };
  for (int t = 0;; t += 4) {
    if (!tile(t, k_lds0, v_lds0, k_lds3, v_lds3)) break;
    if (!tile(t + 1, k_lds1, v_lds1, k_lds0, v_lds0)) break;
    if (!tile(t + 2, k_lds2, v_lds2, k_lds1, v_lds1)) break;
    if (!tile(t + 3, k_lds3, v_lds3, k_lds2, v_lds2)) break;
  }

  // Merge the two key halves of each row group through LDS (the buffers are
  // free once every wave is past its last tile): wave (rg, kh) hands its
  // state for row block 1 - kh to its partner and merges the partner's state
  // for row block kh into its own.  Record (rg, kh): o as [8 db][64 lanes]
  // f32x4 in K buffer rg at 8 KB * kh; m and the row sum per lane in V
  // buffer 0 at 128 floats * (2 rg + kh).
  // (the row sums over all of this wave's keys: its lanes l, l ^ 16, l ^ 32
  // and l ^ 48 hold the same row)
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) lsum[rb] = add_xor32(add_xor16(lsum[rb]));
  __syncthreads();
  uint4* kbuf = rg == 0 ? k_lds0 : rg == 1 ? k_lds1 : rg == 2 ? k_lds2 : k_lds3;
  float* xm = reinterpret_cast<float*>(v_lds0);
  // (Row block selected by value, not by a run-time index, so that o stays
  // in registers.)
  {
    f32x4* xo = reinterpret_cast<f32x4*>(kbuf) + kh * 512;
#pragma unroll
    for (int db = 0; db < 8; ++db) xo[db * 64 + lane] = kh ? o[db][0] : o[db][1];
    xm[(2 * rg + kh) * 128 + lane] = kh ? m[0] : m[1];
    xm[(2 * rg + kh) * 128 + 64 + lane] = kh ? lsum[0] : lsum[1];
  }
  __syncthreads();
  const int rb = kh;
  f32x4 om[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) om[db] = kh ? o[db][1] : o[db][0];
  const float mm = kh ? m[1] : m[0];
  const float lm = kh ? lsum[1] : lsum[0];
  const f32x4* po = reinterpret_cast<const f32x4*>(kbuf) + (1 - kh) * 512;
  const float* pm = xm + (2 * rg + 1 - kh) * 128;
  const float m2 = pm[lane];
  const float l2 = pm[64 + lane];
  const float mn = fmaxf(mm, m2);
  // A half that saw no visible key keeps m = -inf and o = l = 0.
  const float a1 = mm == -INFINITY ? 0.f : fast_exp2(mm - mn);
  const float a2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - mn);
  const float lt = lm * a1 + l2 * a2;
  const int r = row0 + rb * 16 + col;
  if (r < n_rows) {
    const int64_t pr = (rec_base + (static_cast<int64_t>(r / G) * Hkv + kvh) * nsplit + ks) * G + r % G;
    const bool any = lt > 0.f;
    const float inv = any ? 1.0f / lt : 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const f32x4 v = (om[db] * a1 + po[db * 64 + lane] * a2) * inv;
      *reinterpret_cast<f32x4*>(pre_o + pr * D + db * 16 + lg * 4) = v;
    }
    if (lg == 0) pre_lse[pr] = any ? mn + fast_log2(lt) : -INFINITY;
  }
}

// Merge the key splits of one chunk token (all G heads of a kv-head) and
// write its output row.
template <int G>
__global__ __launch_bounds__(64) void chunk_merge_kernel(uint16_t* __restrict__ out, float* __restrict__ lse_out,
                                                         const int32_t* __restrict__ ctx,
                                                         const int32_t* __restrict__ cu_q, ChunkList chunks, int Hkv,
                                                         const float* __restrict__ pre_o,
                                                         const float* __restrict__ pre_lse) {
  constexpr int D = 128;
  const int lane = lane_id();
  const int ct = chunks.tok_off[0] + static_cast<int>(blockIdx.x);  // chunk token
  const int kvh = blockIdx.y;
  const int Hq = Hkv * G;
  int u = 0;
  while (u + 1 < chunks.n && chunks.tok_off[u + 1] <= ct) ++u;
  const int i = ct - chunks.tok_off[u];
  const int s = chunks.seg[u];
  const int n_tok = cu_q[s + 1] - cu_q[s];
  if (i >= n_tok) return;
  const int L = ctx[s];
  // The key splits tile_kernel wrote for this token's row chunk.
  const int n_rows = n_tok * G;
  const int rc = (i * G) / kRows;
  const int i_max = (min(n_rows, (rc + 1) * kRows) - 1) / G;
  const int k_end = min(L, L - n_tok + i_max + 1);
  const int nks = chunks.nks[u];
  const int kps = chunks.kps[u];
  const int nsp = min(nks, (k_end + kps - 1) / kps);
#pragma unroll 1
  for (int h = 0; h < G; ++h) {
    const int64_t p0 = (chunks.rec[u] + (static_cast<int64_t>(i) * Hkv + kvh) * nks) * G + h;
    float M = -INFINITY;
    for (int j = lane; j < nsp; j += 64) M = fmaxf(M, pre_lse[p0 + static_cast<int64_t>(j) * G]);
    M = wave_max(M);
    float acc0 = 0.f, acc1 = 0.f, wsum = 0.f;
    for (int j = 0; j < nsp; ++j) {
      const int64_t pr = p0 + static_cast<int64_t>(j) * G;
      const float a = fast_exp2(pre_lse[pr] - M);  // -inf (no visible key) -> 0
      wsum += a;
      acc0 = fmaf(a, pre_o[pr * D + 2 * lane], acc0);
      acc1 = fmaf(a, pre_o[pr * D + 2 * lane + 1], acc1);
    }
    const float inv = 1.0f / wsum;
    const int64_t row = static_cast<int64_t>(cu_q[s] + i) * Hq + kvh * G + h;
    reinterpret_cast<uint32_t*>(out)[row * (D / 2) + lane] = bf16x2_rne(acc0 * inv, acc1 * inv);
    if (lse_out && lane == 0) lse_out[row] = (M + fast_log2(wsum)) * kLn2;
  }
}

// Final merge per (sequence, kv-head): the prefix splits of the sequence's
// group (from begin_pages: the prefix length) and its suffix, which is one
// partial (seq_part) when a single wave covered it and one partial per wave
// otherwise.
// (The stream kernel's partials hold PR rows per (wave, kv-head, slot):
// G, or 16 where its waves run on the matrix cores.)
template <typename T, int D, int G>
__global__ __launch_bounds__(64) void cascade_merge_kernel(
    T* __restrict__ out, float* __restrict__ lse_out, int S, int Hkv, int W, int nks, int kps,
    const int32_t* __restrict__ begin_pages, const float* __restrict__ pre_o, const float* __restrict__ pre_lse,
    const float* __restrict__ seq_part, const int32_t* __restrict__ seq_info, const float* __restrict__ part_o,
    const float* __restrict__ part_lse, int PR) {
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
    return part_lse[((static_cast<int64_t>(w0 + k) * Hkv + kvh) * 2 + (k == 0 ? slot0 : 0)) * PR + h];
  };
  auto o_at = [&](int j, int h) -> const float* {
    if (j < np) return pre_o + (((static_cast<int64_t>(s) * Hkv + kvh) * nks + j) * G + h) * D;
    const int k = j - np;
    if (!shared) return seq_part + (static_cast<int64_t>(s) * Hq + kvh * G + h) * D;
    return part_o + (((static_cast<int64_t>(w0 + k) * Hkv + kvh) * 2 + (k == 0 ? slot0 : 0)) * PR + h) * D;
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
            bf16x2_rne(acc[0] * inv, acc[1] * inv);
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
  ChunkList none;
  none.n = 0;
  const int n_items = c.num_groups * a.num_kv_heads * c.nks;
  const unsigned blocks = static_cast<unsigned>((n_items + 7) / 8 * 8 * c.row_chunks);
  hipLaunchKernelGGL((tile_kernel<G, false>), dim3(blocks), dim3(512), 0, st, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k_pool), static_cast<const uint16_t*>(a.v_pool),
                     a.block_tables, a.max_blocks, a.context_lens, nullptr, c.group_offsets, c.prefix_lens, none,
                     a.num_seqs, c.row_chunks, c.nks, c.kps, a.num_kv_heads, n_items, static_cast<int>(a.num_pages),
                     scale_log2, begin_pages, nullptr, pre_o, pre_lse);
  profile_after(a.stream);
  if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_prefix_cascade: prefix kernel launch failed");
  // Suffix: the stream decode kernel over the pages after each prefix.
  DecodeLaunch sfx = a;
  sfx.workspace = ws + L.stream_offset;
  sfx.workspace_bytes = c.workspace_bytes - L.stream_offset;
  sfx.total_pages = c.suffix_pages;
  sfx.timed = false;
  StreamPlan plan;
  int rc = launch_stream(sfx, begin_pages, seq_part, nullptr, /*merge=*/false, &plan);
  if (rc) return rc;
  char* sws = static_cast<char*>(sfx.workspace);
  hipLaunchKernelGGL((cascade_merge_kernel<uint16_t, 128, G>), dim3(a.num_seqs, a.num_kv_heads), dim3(64), 0, st,
                     static_cast<uint16_t*>(a.out), a.lse_out, a.num_seqs, a.num_kv_heads,
                     static_cast<int>(plan.waves), c.nks, c.kps, begin_pages, pre_o, pre_lse, seq_part,
                     reinterpret_cast<const int32_t*>(sws + plan.layout.info_offset),
                     reinterpret_cast<const float*>(sws + plan.layout.o_offset),
                     reinterpret_cast<const float*>(sws + plan.layout.lse_offset), plan.rows);
  if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_prefix_cascade: merge kernel launch failed");
  return PA_OK;
}

template <int G>
int launch_mixed_g(const MixedLaunch& mx) {
  const DecodeLaunch& a = mx.base;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  char* ws = static_cast<char*>(mx.workspace);
  const MixedLayout& L = mx.layout;
  int32_t* begin_pages = reinterpret_cast<int32_t*>(ws + L.begin_offset);
  float* pre_o = reinterpret_cast<float*>(ws + L.pre_o_offset);
  float* pre_lse = reinterpret_cast<float*>(ws + L.pre_lse_offset);
  char* sws = ws + L.stream_offset;
  // The stream kernel's per-sequence records start its workspace.
  int32_t* seq_info = reinterpret_cast<int32_t*>(sws + partial_layout(1, a.num_seqs, a.num_kv_heads,
                                                                      stream_rows(a.gqa), a.head_dim).info_offset);
  const float scale_log2 = a.scale * kLog2e;
  const ChunkPlan& plan = *mx.plan;
  auto chunk_list = [&](int b0) {
    ChunkList cl;
    cl.n = std::min(kMaxChunkSegments, mx.num_chunks - b0);
    for (int i = 0; i < cl.n; ++i) {
      cl.seg[i] = mx.chunk_seg[b0 + i];
      cl.tok_off[i] = mx.chunk_tok[b0 + i];
      cl.nks[i] = plan.nks[b0 + i];
      cl.kps[i] = plan.kps[b0 + i];
      cl.rec[i] = plan.rec[b0 + i];
      cl.ord[i] = i;
    }
    cl.tok_off[cl.n] = mx.chunk_tok[b0 + cl.n];
    // Longest work items first, so that the short ones fill in at the end.
    std::stable_sort(cl.ord, cl.ord + cl.n,
                     [&](int x, int y) { return plan.tiles[b0 + x] > plan.tiles[b0 + y]; });
    int items = 0;
    for (int j = 0; j < cl.n; ++j) {
      items += a.num_kv_heads * cl.nks[cl.ord[j]];
      cl.item_end[j] = items;
    }
    return cl;
  };
  if (mx.num_chunks > 0) {
    profile_before(a.stream);
    for (int b0 = 0; b0 < mx.num_chunks; b0 += kMaxChunkSegments) {
      const ChunkList cl = chunk_list(b0);
      const int n_items = cl.item_end[cl.n - 1];
      const unsigned blocks = static_cast<unsigned>((n_items + 7) / 8 * 8 * mx.row_chunks);
      hipLaunchKernelGGL((tile_kernel<G, true>), dim3(blocks), dim3(512), 0, st, static_cast<const uint16_t*>(a.q),
                         static_cast<const uint16_t*>(a.k_pool), static_cast<const uint16_t*>(a.v_pool),
                         a.block_tables, a.max_blocks, a.context_lens, mx.cu_q_lens, nullptr, nullptr, cl,
                         a.num_seqs, mx.row_chunks, 0, 0, a.num_kv_heads, n_items,
                         static_cast<int>(a.num_pages), scale_log2, begin_pages, seq_info, pre_o, pre_lse);
      if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_mixed_chunk: chunk kernel launch failed");
    }
    profile_after(a.stream);
  }
  if (mx.decode_pages > 0) {
    DecodeLaunch dec = a;
    dec.workspace = sws;
    dec.workspace_bytes = mx.workspace_bytes - L.stream_offset;
    dec.total_pages = mx.decode_pages;
    const int rc = launch_stream(dec, mx.num_chunks > 0 ? begin_pages : nullptr, nullptr, mx.cu_q_lens,
                                 /*merge=*/true, nullptr);
    if (rc) return rc;
  }
  for (int b0 = 0; b0 < mx.num_chunks; b0 += kMaxChunkSegments) {
    const ChunkList cl = chunk_list(b0);
    hipLaunchKernelGGL((chunk_merge_kernel<G>), dim3(cl.tok_off[cl.n] - cl.tok_off[0], a.num_kv_heads), dim3(64), 0,
                       st, static_cast<uint16_t*>(a.out), a.lse_out, a.context_lens, mx.cu_q_lens, cl, a.num_kv_heads,
                       pre_o, pre_lse);
    if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_mixed_chunk: chunk merge launch failed");
  }
  return PA_OK;
}

}  // namespace

bool mixed_supported(pa_dtype dtype, int32_t head_dim, int32_t gqa) { return cascade_supported(dtype, head_dim, gqa); }

int launch_mixed(const MixedLaunch& m) {
  if (m.num_chunks == 0) {
    DecodeLaunch dec = m.base;
    dec.workspace = static_cast<char*>(m.workspace) + m.layout.stream_offset;
    dec.workspace_bytes = m.workspace_bytes - m.layout.stream_offset;
    dec.total_pages = m.decode_pages;
    return launch_stream(dec, nullptr, nullptr, m.cu_q_lens, /*merge=*/true, nullptr);
  }
  switch (m.base.gqa) {
    case 1: return launch_mixed_g<1>(m);
    case 2: return launch_mixed_g<2>(m);
    case 4: return launch_mixed_g<4>(m);
    case 8: return launch_mixed_g<8>(m);
    case 16: return launch_mixed_g<16>(m);
  }
  return fail(PA_EUNSUPPORTED, "pa_mixed_chunk: gqa_ratio not built");
}

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
