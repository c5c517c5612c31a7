// MFMA tile kernels for gfx950 (MI355X): the dense parts of paged attention.
//
// Shared-prefix (cascade / Hydragen) decode.  A group is a contiguous range
// of sequences whose block tables start with the same prefix pages (shared
// blocks, SwiftLLM page section 3.1).  The Tokasaurus page ("dynamic prefix
// identification") describes attending to the shared prefix once for the
// whole group: the group's queries against the prefix keys form one dense
// product.  Attention over prefix + suffix is then the log-sum-exp merge of
// attention over each part.  Over bf16 pools or fp8 ones (e4m3fn codes
// widened exactly to bf16 in the tile, each key's K scale on its scores and
// V scale on its probabilities), three launches on the caller's stream:
//  1. tile_kernel<G, false, FP8> (MFMA): per (group, row block, key split,
//     kv-head) a workgroup of 4 waves takes up to 128 query rows --
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
// and decode tokens in one call, over bf16 pools or fp8 ones (e4m3fn codes
// and per-row scales, read as the prefix tiles read them).  With 4 or more
// q-heads per kv-head and decode tokens present, one launch:
//  1. mixed_kernel<G, FP8>: chunk workgroups (the tile body on one (chunk,
//     row block, key split, kv-head), causal mask by select) and decode
//     workgroups (two matrix-core stream waves, one run of decode pages
//     each) interleaved along each XCD's dispatch order, so the
//     matrix-bound and the HBM-bound work share the CUs for the whole
//     launch.
//  2. The decode merge, then chunk_merge_kernel: per (chunk token, kv-head),
//     the key splits.
// Otherwise tile_kernel<G, true, FP8> for the chunks, then the stream kernel
// (+ its merge) over the decode segments, then chunk_merge_kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>
#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_stream.h"

namespace pa {
namespace {

constexpr int kRows = kPrefixRowsPerBlock;  // query rows per workgroup: 4 waves of 32
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
// One workgroup = 4 waves = up to 128 query rows of one kv-head against the
// keys [k_lo, k_hi) of one block-table row, in tiles of 64 keys (4 pages)
// that stream through two LDS buffer pairs (tile t + 1 lands while tile t is
// used).  Wave w takes query rows 32 w .. +32 against all 64 keys of every
// tile, so every K/V byte in LDS is read by the four waves.  The workgroup
// needs 66 KB of LDS (35 KB over fp8 pools) and about 240 VGPRs per wave
// (220 for fp8), so two workgroups share a CU; their barriers are
// independent, and the matrix work of one overlaps the softmax of the other
// on the same SIMD.
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
constexpr int kTileThreads = 256;

template <int KT, int NB, bool FP8 = false>
struct TileLds {
  uint4 k[NB][KT * 16];         // [key][16 chunks of 16 bytes], chunk XOR-swizzled by tswz(key % 16)
  uint4 v[NB][KT * 16];         // the same layout
  int32_t pid[2][kPidWindow];   // page ids of the key range, two windows of 256 pages
};
// fp8 pools (e4m3fn codes, one float32 scale per (page, kv-head, slot)):
// rows of 128 codes, and each key's K and V scale.
template <int KT, int NB>
struct TileLds<KT, NB, true> {
  uint4 k[NB][KT * 8];          // [key][8 chunks of 16 codes], chunk XOR-swizzled by fswz(key)
  uint4 v[NB][KT * 8];          // the same layout
  float ks[NB][KT];             // K scale of each key of the tile
  float vs[NB][KT];             // V scale of each key of the tile
  int32_t pid[2][kPidWindow];
};

// Chunk swizzle of a K/V row in LDS: global chunk c of row r sits at LDS
// chunk c ^ (r % 16), so that the K operand read (16 lanes, 16 consecutive
// rows, one 16-byte chunk each) touches 16 distinct chunk slots.  (A swizzle
// that also spreads the transposed V reads, whose 4 rows x 2 chunks share 4
// slots here, measured no faster.)
__device__ __forceinline__ int tswz(int r) { return r & 15; }
// Rows of 128 bytes (fp8 codes): rows r and r + 8 would sit on the same
// banks of the 64-bank LDS; (r / 2) mod 8 spreads the 16 rows a K operand
// read touches over distinct chunk slots (the fp8 stream wave's layout).
__device__ __forceinline__ int fswz(int r) { return (r >> 1) & 7; }

// What one tile workgroup computes.
struct TileWork {
  int seg;          // block-table row the keys are read through
  int kvh;          // kv-head
  int n_rows;       // query rows of the unit
  int row_base;     // first row of this workgroup
  int k_lo, k_hi;   // key range
  int L, n_tok;     // CHUNK: the segment's rows and query tokens
  int q_base;       // q row of the unit's first token (chunk) or member (prefix)
  int64_t rec_base; // partial record of the unit's first row
  int nsplit, ks;   // key splits of the unit, and this one
};

// Workgroup slot -> its work; false if the slot has none.  Slot j of XCD x
// holds row block j % RC of item (j / RC) * 8 + x.  Chunks: items are
// numbered chunk by chunk in launch order (the chunks with the longest
// splits first), each chunk's (kv-head, split) pairs together; prefix
// groups: (group, kv-head, split) in order.  Prefix groups also record each
// member's first suffix page (by the first row block of split 0, kv-head 0).
template <int G, bool CHUNK>
__device__ __forceinline__ bool tile_work(int b, int RC, int n_items, int Hkv, int nks, int kps,
                                          const ChunkList& chunks, const int32_t* __restrict__ ctx,
                                          const int32_t* __restrict__ cu_q, const int32_t* __restrict__ group_off,
                                          const int32_t* __restrict__ prefix_lens, int32_t* __restrict__ begin_pages,
                                          TileWork& tw) {
  const int xcd = b & 7;
  const int slot = b >> 3;
  const int w = (slot / RC) * 8 + xcd;
  const int rc = slot % RC;
  if (w >= n_items) return false;
  int u;
  if constexpr (CHUNK) {
    int j = 0;
    while (chunks.item_end[j] <= w) ++j;  // w < n_items = item_end[n - 1]
    u = chunks.ord[j];
    const int local = w - (j > 0 ? chunks.item_end[j - 1] : 0);
    tw.nsplit = chunks.nks[u];
    const int kpsplit = chunks.kps[u];
    tw.ks = local % tw.nsplit;
    tw.kvh = local / tw.nsplit;
    tw.seg = chunks.seg[u];
    tw.n_tok = cu_q[tw.seg + 1] - cu_q[tw.seg];
    tw.L = ctx[tw.seg];
    tw.n_rows = tw.n_tok * G;
    tw.q_base = cu_q[tw.seg];
    tw.rec_base = chunks.rec[u];
    const int r_end = min(tw.n_rows, (rc + 1) * kRows);
    const int i_max = (r_end - 1) / G;
    const int k_end = min(tw.L, tw.L - tw.n_tok + i_max + 1);
    tw.k_lo = tw.ks * kpsplit;
    tw.k_hi = min(k_end, tw.k_lo + kpsplit);
  } else {
    tw.nsplit = nks;
    tw.ks = w % nks;
    tw.kvh = (w / nks) % Hkv;
    u = w / (nks * Hkv);
    const int off0 = group_off[u];
    const int n_g = group_off[u + 1] - off0;
    const int P = prefix_lens[u];  // prefix tokens (whole pages)
    if (tw.kvh == 0 && rc == 0 && tw.ks == 0)
      for (int i = threadIdx.x; i < n_g; i += kTileThreads) begin_pages[off0 + i] = P / 16;
    tw.seg = off0;
    tw.n_rows = n_g * G;
    tw.q_base = off0;
    tw.rec_base = static_cast<int64_t>(off0) * Hkv * nks;
    tw.k_lo = tw.ks * kps;
    tw.k_hi = min(P, tw.k_lo + kps);
    tw.L = 0;
    tw.n_tok = 1;
  }
  tw.row_base = rc * kRows;
  return tw.k_lo < tw.k_hi && tw.row_base < tw.n_rows;
}

// KT keys per tile (32 or 64: 2 or 4 pages), NB buffers (NB - 1 tiles in
// flight while one is used).  FP8: the pools hold e4m3fn codes with one
// float32 scale per (page, kv-head, slot) (k_scales, v_scales); K operands
// are read as codes and widened to bf16 pairs (exact), the V^T operand by
// the transposed 8-bit read; each key's K scale multiplies its scores, its V
// scale the probability P^T carries (the normaliser sums the plain
// probabilities), as in the fp8 stream wave.
template <int G, bool CHUNK, int KT, int NB, bool FP8 = false>
__device__ __forceinline__ void tile_body(const TileWork& tw, TileLds<KT, NB, FP8>& lds,
                                          const uint16_t* __restrict__ q, const void* __restrict__ k_pool,
                                          const void* __restrict__ v_pool, const int32_t* __restrict__ block_tables,
                                          int max_blocks, int Hkv, int num_pages, float scale_log2,
                                          float* __restrict__ pre_o, float* __restrict__ pre_lse,
                                          const float* __restrict__ k_scales = nullptr,
                                          const float* __restrict__ v_scales = nullptr) {
  constexpr int D = 128;
  constexpr int ROWB = FP8 ? D : 2 * D;  // bytes of one K/V row
  constexpr int NCHR = ROWB / 16;        // 16-byte chunks of a row
  constexpr int TILE = 16 * ROWB;        // bytes of one (page, kv-head) tile
  constexpr int KPL = 64 / NCHR;         // keys one 1 KB load covers (4, fp8 8)
  constexpr int LPP = 16 / KPL;          // 1 KB loads per page (4, fp8 2)
  constexpr int NKB = KT / 16;           // 16-key blocks of a tile
  constexpr int NKS = KT / 32;           // 32-key steps of P.V
  constexpr int LPW = KT / KPL / 4;      // 1 KB loads per wave per tile, each of K and V
  constexpr int TPW = kPidWindow * 16 / KT;  // tiles per page-id window
  static_assert(KT == 32 || KT == 64, "tiles of 2 or 4 pages");
  static_assert(!FP8 || KT == 64, "fp8 tiles of 64 keys (one 4-byte scale DMA per lane covers a tile)");
  static_assert(LPW >= 1 && LPP % LPW == 0, "a wave's loads of a whole tile stay in one page");
  auto swzf = [](int r) { return FP8 ? fswz(r) : tswz(r); };
  static_assert(NB >= 2 && NB <= 4 && TPW > NB, "buffer count");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // (wave-uniform: scalar from here on)
  const int Hq = Hkv * G;
  // (the work is uniform over the workgroup: keep it in scalar registers,
  // so that the page bases of the DMAs are scalar)
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  const int kvh = uni(tw.kvh), n_rows = uni(tw.n_rows), L = uni(tw.L), n_tok = uni(tw.n_tok);
  const int k_lo = uni(tw.k_lo), k_hi = uni(tw.k_hi), seg = uni(tw.seg), q_base = uni(tw.q_base);

  const int row0 = uni(tw.row_base) + wv * 32;  // first of this wave's 32 query rows
  const int col = lane & 15;
  const int lg = lane >> 4;
  // Q^T operand (B of S^T = K Q^T): row r = row0 + 16 rb + col, d = 32 c + 8 lg.
  u32x4 qb[2][4];
  int vis[2];  // CHUNK: last visible key of the lane's query row
  // CHUNK: last key every row of this wave sees (uniform).
  const int vis_lo = CHUNK ? L - n_tok + min(row0, n_rows - 1) / G : 0x7fffffff;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) vis[rb] = CHUNK ? L - n_tok + min(row0 + rb * 16 + col, n_rows - 1) / G : 0x7fffffff;
  const int32_t* bt = block_tables + static_cast<int64_t>(seg) * max_blocks;
  const char* kbytes = reinterpret_cast<const char*>(k_pool);
  const char* vbytes = reinterpret_cast<const char*>(v_pool);

  // O^T accumulators, and the float32 row sums of P over this lane's keys
  // (the lanes l ^ 16, l ^ 32, l ^ 48 hold the rest of the row's keys; the
  // sums are reduced over them at the end).  As in the decode kernels, the
  // normaliser sums the float32 probabilities while P.V takes them rounded
  // to bf16.
  f32x4 o[8][2];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum[2] = {0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};

  // K or V of tile t (keys k_lo + KT t ..) -> an LDS buffer, by DMA: the
  // tile's KT / 4 loads of 1 KB (4 keys each) are spread over the 4 waves;
  // load g covers page g / 4, keys 4 (g % 4) .. +3, and lane (lg, col) of it
  // writes LDS chunk col of key 4 (g % 4) + lg, which holds global chunk
  // col ^ tswz(key).  Keys past the tile's end (past the split or the
  // sequence) load the last valid key's row: finite values whose
  // probability is 0.
  const int nt = (k_hi - k_lo + KT - 1) / KT;
  uint32_t dma_off[LPW];  // inside a page tile, for this wave's loads
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int g = wv * LPW + i;
    const int key = KPL * (g % LPP) + lane / NCHR;
    dma_off[i] = key * ROWB + (((lane % NCHR) ^ swzf(key)) * 16);
  }
  // Window w of page ids: pages k_lo/16 + 256 w .. +256 of the table row
  // (entries past the row read its last entry), one dword DMA per lane.
  const int pg0 = k_lo / 16;
  auto issue_pids = [&](int w) {
    const int p = min(pg0 + w * kPidWindow + wv * 64 + lane, max_blocks - 1);
    dma4(bt + p, lds_offset(&lds.pid[w & 1][wv * 64]));
  };
  auto issue_half = [&](int t, const char* pool, uint4* dst) {
    const int kt = k_lo + t * KT;
    const int nk = min(KT, k_hi - kt);
    const int32_t* pw = &lds.pid[(t / TPW) & 1][(t * NKB) % kPidWindow];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int g = wv * LPW + i;
      const int page = g / LPP;
      uint4* d = dst + g * 64;
      if (nk >= 16 * page + KPL * (g % LPP) + KPL) {
        // all KPL keys of the load exist: the page's tile base is scalar,
        // the lane's row and chunk a fixed offset
        const int pid = __builtin_amdgcn_readfirstlane(min(max(pw[page], 0), num_pages - 1));
        dma16_sbase(pool + (static_cast<int64_t>(pid) * Hkv + kvh) * TILE, dma_off[i], lds_offset(d));
      } else {
        const int key = 16 * page + KPL * (g % LPP) + lane / NCHR;
        const int kc = min(key, nk - 1);
        const int pid = min(max(pw[kc >> 4], 0), num_pages - 1);
        const int64_t off = (static_cast<int64_t>(pid) * Hkv + kvh) * TILE + (kc & 15) * ROWB +
                            (((lane % NCHR) ^ swzf(key & 15)) * 16);
        dma16(pool + off, lds_offset(d));
      }
    }
  };
  // fp8: the K (wave 0) and V (wave 1) scales of tile t's keys, one dword
  // per lane (lane j: key j; keys past the tile's end take the last valid
  // key's scale, finite).
  auto issue_scales = [&](int t, int b) {
    if constexpr (FP8) {
      if (wv < 2) {
        const int kt = k_lo + t * KT;
        const int nk = min(KT, k_hi - kt);
        const int32_t* pw = &lds.pid[(t / TPW) & 1][(t * NKB) % kPidWindow];
        const int j = min(lane, nk - 1);
        const int pid = min(max(pw[j >> 4], 0), num_pages - 1);
        const int64_t at = (static_cast<int64_t>(pid) * Hkv + kvh) * 16 + (j & 15);
        dma4((wv == 0 ? k_scales : v_scales) + at, lds_offset(wv == 0 ? &lds.ks[b][0] : &lds.vs[b][0]));
      }
    }
  };
  // A whole tile: all of this wave's loads fall in one page (loads
  // LPW wv .. cover keys 16 page ..), so its id is read from LDS once for
  // the K and the V loads.  (Read per load, behind each DMA's memory
  // clobber, it cost an LDS round trip per load.)
  auto issue_tile = [&](int t, int b) {
    if (k_hi - (k_lo + t * KT) >= KT) {
      const int32_t* pw = &lds.pid[(t / TPW) & 1][(t * NKB) % kPidWindow];
      const int pid = min(max(__builtin_amdgcn_readfirstlane(pw[(wv * LPW) / LPP]), 0), num_pages - 1);
      const int64_t base = (static_cast<int64_t>(pid) * Hkv + kvh) * TILE;
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        dma16_sbase(kbytes + base, dma_off[i], lds_offset(lds.k[b] + (wv * LPW + i) * 64));
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        dma16_sbase(vbytes + base, dma_off[i], lds_offset(lds.v[b] + (wv * LPW + i) * 64));
    } else {
      issue_half(t, kbytes, lds.k[b]);
      issue_half(t, vbytes, lds.v[b]);
    }
    issue_scales(t, b);
  };
  // Per-lane row and chunk of the transposed V reads: lane (group lg, j)
  // reads row key0 + j/4, columns d0 + 4(j%4) .. +3, with key0 = 32 ks + 4 lg
  // (+16) and d0 = 16 db.
  const int tr_r = col >> 2;
  const int tr_c = col & 3;

  // S^T = K Q^T over the K tile in kb_lds: s[kb][rb] holds keys
  // 16 kb + 4 lg + i, query row 16 rb + col.  Each K operand serves both row
  // blocks.
  auto scores = [&](const uint4* kb_lds, f32x4 (&s)[NKB][2]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int key = kb * 16 + col;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) s[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u32x4 a;
        if constexpr (FP8) {
          // codes 32 c + 8 lg .. +7 of the key: half of swizzled chunk 2 c + lg / 2
          const int ch = (2 * c + (lg >> 1)) ^ fswz(key);
          const u32x2 w8 = *(__attribute__((address_space(3))) const u32x2*)(
              reinterpret_cast<const char*>(kb_lds) + key * ROWB + ch * 16 + (lg & 1) * 8);
          a = u32x4{fp8x2_to_bf16x2<false>(w8.x), fp8x2_to_bf16x2<true>(w8.x), fp8x2_to_bf16x2<false>(w8.y),
                    fp8x2_to_bf16x2<true>(w8.y)};
        } else {
          const int cc = c * 4 + lg;
          a = *(LdsU4*)(&kb_lds[key * 16 + (cc ^ tswz(col))]);
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) s[kb][rb] = mfma16x16x32(a, qb[rb][c], s[kb][rb]);
      }
    }
  };
  // fp8: each key's K scale (scale buffer sb) on its scores.
  auto scale_scores = [&](int sb, f32x4 (&s)[NKB][2]) {
    if constexpr (FP8) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4 k4 = *(__attribute__((address_space(3))) const f32x4*)(&lds.ks[sb][kb * 16 + 4 * lg]);
        const float kq[4] = {k4[0], k4[1], k4[2], k4[3]};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[kb][rb][i] *= kq[i];
      }
    }
  };
  // Keys are masked (by select) only in tiles that need it: the last,
  // partial tile of a split, and chunk tiles that cross the causal
  // diagonal of this wave's rows.
  auto mask_scores = [&](int kt, int nk, f32x4 (&s)[NKB][2]) {
    const bool need_mask = nk < KT || (CHUNK && kt + KT - 1 > vis_lo);
    if (need_mask) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kb * 16 + lg * 4 + i;
            const bool ok = key < nk && (!CHUNK || kt + key <= vis[rb]);
            s[kb][rb][i] = ok ? s[kb][rb][i] : -INFINITY;
          }
    }
  };
  // Online softmax per query row (column of S^T): the row's KT keys are
  // spread over this lane's 4 NKB values and the lanes l^16, l^32, l^48.
  // First the row maxima and the reference m.  Lazy rescaling:
  // probabilities are taken against the running reference m, which moves
  // (and o, the row sums are rescaled) only when a row's maximum exceeds it
  // by more than 2^8 -- so p <= 256, and the rescale, a wave-wide branch, is
  // rare after the first tiles.
  auto rescale = [&](const f32x4 (&s)[NKB][2]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float x = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x = fmaxf(x, s[kb][rb][i]);
      const float mx = max_xor32(max_xor16(x)) * scale_log2;  // scale > 0 keeps the order
      if (__ballot(mx > m[rb] + 8.f) != 0ull) {
        const float mn = fmaxf(m[rb], mx);
        // m = -inf (nothing visible yet): o and the sums are 0, any factor will do
        const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m[rb] - mn);
        m[rb] = mn;
        lsum[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][rb] *= alpha;
      }
    }
  };
  // Then the probabilities against m, rounded to bf16 into the P^T operand
  // (scale buffer sb: fp8 V scales), and their float32 row sums.
  auto probs = [&](const f32x4 (&s)[NKB][2], int sb, u32x4 (&pb)[NKS][2]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      // A row with no visible key so far keeps m = -inf: its p are all 0.
      const float nref = m[rb] == -INFINITY ? 0.f : -m[rb];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint32_t pw[2][2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(fmaf(s[2 * ks + e][rb][i], scale_log2, nref));
            lsum[rb] += p[i];
          }
          if constexpr (FP8) {
            // P^T carries p times the key's V scale (keys 32 ks + 16 e + 4 lg + i;
            // a masked key's p is 0 and its scale finite)
            const f32x4 v4 =
                *(__attribute__((address_space(3))) const f32x4*)(&lds.vs[sb][(2 * ks + e) * 16 + 4 * lg]);
            p[0] *= v4[0];
            p[1] *= v4[1];
            p[2] *= v4[2];
            p[3] *= v4[3];
          }
          pw[e][0] = bf16x2_rne(p[0], p[1]);
          pw[e][1] = bf16x2_rne(p[2], p[3]);
        }
        // k slots 8 lg .. 8 lg + 7 = keys 32 ks + 4 lg + [0, 4) and
        // 32 ks + 16 + 4 lg + [0, 4): the same order the V^T operand uses.
        pb[ks][rb] = u32x4{pw[0][0], pw[0][1], pw[1][0], pw[1][1]};
      }
    }
  };
  // O^T += V^T P^T over the V tile in vb_lds; the V^T operand (d = 16 db +
  // col, keys as above) comes from two transposed reads of 4 keys each and
  // serves both row blocks.
  auto accumulate = [&](const char* vb_lds, const u32x4 (&pb)[NKS][2]) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        u32x4 a;
        if constexpr (FP8) {
          // one transposed read of 8 rows: lanes 2 r, 2 r + 1 name row r of
          // the block, the keys in P^T's order
          const int r8 = col >> 1;
          const int row = ks * 32 + (r8 >> 2) * 16 + lg * 4 + (r8 & 3);
          const u32x2 w8 = lds_read_tr8(vb_lds + row * ROWB + (db ^ fswz(row)) * 16 + (col & 1) * 8);
          a = u32x4{fp8x2_to_bf16x2<false>(w8.x), fp8x2_to_bf16x2<true>(w8.x), fp8x2_to_bf16x2<false>(w8.y),
                    fp8x2_to_bf16x2<true>(w8.y)};
        } else {
          u32x2 part[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int row = ks * 32 + e * 16 + lg * 4 + tr_r;
            const int ch = (db * 2 + (tr_c >> 1)) ^ tswz(row & 15);
            part[e] = lds_read_tr16(vb_lds + row * (D * 2) + ch * 16 + (tr_c & 1) * 8);
          }
          a = u32x4{part[0].x, part[0].y, part[1].x, part[1].y};
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) o[db][rb] = mfma16x16x32(a, pb[ks][rb], o[db][rb]);
      }
    }
  };

  // The q rows and the first page-id window in one round trip, then (the
  // second window, if the range needs it, and) tiles 0 .. NB - 2 in flight
  // before the loop.
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = row0 + rb * 16 + col;
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
  issue_pids(0);
  // Wait for the q rows here, before any tile DMA is in flight: the
  // compiler does not see the (inline-assembly) DMAs, and left to itself it
  // would wait for q -- with vmcnt(0), draining the tile pipeline -- at the
  // first MFMA of every tile.
  asm volatile("" ::"v"(qb[0][0]), "v"(qb[0][1]), "v"(qb[0][2]), "v"(qb[0][3]), "v"(qb[1][0]), "v"(qb[1][1]),
               "v"(qb[1][2]), "v"(qb[1][3]));
  wait_vmcnt<0>();
  lds_barrier();
#pragma unroll
  for (int t = 0; t < NB - 1; ++t)
    if (t < nt) issue_tile(t, t);
  if (nt > TPW) issue_pids(1);

  int buf = 0;  // buffer of tile t
  for (int t = 0; t < nt; ++t) {
    const int kt = k_lo + t * KT;
    const int nk = min(KT, k_hi - kt);  // keys of this tile that exist
    // This wave's loads of tile t have landed once only the loads of the
    // tiles after it (at most NB - 2, 2 LPW loads each, plus any page-id
    // load issued after them) remain; after the barrier every wave's have,
    // and every wave is done with tile t - 1, whose buffer takes tile
    // t + NB - 1.
    const int ahead = min(NB - 2, nt - 1 - t);
    if constexpr (NB >= 4) {
      if (ahead >= 2) wait_vmcnt<4 * LPW>();
      else if (ahead == 1) wait_vmcnt<2 * LPW>();
      else wait_vmcnt<0>();
    } else if constexpr (NB == 3) {
      if (ahead >= 1) wait_vmcnt<2 * LPW>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    const int tn = t + NB - 1;
    if (tn < nt) {
      const int bn = buf == 0 ? NB - 1 : buf - 1;  // (tn % NB: the buffer tile t - 1 used)
      issue_tile(tn, bn);
      // The first tile of page-id window W has just been issued: load
      // window W + 1 into the buffer window W - 1 used (every tile of it was
      // issued before this iteration's barrier).
      if (tn % TPW == 0 && tn > 0 && tn + TPW < nt) issue_pids(tn / TPW + 1);
    }
    const int sbuf = buf;  // (fp8: the scale buffers of tile t)
    f32x4 s[NKB][2];
    scores(lds.k[buf], s);
    scale_scores(sbuf, s);
    mask_scores(kt, nk, s);
    rescale(s);
    u32x4 pb[NKS][2];  // P^T operand [32-key step ks][row block rb]
    probs(s, sbuf, pb);
    accumulate(reinterpret_cast<const char*>(lds.v[buf]), pb);
    buf = buf + 1 == NB ? 0 : buf + 1;
  }

  // Normalise and write this wave's rows: the row sums over all the keys of
  // the split (lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same row).
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float lt = add_xor32(add_xor16(lsum[rb]));
    const int r = row0 + rb * 16 + col;
    if (r < n_rows) {
      const int64_t pr = (tw.rec_base + (static_cast<int64_t>(r / G) * Hkv + kvh) * tw.nsplit + tw.ks) * G + r % G;
      const bool any = lt > 0.f;
      const float inv = any ? 1.0f / lt : 0.f;
      // (the row as bf16, rounded to nearest even: 256 bytes per partial)
      uint16_t* row = reinterpret_cast<uint16_t*>(pre_o) + pr * D + lg * 4;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *reinterpret_cast<uint2*>(row + db * 16) =
            make_uint2(bf16x2_rne(o[db][rb][0] * inv, o[db][rb][1] * inv), bf16x2_rne(o[db][rb][2] * inv, o[db][rb][3] * inv));
      if (lg == 0) pre_lse[pr] = any ? m[rb] + fast_log2(lt) : -INFINITY;
    }
  }
}

// Tile shape of the launches: PA_TILE_KEYS keys per tile, PA_TILE_BUFS buffers.
#ifndef PA_TILE_KEYS
#define PA_TILE_KEYS 64
#endif
#ifndef PA_TILE_BUFS
#define PA_TILE_BUFS 2
#endif
constexpr int kTK = PA_TILE_KEYS;
constexpr int kTB = PA_TILE_BUFS;

// FP8: pools of e4m3fn codes with their row scales (built for the shared
// prefix, whose tiles hold 64 keys).
template <int G, bool CHUNK, bool FP8 = false>
__global__ __launch_bounds__(kTileThreads, FP8 ? kTileFp8WorkgroupsPerCU : kTileWorkgroupsPerCU) void tile_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ group_off, const int32_t* __restrict__ prefix_lens,
    ChunkList chunks, int RC, int nks, int kps, int Hkv, int n_items, int num_pages, float scale_log2,
    int32_t* __restrict__ begin_pages, float* __restrict__ pre_o, float* __restrict__ pre_lse,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales) {
  __shared__ TileLds<kTK, kTB, FP8> lds;
  TileWork tw;
  if (!tile_work<G, CHUNK>(blockIdx.x, RC, n_items, Hkv, nks, kps, chunks, ctx, cu_q, group_off, prefix_lens,
                           begin_pages, tw))
    return;  // uniform over the workgroup
  tile_body<G, CHUNK, kTK, kTB, FP8>(tw, lds, q, k_pool, v_pool, block_tables, max_blocks, Hkv, num_pages, scale_log2,
                                     pre_o, pre_lse, k_scales, v_scales);
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
  // Split j of head h: record p0 + G j + h (the G heads of a split are
  // consecutive records).
  const int64_t p0 = (chunks.rec[u] + (static_cast<int64_t>(i) * Hkv + kvh) * nks) * G;
  auto lse_at = [&](int j, int h) -> float { return pre_lse[p0 + static_cast<int64_t>(j) * G + h]; };
  auto load_row = [&](int j, int h, float (&v)[2]) {
    load_bf16_pair(reinterpret_cast<const uint16_t*>(pre_o) + (p0 + static_cast<int64_t>(j) * G + h) * D, lane, v);
  };
  float M[G], wsum[G], acc[G][2];
  merge_init<G, D>(M, wsum, acc);
  merge_partials<G, D>(nsp, lse_at, load_row, M, wsum, acc);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float inv = 1.0f / wsum[h];
    const int64_t row = static_cast<int64_t>(cu_q[s] + i) * Hq + kvh * G + h;
    reinterpret_cast<uint32_t*>(out)[row * (D / 2) + lane] = bf16x2_rne(acc[h][0] * inv, acc[h][1] * inv);
    if (lse_out && lane == 0) lse_out[row] = (M[h] + fast_log2(wsum[h])) * kLn2;
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
  // The prefix splits (bf16 rows), then the suffix: one whole-sequence
  // partial (seq_part, a bf16 row) or one per wave that shared the sequence
  // (float32 rows), merged in that order, each kind in a pass of its own.
  static_assert(EPL == 2, "rows of 128 elements");
  float M[G], wsum[G], acc[G][EPL];
  merge_init<G, D>(M, wsum, acc);
  const int64_t pre0 = (static_cast<int64_t>(s) * Hkv + kvh) * nks * G;  // split 0, head 0
  merge_partials<G, D>(
      np, [&](int j, int h) { return pre_lse[pre0 + static_cast<int64_t>(j) * G + h]; },
      [&](int j, int h, float (&v)[EPL]) {
        load_bf16_pair(reinterpret_cast<const uint16_t*>(pre_o) + (pre0 + static_cast<int64_t>(j) * G + h) * D, lane, v);
      },
      M, wsum, acc);
  if (!shared) {
    const int64_t r0 = static_cast<int64_t>(s) * Hq + kvh * G;
    merge_partials<G, D>(
        1, [&](int, int h) { return seq_part[static_cast<int64_t>(S) * Hq * D + r0 + h]; },
        [&](int, int h, float (&v)[EPL]) {
          load_bf16_pair(reinterpret_cast<const uint16_t*>(seq_part) + (r0 + h) * D, lane, v);
        },
        M, wsum, acc);
  } else {
    auto rec = [&](int k, int h) -> int64_t {
      return ((static_cast<int64_t>(w0 + k) * Hkv + kvh) * 2 + (k == 0 ? slot0 : 0)) * PR + h;
    };
    merge_partials<G, D>(
        ns, [&](int k, int h) { return part_lse[rec(k, h)]; },
        [&](int k, int h, float (&v)[EPL]) {
          const float* src = part_o + rec(k, h) * D + lane * EPL;
          v[0] = src[0];
          v[1] = src[1];
        },
        M, wsum, acc);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float inv = 1.0f / wsum[h];
    const int64_t row = static_cast<int64_t>(s) * Hq + kvh * G + h;
    if constexpr (sizeof(T) == 2) {
      if constexpr (EPL == 2) {
        reinterpret_cast<uint32_t*>(out)[row * (D / 2) + lane] = bf16x2_rne(acc[h][0] * inv, acc[h][1] * inv);
      } else {
        reinterpret_cast<uint16_t*>(out)[row * D + lane] = static_cast<uint16_t>(bf16_bits_rne(acc[h][0] * inv));
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) reinterpret_cast<float*>(out)[row * D + lane * EPL + e] = acc[h][e] * inv;
    }
    if (lse_out && lane == 0) lse_out[row] = (M[h] + fast_log2(wsum[h])) * kLn2;
  }
}

// Decode runs of the one-launch mixed kernel: the runs of a plain decode
// launch (4 matrix-core stream waves per CU) times PA_MIXED_RUNS_PER_WAVE
// (bf16 pools) or PA_MIXED_RUNS_PER_WAVE_FP8.  (With the chunk splits
// planned for one chunk workgroup per CU, 3 runs per wave measured 850-859
// against 864-869 us at 2 and 871-873 us at 4.)
#ifndef PA_MIXED_RUNS_PER_WAVE
#define PA_MIXED_RUNS_PER_WAVE 3
#endif
#ifndef PA_MIXED_RUNS_PER_WAVE_FP8
#define PA_MIXED_RUNS_PER_WAVE_FP8 3
#endif
// Decode workgroups per chunk workgroup in the dispatch order (bf16, fp8
// pools: an fp8 decode run streams half the bytes of a bf16 one).
#ifndef PA_MIXED_DECODE_PER_CHUNK
#define PA_MIXED_DECODE_PER_CHUNK 3
#endif
#ifndef PA_MIXED_DECODE_PER_CHUNK_FP8
#define PA_MIXED_DECODE_PER_CHUNK_FP8 5
#endif
// Keys per tile of the mixed kernel's chunk workgroups (two buffers; 64
// keys, 66 KB, fit inside a decode workgroup's 80 KB of LDS).
#ifndef PA_MIXED_TILE_KEYS
#define PA_MIXED_TILE_KEYS 64
#endif
// Build switch: 0 runs every mixed batch as the chunk launch(es), then the
// decode stream (for measuring the one-launch kernel against them).
#ifndef PA_MIXED_ONE_LAUNCH
#define PA_MIXED_ONE_LAUNCH 1
#endif
// Stream waves (runs) per decode workgroup, each with its own LDS.
#ifndef PA_MIXED_DECODE_WAVES
#define PA_MIXED_DECODE_WAVES 2
#endif
constexpr int kMixDecodeWaves = PA_MIXED_DECODE_WAVES;
static_assert(kMixDecodeWaves >= 1 && kMixDecodeWaves <= 4, "decode waves per workgroup");
constexpr int kMixTK = PA_MIXED_TILE_KEYS;

// Prefill chunks and decode tokens of a mixed batch in one launch (SwiftLLM
// page, section 3.3: decode tokens piggybacked on a prefill chunk, so that
// the chunk's matrix work and the decode's HBM streaming run at the same
// time).  A workgroup of 4 waves is either a chunk workgroup (tile_body with
// tiles of kMixTK keys, 64 over fp8 pools: 128 (token, q-head) rows against
// one key split of one kv-head) or a decode workgroup whose first
// kMixDecodeWaves waves each stream one decode run with LDS of their own
// (stream_mfma_body; the other waves end at once): 80 KB (bf16) or 50 KB
// (fp8), so that two decode workgroups on a CU -- the chunk body's registers
// let two workgroups share one -- stream with four waves, as a plain decode
// launch does.  Along each XCD's dispatch order one chunk workgroup comes
// before every `ratio` decode workgroups while both kinds remain.  Decode segments
// find their pages themselves (a walk over the segments with one query
// token, cu_q); the merges of both run as launches after this one.
// (The same pairing for a cascade's prefix tiles and suffix stream measured
// slower than the separate launches on the shared-prefix batch, whose prefix
// work is small next to its suffix stream: 313 against 304 us with one
// stream wave per suffix workgroup; 320 us for the kernel alone against a
// 299 us step with two, one suffix workgroup per CU and each member's first
// suffix page written by a set-up kernel beforehand.)
struct PairGrid {
  int ncw;   // chunk workgroups (a multiple of 8, as tile_work numbers them)
  int ndw;   // decode workgroups (a multiple of 8): kMixDecodeWaves runs each
  int runs;  // decode runs: runs per kv-head x kv-heads
  int W;     // decode runs per kv-head
};

// Chunk-side arguments.
struct PairTiles {
  int RC, n_items;
  const int32_t* cu_q;  // the batch's cumulative query counts
  float* pre_o;
  float* pre_lse;
};

template <int G, bool FP8>
__global__ __launch_bounds__(kTileThreads, 2) void mixed_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ ctx, ChunkList chunks,
    PairTiles tiles, int Hkv, int num_pages, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse_out, int S, int per, int total_pages, int32_t* __restrict__ seq_info,
    float* __restrict__ part_o, float* __restrict__ part_lse, PairGrid grid) {
  // fp8 pools: code tiles of 64 keys (35 KB with their scales), the fp8
  // stream wave (25 KB)
  using TKV = typename std::conditional<FP8, uint8_t, uint16_t>::type;
  constexpr int CKT = FP8 ? 64 : kMixTK;
  using WaveLds = StreamMfmaLds<TKV, 128>;
  using ChunkLds = TileLds<CKT, 2, FP8>;
  constexpr size_t kWaveBytes = kMixDecodeWaves * sizeof(WaveLds);
  constexpr size_t kBytes = sizeof(ChunkLds) > kWaveBytes ? sizeof(ChunkLds) : kWaveBytes;
  __shared__ __align__(16) unsigned char raw[kBytes];
  // Workgroup -> kind and index along XCD x's dispatch order: cycles of one
  // chunk workgroup and `ratio` decode workgroups while both kinds
  // remain, then the remaining decode workgroups, then the remaining chunk
  // workgroups.
  const int x = blockIdx.x & 7;
  const int j = blockIdx.x >> 3;
  const int nc = grid.ncw >> 3, nd = grid.ndw >> 3;
  constexpr int ratio = FP8 ? PA_MIXED_DECODE_PER_CHUNK_FP8 : PA_MIXED_DECODE_PER_CHUNK;
  const int full = nc < nd / ratio ? nc : nd / ratio;
  bool chunk;
  int idx;
  if (j < (1 + ratio) * full) {
    const int k = j / (1 + ratio), r = j % (1 + ratio);
    chunk = r == 0;
    idx = chunk ? k : k * ratio + r - 1;
  } else {
    const int j2 = j - (1 + ratio) * full;
    const int left_d = nd - ratio * full;
    chunk = j2 >= left_d;
    idx = chunk ? full + j2 - left_d : ratio * full + j2;
  }
  if (chunk) {
    TileWork tw;
    if (!tile_work<G, true>(idx * 8 + x, tiles.RC, tiles.n_items, Hkv, 0, 0, chunks, ctx, tiles.cu_q, nullptr,
                            nullptr, nullptr, tw))
      return;  // uniform over the workgroup
    tile_body<G, true, CKT, 2, FP8>(tw, *reinterpret_cast<ChunkLds*>(raw), q, k_pool, v_pool, block_tables,
                                    max_blocks, Hkv, num_pages, scale_log2, tiles.pre_o, tiles.pre_lse, k_scales,
                                    v_scales);
  } else {
    const int wv = threadIdx.x >> 6;
    const int r = (idx * 8 + x) * kMixDecodeWaves + wv;
    if (wv >= kMixDecodeWaves || r >= grid.runs) return;
    const Fold fold{1, G, __builtin_ctz(G), 0, 1, 0};
    stream_mfma_body<TKV, 128, false>(*reinterpret_cast<WaveLds*>(raw + wv * sizeof(WaveLds)), r % grid.W, r / grid.W,
                                      out, lse_out, q,
                                      static_cast<const TKV*>(k_pool), static_cast<const TKV*>(v_pool), k_scales,
                                      v_scales, block_tables, ctx, max_blocks, S, Hkv, num_pages, scale_log2, per,
                                      /*lead=*/0, total_pages, seq_info, part_o, part_lse, PageSkip{}, nullptr, tiles.cu_q, fold);
  }
}

// Decode runs of a mixed launch over `pages` pages per kv-head.
struct PairPlan {
  int64_t per, W;
};
PairPlan pair_plan(int64_t pages, int32_t num_kv_heads, bool kv_fp8) {
  const int cus = device_cu_count();
  const int64_t target = static_cast<int64_t>(4) * (kv_fp8 ? PA_MIXED_RUNS_PER_WAVE_FP8 : PA_MIXED_RUNS_PER_WAVE) *
                         (cus > 0 ? cus : 256);
  const int64_t per_head = std::max<int64_t>(1, std::min<int64_t>(target, kMaxResidentWaves) / num_kv_heads);
  PairPlan p;
  p.per = std::max<int64_t>(kMinPagesPerWave, (pages + per_head - 1) / per_head);
  p.W = std::max<int64_t>(1, (pages + p.per - 1) / p.per);
  return p;
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
  ChunkList none;
  none.n = 0;
  const int n_items = c.num_groups * a.num_kv_heads * c.nks;
  profile_before(a.stream);
  const unsigned blocks = static_cast<unsigned>((n_items + 7) / 8 * 8 * c.row_chunks);
  if (a.kv_fp8)
    hipLaunchKernelGGL((tile_kernel<G, false, true>), dim3(blocks), dim3(kTileThreads), 0, st,
                       static_cast<const uint16_t*>(a.q), a.k_pool, a.v_pool, a.block_tables, a.max_blocks,
                       a.context_lens, nullptr, c.group_offsets, c.prefix_lens, none, c.row_chunks, c.nks, c.kps,
                       a.num_kv_heads, n_items, static_cast<int>(a.num_pages), scale_log2, begin_pages, pre_o,
                       pre_lse, a.k_scales, a.v_scales);
  else
    hipLaunchKernelGGL((tile_kernel<G, false, false>), dim3(blocks), dim3(kTileThreads), 0, st,
                       static_cast<const uint16_t*>(a.q), a.k_pool, a.v_pool, a.block_tables, a.max_blocks,
                       a.context_lens, nullptr, c.group_offsets, c.prefix_lens, none, c.row_chunks, c.nks, c.kps,
                       a.num_kv_heads, n_items, static_cast<int>(a.num_pages), scale_log2, begin_pages, pre_o,
                       pre_lse, nullptr, nullptr);
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
  float* pre_o = reinterpret_cast<float*>(ws + L.pre_o_offset);
  float* pre_lse = reinterpret_cast<float*>(ws + L.pre_lse_offset);
  char* sws = ws + L.stream_offset;
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
  // One launch for chunks and decode tokens when the decode tokens run on
  // the matrix-core stream wave (4 or more q-heads per kv-head) and the
  // chunks fit one chunk list; otherwise the chunk tiles, then the decode
  // stream, one after the other.
  const bool one = PA_MIXED_ONE_LAUNCH && G >= 4 && mx.decode_pages > 0 && mx.num_chunks <= kMaxChunkSegments;
  if (one) {
    const ChunkList cl = chunk_list(0);
    const int n_items = cl.item_end[cl.n - 1];
    const PairPlan pp = pair_plan(mx.decode_pages, a.num_kv_heads, a.kv_fp8);
    const PartialLayout pl = partial_layout(pp.W, a.num_seqs, a.num_kv_heads, 16, 128);
    if (pl.bytes > mx.workspace_bytes - L.stream_offset)
      return fail(PA_EWORKSPACE, "pa_mixed_chunk: workspace too small for the decode plan");
    PairGrid grid;
    grid.W = static_cast<int>(pp.W);
    grid.runs = static_cast<int>(pp.W * a.num_kv_heads);
    grid.ndw = ((grid.runs + kMixDecodeWaves - 1) / kMixDecodeWaves + 7) / 8 * 8;  // kMixDecodeWaves runs each
    grid.ncw = (n_items + 7) / 8 * 8 * mx.row_chunks;
    PairTiles tiles{};
    tiles.RC = mx.row_chunks;
    tiles.n_items = n_items;
    tiles.cu_q = mx.cu_q_lens;
    tiles.pre_o = pre_o;
    tiles.pre_lse = pre_lse;
    profile_before(a.stream);
    const unsigned blocks = static_cast<unsigned>(grid.ncw + grid.ndw);
    auto launch = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kTileThreads), 0, st, static_cast<const uint16_t*>(a.q),
                         a.k_pool, a.v_pool, a.k_scales, a.v_scales, a.block_tables, a.max_blocks, a.context_lens, cl,
                         tiles, a.num_kv_heads, static_cast<int>(a.num_pages), scale_log2,
                         static_cast<uint16_t*>(a.out), a.lse_out, a.num_seqs, static_cast<int>(pp.per),
                         static_cast<int>(mx.decode_pages), reinterpret_cast<int32_t*>(sws + pl.info_offset),
                         reinterpret_cast<float*>(sws + pl.o_offset), reinterpret_cast<float*>(sws + pl.lse_offset),
                         grid);
    };
    if (a.kv_fp8)
      launch(mixed_kernel<G, true>);
    else
      launch(mixed_kernel<G, false>);
    profile_after(a.stream);
    if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_mixed_chunk: mixed kernel launch failed");
    DecodeLaunch dec = a;
    dec.workspace = sws;
    dec.workspace_bytes = mx.workspace_bytes - L.stream_offset;
    dec.total_pages = mx.decode_pages;
    const int rc = launch_stream_merge(dec, mx.cu_q_lens, pp.W);
    if (rc) return rc;
  } else {
    if (mx.num_chunks > 0) {
      profile_before(a.stream);
      for (int b0 = 0; b0 < mx.num_chunks; b0 += kMaxChunkSegments) {
        const ChunkList cl = chunk_list(b0);
        const int n_items = cl.item_end[cl.n - 1];
        const unsigned blocks = static_cast<unsigned>((n_items + 7) / 8 * 8 * mx.row_chunks);
        auto launch = [&](auto kernel) {
          hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kTileThreads), 0, st, static_cast<const uint16_t*>(a.q),
                             a.k_pool, a.v_pool, a.block_tables, a.max_blocks, a.context_lens, mx.cu_q_lens, nullptr,
                             nullptr, cl, mx.row_chunks, 0, 0, a.num_kv_heads, n_items,
                             static_cast<int>(a.num_pages), scale_log2, nullptr, pre_o, pre_lse, a.k_scales,
                             a.v_scales);
        };
        if (a.kv_fp8)
          launch(tile_kernel<G, true, true>);
        else
          launch(tile_kernel<G, true, false>);
        if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_mixed_chunk: chunk kernel launch failed");
      }
      profile_after(a.stream);
    }
    if (mx.decode_pages > 0) {
      DecodeLaunch dec = a;
      dec.workspace = sws;
      dec.workspace_bytes = mx.workspace_bytes - L.stream_offset;
      dec.total_pages = mx.decode_pages;
      // (the walk skips the chunks' segments: q_rows is the batch's cu_q_lens)
      const int rc = launch_stream(dec, nullptr, nullptr, mx.cu_q_lens, /*merge=*/true, nullptr);
      if (rc) return rc;
    }
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
