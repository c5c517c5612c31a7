// Device code shared by the stream (decode) kernels and the mixed-batch
// kernel: the stream-K page walk of one wave's run, and the matrix-core
// stream wave (stream_mfma_body).  The work split and the per-batch
// pipeline are described in pa_decode.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_common.h"

namespace pa {

template <typename T, int D>
struct Geom {
  static constexpr int EB = sizeof(T);        // element bytes
  static constexpr int RD = D * EB / 4;       // dwords per row
  static constexpr int NCH = RD / 4;          // 16-byte chunks per row
  static constexpr int TILE = 16 * RD * 4;    // bytes of one (page, kv-head) tile
  static constexpr int NI = 4 * TILE / 1024;  // 1 KB loads per 4-page batch (K and V each)
  static constexpr int RPI = 64 / NCH;        // rows one 1 KB load covers
  static constexpr int EPC = 16 / EB;         // elements per 16-byte chunk
  static_assert(RD == 32 || RD == 64, "row must be 128 or 256 bytes");
  static_assert(NI * RPI == 64, "a batch is 64 rows");
  // XOR applied to the chunk index of row r in the K buffer, so that the
  // transposed read (lane r takes row r) of the 16 lanes the 64-bank LDS
  // serves at once touches 16 different 16-byte bank groups: rows of 256
  // bytes use r mod 16; rows of 128 bytes pair up rows r, r+1 (they sit 8
  // groups apart) and use (r / 2) mod 8.
  static __device__ __forceinline__ int swz(int r) { return NCH == 16 ? (r & 15) : ((r >> 1) & 7); }
};

// One batch: rows [16*pb, 16*pb + 64) of sequence s, pages clamped to the
// segment [.., seg_hi) this wave covers.
struct Batch {
  int s;       // sequence
  int L;       // its context length
  int P;       // its page count
  int pb;      // first page of the batch
  int B;       // first page of the sequence the walk covers at all (cascade: after the shared prefix)
  int seg_lo;  // first page of the sequence this wave covers
  int seg_hi;  // one past the last page this wave covers
  int cs;      // flattened index of the sequence's first page
  int qb;      // q buffer holding the sequence's q rows
  int lo;      // first row the query sees (sliding window; else 0)
  int pid[4];  // physical pages (entries past seg_hi repeat the last one)
};

// Runs of a kv-head's flattened pages: waves 2j and 2j + 1 share 2 per
// pages, the even one taking per + lead of them (lead = 0: equal runs).
// With an even number of waves per kv-head in the grid's x extent, a
// wave's parity is that of its workgroup index, and so of its XCD.
__device__ __forceinline__ int run_begin(int w, int per, int lead) { return w * per + ((w & 1) ? lead : 0); }
// The wave whose run holds flattened page `page`.
__device__ __forceinline__ int run_wave(int page, int per, int lead) {
  const int j = page / (2 * per);
  return 2 * j + (page - 2 * j * per >= per + lead ? 1 : 0);
}

__device__ __forceinline__ int pages_of_len(int L, int max_blocks) {
  const int64_t pg = (static_cast<int64_t>(L) + 15) >> 4;
  return static_cast<int>(pg < max_blocks ? (pg > 0 ? pg : 0) : max_blocks);
}

__device__ __forceinline__ void load_pids(const int32_t* __restrict__ block_tables, int max_blocks, int num_pages,
                                          Batch& b) {
  const int32_t* bt = block_tables + static_cast<int64_t>(b.s) * max_blocks;
  if (b.pb + 4 <= b.seg_hi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) b.pid[i] = bt[b.pb + i];
  } else {
    b.pid[0] = bt[b.pb];
#pragma unroll
    for (int i = 1; i < 4; ++i) b.pid[i] = (b.pb + i < b.seg_hi) ? bt[b.pb + i] : b.pid[i - 1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) b.pid[i] = min(max(b.pid[i], 0), num_pages - 1);
}

// The workgroup is one wave, whose LDS accesses execute in order: sharing
// values between lanes through LDS needs no barrier, only that the compiler
// keep the accesses in program order.  (__syncthreads() would also wait for
// every outstanding global load, draining the K/V prefetch.)  LDS DMA
// (global_load_lds) is waited for by vmcnt explicitly.
__device__ __forceinline__ void lds_order() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// The page walk of one wave's run [run_a, run_b) of a kv-head's flattened
// pages: the batch the run starts with, and the batch after each batch.
// `trim` rows are taken off the end of every context (a multi-token pass
// that stops before a sequence's last new tokens).
struct Walk {
  const int32_t* __restrict__ ctx;
  PageSkip skip;
  const int32_t* __restrict__ cu_q;  // mixed batch: cumulative query counts (chunks hold no pages of the walk)
  const int32_t* __restrict__ block_tables;
  int S, max_blocks, num_pages, trim, run_b;

  __device__ int first_page(int s, int L, int P) const {
    return min(max(walk_begin(skip, cu_q, s, L), 0), P);
  }
  // First row a sequence's query sees: 0, or the start of the sliding window.
  __device__ int first_row(int L) const { return skip.window > 0 && L > skip.window ? L - skip.window : 0; }

  // The run's first batch (qb = 0); false if the run holds no page.
  __device__ bool start(int run_a, Batch& b) const {
    ItemLoc loc;
    // (Cascade suffix: only the pages after each prefix are laid end to end.)
    if (!locate_item(ctx, skip, cu_q, S, max_blocks, 1, run_a, loc, trim)) return false;
    b.s = __builtin_amdgcn_readfirstlane(loc.s);
    b.L = ctx[b.s] - trim;
    b.P = pages_of_len(b.L, max_blocks);
    b.B = first_page(b.s, b.L, b.P);
    b.lo = first_row(b.L);
    b.cs = __builtin_amdgcn_readfirstlane(loc.base);
    b.seg_lo = b.B + (run_a - b.cs);
    b.seg_hi = min(b.P, b.B + (run_b - b.cs));
    b.pb = b.seg_lo;
    b.qb = 0;
    load_pids(block_tables, max_blocks, num_pages, b);
    return true;
  }

  // The batch after x (same sequence, or the next one holding pages of
  // this run); false if the run ends with x.
  __device__ bool advance(const Batch& x, Batch& y) const {
    y = x;
    if (x.pb + 4 < x.seg_hi) {
      y.pb = x.pb + 4;
    } else if (x.cs + (x.P - x.B) < run_b && x.s + 1 < S) {
      y.s = x.s + 1;
      y.cs = x.cs + (x.P - x.B);
      y.L = ctx[y.s] - trim;
      y.P = pages_of_len(y.L, max_blocks);
      y.B = first_page(y.s, y.L, y.P);
      // Sequences with nothing after begin_pages (the prefill chunks of a
      // mixed batch) hold no pages of the walk: step over them.  Pages of
      // this run remain, so a sequence that holds some follows.
      while (y.B >= y.P && y.s + 1 < S) {
        y.s += 1;
        y.L = ctx[y.s] - trim;
        y.P = pages_of_len(y.L, max_blocks);
        y.B = first_page(y.s, y.L, y.P);
      }
      y.lo = first_row(y.L);
      y.seg_lo = y.B;
      y.seg_hi = min(y.P, y.B + (run_b - y.cs));
      y.pb = y.B;
      y.qb = x.qb ^ 1;
      if (y.seg_hi <= y.seg_lo) return false;
    } else {
      return false;
    }
    load_pids(block_tables, max_blocks, num_pages, y);
    return true;
  }
};

// Which query rows a wave holds.  Multi-token pass: tokens tok0 ..
// tok0+fe-1 of every sequence's n new tokens (q / out rows s*n .. s*n+n-1;
// token i sits at position L - n + i), folded into the wave's rows: row r
// = token r >> lg, head r & (g-1).  One token per sequence: n = fe = 1,
// tok0 = 0, and row r is q-head r of the kv-head.  Rows of tokens past fe
// (past g heads) are idle.
struct Fold {
  int n;     // new tokens per sequence
  int g;     // q-heads per kv-head (a power of two)
  int lg;    // log2(g)
  int tok0;  // first token of the pass
  int fe;    // tokens in the pass
  int trim;  // n - tok0 - fe: context rows after the pass's last token
  int win = 0;  // sliding window in tokens (0: none): token j of the pass sees
                // only the win rows up to its own position; the walk then
                // starts at the pass's earliest token's window
};

// LDS of one matrix-core stream wave: the batch's K and V (64 rows,
// swizzled), two sequences' q rows (16 rows each) and, for fp8 pools, two
// batches' K and V row scales.  bf16 pools take 40 KB at D = 128.
template <typename TKV, int D, bool FP8 = sizeof(TKV) == 1>
struct StreamMfmaLds {
  uint4 k[64 * Geom<TKV, D>::NCH];
  uint4 v[64 * Geom<TKV, D>::NCH];
  uint4 q[2][2 * D];  // 16 rows x D/8 chunks of 16 bytes
  float4 ks[2][16];
  float4 vs[2][16];
};
template <typename TKV, int D>
struct StreamMfmaLds<TKV, D, false> {
  uint4 k[64 * Geom<TKV, D>::NCH];
  uint4 v[64 * Geom<TKV, D>::NCH];
  uint4 q[2][2 * D];
};
// The K (or V) scales of batch rows 4 i .. 4 i + 3 in scale buffer sb
// (fp8 pools); 1 otherwise.
template <bool FP8, typename L>
__device__ __forceinline__ float4 row_scales(const L& lds, bool k, int sb, int i) {
  if constexpr (FP8)
    return k ? lds.ks[sb][i] : lds.vs[sb][i];
  else
    return make_float4(1.f, 1.f, 1.f, 1.f);
}

// The stream kernel for waves that hold 16 query rows (16 q-heads per
// kv-head, or a multi-token pass's folded (token, head) rows), on the
// matrix cores.  Same work split, page walk, K/V/q DMA pipeline, partials
// and merge as stream_decode_kernel; per 64-row batch:
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: the A operand is a K tile
//    (16 rows, 32 columns) read from the swizzled K buffer, the B operand a
//    q tile; lane l ends up with query row l % 16 against the batch rows
//    16 kb + 4 (l / 16) + i (kb, i = 0..3).
//  * Online softmax per query row: a lane's 16 scores, then the lanes
//    l ^ 16 and l ^ 32 that hold the same row.  The probabilities stay in
//    registers as the P^T operand (bf16 pairs, rounded to nearest even);
//    the normaliser sums the float32 values, as the other decode paths do.
//  * O^T += V^T P^T: V lands in LDS swizzled like K and is read transposed
//    (ds_read_b64_tr_b16), its rows in the same order as P^T's; lane l
//    accumulates row l % 16, columns 16 db + 4 (l / 16) + i.
// Each wave's matrix work per batch is 32 MFMAs where the vector path
// needs about 2000 dot2 instructions for 16 rows.
// fp8 pools (TKV = uint8_t, e4m3fn codes with a float32 scale per row):
// K operands come from 8-byte reads of the codes widened to bf16 pairs
// (exact), V^T operands from ds_read_b64_tr_b8 (lane j of a 16-lane group
// passes row j/2, bytes 8 (j % 2) .. +7 of an 8 x 16-byte block and
// receives column j, rows 0..7), widened the same way; the K scale of a row
// multiplies its scores, its V scale the probability P^T carries (the
// normaliser sums the plain probabilities), as in the vector fp8 path.
// The body takes its LDS and its (run, kv-head) as arguments, so that the
// one-wave stream_mfma_kernel and the mixed-batch kernel (several waves
// per workgroup, each with its own LDS part) both run it.
template <typename TKV, int D, bool MT>
__device__ __forceinline__ void stream_mfma_body(
    StreamMfmaLds<TKV, D>& lds, int w, int kvh, uint16_t* __restrict__ out, float* __restrict__ lse_out, const uint16_t* __restrict__ q,
    const TKV* __restrict__ k_pool, const TKV* __restrict__ v_pool, const float* __restrict__ k_scales,
    const float* __restrict__ v_scales, const int32_t* __restrict__ block_tables, const int32_t* __restrict__ ctx,
    int max_blocks, int S, int Hkv, int num_pages, float scale_log2, int per, int lead, int total_pages,
    int32_t* __restrict__ seq_info, float* __restrict__ part_o, float* __restrict__ part_lse,
    PageSkip skip, float* __restrict__ seq_part, const int32_t* __restrict__ q_rows, Fold fold) {
  using Gm = Geom<TKV, D>;
  constexpr bool FP8 = sizeof(TKV) == 1;
  constexpr int R = 16;  // query rows
  constexpr int RD = Gm::RD, NCH = Gm::NCH, TILE = Gm::TILE, NI = Gm::NI;
  constexpr int NK = NI + (FP8 ? 2 : 0), NV = NI;  // loads of one issue_k (+ the K and V scales) / issue_v
  constexpr int QNCH = D / 8;                      // 16-byte chunks of one bf16 q row
  constexpr int QPL = R * QNCH / 64;
  constexpr int KC = D / 32;  // 32-column steps of the scores
  constexpr int DB = D / 16;  // 16-column blocks of the output
  constexpr int per_tile = TILE / 1024;
  static_assert(NV + NK <= 63, "vmcnt counts at most 63 loads");
  static_assert(sizeof(lds.k) == sizeof(uint4) * 64 * NCH && sizeof(lds.q[0]) == sizeof(uint4) * QPL * 64,
                "LDS layout");
  uint4* k_lds = lds.k;
  uint4* v_lds = lds.v;
  auto& q_lds = lds.q;

  const int lane = lane_id();
  const int col = lane & 15;  // query row of this lane (C/D column; B column)
  const int lg = lane >> 4;   // k group of the operands; row group of C/D
  const int GH = fold.g;  // q-heads per kv-head (8 or 16; fewer when tokens are folded)
  const int Hq = Hkv * GH;
  const int trim = MT ? fold.trim : 0;
  const char* kbytes = reinterpret_cast<const char*>(k_pool);
  const char* vbytes = reinterpret_cast<const char*>(v_pool);

  const int run_a = run_begin(w, per, lead);
  const int run_b = min(run_begin(w + 1, per, lead), total_pages);
  if (run_a >= run_b) return;

  // K and V both land swizzled: instruction i of a page tile fills LDS
  // slots 64i..64i+63 of its rows, slot -> (row, chunk ^ swz(row)).
  uint32_t koff[per_tile];
#pragma unroll
  for (int r = 0; r < per_tile; ++r) {
    const int slot = r * 64 + lane;
    const int row = slot / NCH;
    const int ch = (slot % NCH) ^ Gm::swz(row);
    koff[r] = row * (RD * 4) + ch * 16;
  }

  const Walk walk{ctx, skip, q_rows, block_tables, S, max_blocks, num_pages, trim, run_b};
  Batch first;
  if (!walk.start(run_a, first)) return;
  const int s0 = first.s;

  const uint32_t k_base = lds_offset(k_lds);
  const uint32_t v_base = lds_offset(v_lds);
  auto issue_tiles = [&](const char* pool, const Batch& b, uint32_t base) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const char* tile = pool + (static_cast<int64_t>(b.pid[i / per_tile]) * Hkv + kvh) * TILE;
      dma16(tile + koff[i % per_tile], base + i * 1024);
    }
  };
  // fp8: lane r fetches the scales of batch row r (page r / 16, slot r % 16)
  // into scale buffer sb, with the batch's K.
  auto issue_k = [&](const Batch& b, int sb) {
    issue_tiles(kbytes, b, k_base);
    if constexpr (FP8) {
      // (values first: a select over the array itself would keep the batch
      // in scratch memory)
      const int p0 = b.pid[0], p1 = b.pid[1], p2 = b.pid[2], p3 = b.pid[3];
      const int pl = lane < 32 ? (lane < 16 ? p0 : p1) : (lane < 48 ? p2 : p3);
      const int64_t at = (static_cast<int64_t>(pl) * Hkv + kvh) * 16 + (lane & 15);
      dma4(k_scales + at, lds_offset(&lds.ks[sb][0]));
      dma4(v_scales + at, lds_offset(&lds.vs[sb][0]));
    }
  };

  // Row r of the wave: q-head r of the kv-head, or (MT) token tok0 + (r >>
  // lg) and head r & (g-1); idle rows repeat the last active row.
  auto qrow = [&](int s) -> int64_t { return q_rows ? q_rows[s] : s; };
  auto row_index = [&](int s, int r) -> int64_t {
    if constexpr (MT)
      return (static_cast<int64_t>(s) * fold.n + fold.tok0 + (r >> fold.lg)) * Hq + kvh * GH + (r & (GH - 1));
    else
      return qrow(s) * Hq + kvh * GH + r;
  };
  auto load_q = [&](int s, int qb) {
    const int last = (fold.fe << fold.lg) - 1;
#pragma unroll
    for (int i = 0; i < QPL; ++i) {
      const int u = i * 64 + lane;
      const int64_t row = row_index(s, min(u / QNCH, last));
      dma16(reinterpret_cast<const uint4*>(q) + row * QNCH + u % QNCH, lds_offset(&q_lds[qb][i * 64]));
    }
  };

  // Row state of this lane's query row (the lanes l ^ 16, l ^ 32, l ^ 48
  // hold the same m; their l are partial sums over their own batch rows).
  float m = -INFINITY, lsum = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Token of this lane's row within the pass (MT): the rows it may see end
  // fe - 1 - j before the pass's context end.  Idle rows see nothing.
  const int tok = col >> fold.lg;
  const bool active = tok < fold.fe;

  Batch cur = first, nxt;
  int sb = 0;  // scale buffer of the current batch (fp8)
  load_q(cur.s, cur.qb);
  issue_k(cur, sb);
  issue_tiles(vbytes, cur, v_base);

  while (true) {
    const bool has_next = walk.advance(cur, nxt);
    // K (and q, loaded before it, and the fp8 scales) of this batch have
    // landed once only this batch's V may be outstanding.
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NV) : "memory");
    lds_order();
    if (has_next && nxt.s != cur.s) load_q(nxt.s, nxt.qb);

    // S^T = K Q^T.
    const uint4* qcur = &q_lds[cur.qb][0];
    f32x4 sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 qb = *(LdsU4*)(&qcur[col * QNCH + c * 4 + lg]);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key = kb * 16 + col;
        u32x4 a;
        if constexpr (FP8) {
          // codes 32 c + 8 lg .. +7 of the row: half of a swizzled chunk
          const int ch = (2 * c + (lg >> 1)) ^ Gm::swz(key);
          const u32x2 w8 = *(__attribute__((address_space(3))) const u32x2*)(
              reinterpret_cast<const char*>(k_lds) + key * (RD * 4) + ch * 16 + (lg & 1) * 8);
          a = u32x4{fp8x2_to_bf16x2<false>(w8.x), fp8x2_to_bf16x2<true>(w8.x), fp8x2_to_bf16x2<false>(w8.y),
                    fp8x2_to_bf16x2<true>(w8.y)};
        } else {
          a = *(LdsU4*)(&k_lds[key * NCH + ((c * 4 + lg) ^ Gm::swz(key))]);
        }
        sc[kb] = mfma16x16x32(a, qb, sc[kb]);
      }
    }
    // Every read of this batch's K is done: the next K may land.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) issue_k(nxt, sb ^ 1);

    // Online softmax of this lane's row over its 16 batch rows.
    const int nvalid = min(cur.seg_hi * 16, cur.L) - cur.pb * 16;  // rows of this batch (1..64)
    const int lo_b = cur.lo - cur.pb * 16;  // rows before the window (<= 0: none)
    // (MT) rows after this token's own position are not seen
    const int hi_t = cur.L - (fold.fe - 1 - tok) - cur.pb * 16;  // (MT) one past this row's token position
    const int hi_b = !active ? 0 : MT ? min(nvalid, hi_t) : nvalid;
    // (MT with a window) the row's own window starts win rows before its end
    const int lo_r = MT && fold.win > 0 ? max(lo_b, hi_t - fold.win) : lo_b;
    float x[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      // fp8: the K scales of this lane's 4 rows of the block
      const float4 ksc = row_scales<FP8>(lds, true, sb, kb * 4 + lg);
      const float kq[4] = {ksc.x, ksc.y, ksc.z, ksc.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb * 16 + lg * 4 + i;
        x[kb][i] = key < hi_b && key >= lo_r ? sc[kb][i] * (FP8 ? kq[i] * scale_log2 : scale_log2) : -INFINITY;
        mx = fmaxf(mx, x[kb][i]);
      }
    }
    mx = max_xor32(max_xor16(mx));
    const float mn = fmaxf(m, mx);
    // (a row that has seen nothing yet keeps m = -inf: exponents are then
    // taken against 0 so that -inf - -inf never occurs)
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(m - mref);
    m = mn;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    u32x4 pb[2];  // P^T operand of keys 32 ks .. 32 ks + 31
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float p[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 vsc = row_scales<FP8>(lds, false, sb, (2 * ks + h) * 4 + lg);
        const float vq[4] = {vsc.x, vsc.y, vsc.z, vsc.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[h][i] = fast_exp2(x[2 * ks + h][i] - mref);
          lsum += p[h][i];
          // fp8: P^T carries p times the row's V scale (0 for rows not
          // seen, whose scale may be NaN)
          if constexpr (FP8) p[h][i] = x[2 * ks + h][i] == -INFINITY ? 0.f : p[h][i] * vq[i];
        }
      }
      // k slots 8 lg .. 8 lg + 7 = batch rows 32 ks + 4 lg + [0, 4) and
      // 32 ks + 16 + 4 lg + [0, 4): the order the V^T operand uses.
      pb[ks] = u32x4{bf16x2_rne(p[0][0], p[0][1]), bf16x2_rne(p[0][2], p[0][3]), bf16x2_rne(p[1][0], p[1][1]),
                     bf16x2_rne(p[1][2], p[1][3])};
    }

    // V of this batch: the next K may still be outstanding.
    if (has_next)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NK) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_order();
    // Rows past the end (NaN poison in the pool) or before the window are
    // zeroed in LDS before they are read: p = 0 times NaN would be NaN.
    if (nvalid < 64 || lo_b > 0) {
      uint4* vz = v_lds;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int slot = i * 64 + lane;
        const int row = slot / NCH;
        if (row >= nvalid || row < lo_b) vz[slot] = make_uint4(0u, 0u, 0u, 0u);
      }
      lds_order();
    }
    // O^T += V^T P^T: the V^T operand (columns 16 db + col, rows as in
    // P^T) from two transposed reads of 4 rows each.
    const char* vb = reinterpret_cast<const char*>(v_lds);
    const int tr_r = col >> 2, tr_c = col & 3;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        u32x4 a;
        if constexpr (FP8) {
          // one transposed read of 8 rows: lanes 2r, 2r+1 name row r of
          // the block, the batch rows in P^T's order
          const int r8 = col >> 1;
          const int row = ks * 32 + (r8 >> 2) * 16 + lg * 4 + (r8 & 3);
          const u32x2 w8 = lds_read_tr8(vb + row * (RD * 4) + (db ^ Gm::swz(row)) * 16 + (col & 1) * 8);
          a = u32x4{fp8x2_to_bf16x2<false>(w8.x), fp8x2_to_bf16x2<true>(w8.x), fp8x2_to_bf16x2<false>(w8.y),
                    fp8x2_to_bf16x2<true>(w8.y)};
        } else {
          u32x2 part[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int row = ks * 32 + e * 16 + lg * 4 + tr_r;
            const int ch = (db * 2 + (tr_c >> 1)) ^ Gm::swz(row);
            part[e] = lds_read_tr16(vb + row * (RD * 4) + ch * 16 + (tr_c & 1) * 8);
          }
          a = u32x4{part[0].x, part[0].y, part[1].x, part[1].y};
        }
        o[db] = mfma16x16x32(a, pb[ks], o[db]);
      }
    }
    // Every read of this batch's V is done: the next V may land.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) issue_tiles(vbytes, nxt, v_base);

    if (cur.pb + 4 >= cur.seg_hi) {
      // End of this wave's part of sequence cur.s: normalise, write the
      // output (whole sequence), a cascade partial, or a partial.
      const int s = cur.s;
      const bool whole = cur.seg_lo == cur.B && cur.seg_hi == cur.P;
      const int slot = (s == s0) ? 0 : 1;
      if (cur.seg_lo == cur.B && kvh == 0 && lane == 0) {
        seq_info[4 * s + 0] = w;
        seq_info[4 * s + 1] = run_wave(cur.cs + (cur.P - cur.B) - 1, per, lead);  // last wave on the sequence
        seq_info[4 * s + 2] = slot;
        seq_info[4 * s + 3] = 0;
      }
      const float lt = add_xor32(add_xor16(lsum));
      // (a folded row can see no row of this wave's part: a partial of
      // weight 0, zero output, log2-sum-exp -inf)
      const float inv = lt == 0.f ? 0.f : 1.0f / lt;
      const float lse2 = m + fast_log2(lt);
      if (whole && seq_part) {
        // seq_part: bf16 rows [S][Hq][D] (rounded to nearest even), then
        // from float S Hq D on, the log2-sum-exp [S][Hq] as float32.
        if (active) {
          const int64_t r = static_cast<int64_t>(s) * Hq + kvh * GH + col;
          uint16_t* row = reinterpret_cast<uint16_t*>(seq_part) + r * D + lg * 4;
#pragma unroll
          for (int db = 0; db < DB; ++db)
            *reinterpret_cast<uint2*>(row + db * 16) =
                make_uint2(bf16x2_rne(o[db][0] * inv, o[db][1] * inv), bf16x2_rne(o[db][2] * inv, o[db][3] * inv));
          if (lg == 0) seq_part[static_cast<int64_t>(S) * Hq * D + r] = lse2;
        }
      } else if (whole) {
        if (active) {
          const int64_t row = row_index(s, col);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            *reinterpret_cast<uint2*>(out + row * D + db * 16 + lg * 4) =
                make_uint2(bf16x2_rne(o[db][0] * inv, o[db][1] * inv), bf16x2_rne(o[db][2] * inv, o[db][3] * inv));
          if (lse_out && lg == 0) lse_out[row] = lse2 * kLn2;
        }
      } else if (active) {  // (idle rows leave no partial; the merge skips them)
        const int64_t r = ((static_cast<int64_t>(w) * Hkv + kvh) * 2 + slot) * R + col;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<float4*>(part_o + r * D + db * 16 + lg * 4) =
              make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
        if (lg == 0) part_lse[r] = lse2;
      }
      m = -INFINITY;
      lsum = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (!has_next) break;
    cur = nxt;
    sb ^= 1;
  }
}


}  // namespace pa
