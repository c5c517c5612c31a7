// Paged decode attention for gfx950 (MI355X): stream-K split-KV kernels and
// log-sum-exp merge.
//
// Work split.  For each kv-head, the pages of all sequences are laid end to
// end (sequence 0's pages, then sequence 1's, ...) and cut into W equal runs
// of `per` pages; wave w of kv-head g streams run w.  A run can end inside a
// sequence, so a long sequence is shared by several waves and a wave can
// cover many short sequences: every wave gets the same number of bytes to
// read whatever the length mix.  A sequence that one wave covers entirely is
// written out directly; a sequence shared by several waves leaves one
// partial (normalised output + log2-sum-exp) per wave, and the merge kernel
// reduces those by their log-sum-exp.  This is the split-KV / second-pass
// reduction the TokenSpeed deep-dive describes (sections 7 and 7.1), with
// the splits placed by byte count instead of a fixed split count.
//
// Inside a wave: batches of 4 pages (64 rows) of one sequence; the next
// batch's K and V travel while this one is computed.
//  * K and V: the 4 (page, kv-head) tiles go straight from HBM into LDS with
//    16-byte global_load_lds (1 KB contiguous per instruction), K XOR-
//    swizzled so that a read of one row per lane is bank-conflict free; q by
//    DMA into a double buffer when a new sequence starts.
//  * Two kernels share this walk and pipeline and differ in the math.
//    stream_decode_kernel (1 or 2 q-heads per kv-head, and float32): lane =
//    row, the K row against q broadcast from LDS on v_dot2_f32_bf16 (fp32:
//    v_fma); V rows copied to registers; P.V with the probabilities through
//    LDS, rounded to bf16 (nearest even) and paired across rows for
//    v_dot2_f32_bf16 while the normaliser and the log-sum-exp use the
//    float32 values.  stream_mfma_kernel (4 to 16 bf16 query rows per wave):
//    the same batch on 16 x 16 x 32 MFMA tiles (described below).
//    The G q-heads sharing a kv-head all use one pass over K and V (the
//    analog of fold_sq_factor, TokenSpeed deep-dive section 7.2).
//  * Multi-token decode (n new tokens per sequence, causal among them):
//    F tokens of a sequence are folded into the wave's query rows next to
//    the heads (row r = token r / g, head r % g), which is the fold of the
//    same section with the wave's 16 rows in place of the 128-row tile;
//    token j of a pass masks the rows after its own position.
//  * Online softmax per query row in the exp2 domain; rows past the end are
//    masked by select (never by multiplying by zero) so NaN poison in
//    unused rows cannot leak.
// The page walk follows the block table of the PagedAttention cache
// (SwiftLLM page, section 3.1); physical page ids are clamped into the pool.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <string>
#include <vector>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_stream.h"

namespace pa {
namespace {

template <int EPC>
__device__ __forceinline__ void unpack_chunk(const uint4& c, float (&v)[EPC]) {
  if constexpr (EPC == 8) {
    v[0] = bf16_lo(c.x); v[1] = bf16_hi(c.x);
    v[2] = bf16_lo(c.y); v[3] = bf16_hi(c.y);
    v[4] = bf16_lo(c.z); v[5] = bf16_hi(c.z);
    v[6] = bf16_lo(c.w); v[7] = bf16_hi(c.w);
  } else {
    v[0] = __uint_as_float(c.x); v[1] = __uint_as_float(c.y);
    v[2] = __uint_as_float(c.z); v[3] = __uint_as_float(c.w);
  }
}

template <typename T>
__device__ __forceinline__ float dot_chunk(const uint4& k, uint32_t q0, uint32_t q1, uint32_t q2, uint32_t q3,
                                           float acc) {
  if constexpr (sizeof(T) == 2) {
    acc = dot2_bf16(k.x, q0, acc);
    acc = dot2_bf16(k.y, q1, acc);
    acc = dot2_bf16(k.z, q2, acc);
    acc = dot2_bf16(k.w, q3, acc);
  } else {
    acc = fmaf(__uint_as_float(k.x), __uint_as_float(q0), acc);
    acc = fmaf(__uint_as_float(k.y), __uint_as_float(q1), acc);
    acc = fmaf(__uint_as_float(k.z), __uint_as_float(q2), acc);
    acc = fmaf(__uint_as_float(k.w), __uint_as_float(q3), acc);
  }
  return acc;
}

// Pair two rows' bf16 values column by column: (lo: row a, hi: row b).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// G: query rows per wave: the q-heads of one kv-head, or (MT) a pass's
// folded (token, head) rows.
template <typename T, typename TKV, int D, int G, bool MT>
__global__ __launch_bounds__(64) void stream_decode_kernel(
    T* __restrict__ out, float* __restrict__ lse_out, const T* __restrict__ q, const TKV* __restrict__ k_pool,
    const TKV* __restrict__ v_pool, const float* __restrict__ k_scales, const float* __restrict__ v_scales,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ ctx,
    int max_blocks, int S, int Hkv, int num_pages, float scale_log2, int per, int lead, int total_pages,
    int32_t* __restrict__ seq_info, float* __restrict__ part_o, float* __restrict__ part_lse,
    PageSkip skip, float* __restrict__ seq_part, const int32_t* __restrict__ q_rows, Fold fold) {
  using Gm = Geom<TKV, D>;
  constexpr int RD = Gm::RD, NCH = Gm::NCH, TILE = Gm::TILE, NI = Gm::NI, RPI = Gm::RPI, EPC = Gm::EPC;
  constexpr bool FP8 = sizeof(TKV) == 1;
  constexpr bool BF16 = sizeof(T) == 2;  // bf16 q/out; P.V on bf16 pairs (also for fp8 pools)
  static_assert(!FP8 || BF16, "fp8 pools come with bf16 q and out");
  constexpr int NK = NI + (FP8 ? 2 : 0);  // loads one issue_k makes (K rows, + the K and V scales)
  constexpr int NV = NI;                  // loads one issue_v makes
  constexpr int QNCH = D * sizeof(T) / 16;  // 16-byte chunks of one q row
  constexpr int QPC = FP8 ? 2 : 1;          // q chunks per K chunk
  constexpr int per_tile = TILE / 1024;  // 1 KB loads per page tile
  constexpr int CG = (8 / G) < 1 ? 1 : ((8 / G) > 4 ? 4 : (8 / G));  // K chunks per QK step
  static_assert(NCH % CG == 0, "chunk groups must tile the row");
  static_assert(QNCH == NCH * QPC, "q chunks must line up with K chunks");
  constexpr int QU4 = G * QNCH;              // 16-byte chunks of the G q rows
  constexpr int QPL = (QU4 + 63) / 64;        // of them per lane when loading
  static_assert(NV + NK <= 63, "vmcnt counts at most 63 loads");
  static_assert(!MT || (!FP8 && (G & (G - 1)) == 0), "folded passes: bf16/f32 pools, power-of-two rows");
  __shared__ uint4 k_lds[64 * NCH];
  __shared__ uint4 v_lds[64 * NCH];
  __shared__ uint4 q_lds[2][QPL * 64];              // two sequences' q rows (current, next)
  __shared__ __align__(16) uint32_t p_lds[G * 64];  // fp32 bits, or bf16 in the first half
  __shared__ float ks_lds[FP8 ? 64 : 1];            // fp8: scale of each K row of the batch
  __shared__ float vs_lds[FP8 ? 64 : 1];            // fp8: scale of each V row of the batch

  const int lane = lane_id();
  const int grp = lane / NCH;  // V layout: row group of this lane
  const int chk = lane % NCH;  // V layout: 16-byte column chunk of this lane
  const int w = blockIdx.x;
  const int kvh = blockIdx.y;
  const int GH = MT ? fold.g : G;  // q-heads per kv-head
  const int Hq = Hkv * GH;
  const int trim = MT ? fold.trim : 0;
  const char* kbytes = reinterpret_cast<const char*>(k_pool);
  const char* vbytes = reinterpret_cast<const char*>(v_pool);

  const int run_a = run_begin(w, per, lead);
  const int run_b = min(run_begin(w + 1, per, lead), total_pages);
  if (run_a >= run_b) return;

  // Per-lane offsets inside a page tile.  K: instruction i of a tile fills
  // LDS slots 64i..64i+63 of that tile's rows; slot -> (row, chunk) with the
  // chunk XOR-swizzled by the row.  V: lane = (row group, chunk).
  uint32_t koff[per_tile];
#pragma unroll
  for (int r = 0; r < per_tile; ++r) {
    const int slot = r * 64 + lane;
    const int row = slot / NCH;
    const int ch = (slot % NCH) ^ Gm::swz(row);
    koff[r] = row * (RD * 4) + ch * 16;
  }
  const uint32_t voff = grp * (RD * 4) + chk * 16;
  // p slot of the row this lane scores: the rows a V row group holds are
  // contiguous, so its P.V read is one run.
  const int pslot = (lane % RPI) * NI + lane / RPI;

  // Where the run starts: sequence s0 and its first flattened page.
  const Walk walk{ctx, skip, q_rows, block_tables, S, max_blocks, num_pages, trim, run_b};
  Batch first;
  if (!walk.start(run_a, first)) return;
  const int s0 = first.s;

  // K and V of a batch go to LDS by DMA, NI loads of 1 KB each: K with the
  // swizzled layout above; V as it is in the pool (instruction i: rows
  // i*RPI .. +RPI, lane (grp, chk) = its row grp, chunk chk).
  const uint32_t k_base = lds_offset(k_lds);
  const uint32_t v_base = lds_offset(v_lds);
  // fp8: lane r fetches the scale of batch row r (page r / 16, slot r % 16).
  auto scale_src = [&](const float* pool, const Batch& b) {
    // (values first: a conditional over the array elements themselves would
    // load through a selected address and keep the batch in scratch memory)
    const int p0 = b.pid[0], p1 = b.pid[1], p2 = b.pid[2], p3 = b.pid[3];
    const int pl = lane < 32 ? (lane < 16 ? p0 : p1) : (lane < 48 ? p2 : p3);
    return pool + (static_cast<int64_t>(pl) * Hkv + kvh) * 16 + (lane & 15);
  };
  auto issue_k = [&](const Batch& b) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const char* tile = kbytes + (static_cast<int64_t>(b.pid[i / per_tile]) * Hkv + kvh) * TILE;
      dma16(tile + koff[i % per_tile], k_base + i * 1024);
    }
    // fp8: both scale runs of the batch travel with its K, so that they
    // have landed when the batch's scores start.
    if constexpr (FP8) {
      dma4(scale_src(k_scales, b), lds_offset(ks_lds));
      dma4(scale_src(v_scales, b), lds_offset(vs_lds));
    }
  };
  auto issue_v = [&](const Batch& b) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row0 = i * RPI;
      const char* tile = vbytes + (static_cast<int64_t>(b.pid[row0 / 16]) * Hkv + kvh) * TILE;
      dma16(tile + (row0 % 16) * (RD * 4) + voff, v_base + i * 1024);
    }
  };

  // The G q rows of sequence s for this kv-head, by DMA into q buffer qb
  // (lanes past the rows repeat the last chunk into the buffer's tail).
  // Row of q / out / lse of sequence s (mixed batches: its one token).
  auto qrow = [&](int s) -> int64_t { return q_rows ? q_rows[s] : s; };
  auto load_q = [&](int s, int qb) {
    if constexpr (MT) {
      // row r of the pass: token tok0 + (r >> lg), head r & (g-1); idle
      // rows (and lanes past the rows) repeat the last active row
      const int last = (fold.fe << fold.lg) - 1;
#pragma unroll
      for (int i = 0; i < QPL; ++i) {
        const int u = i * 64 + lane;
        const int r = min(u / QNCH, last);
        const int64_t row = (static_cast<int64_t>(s) * fold.n + fold.tok0 + (r >> fold.lg)) * Hq + kvh * GH +
                            (r & (GH - 1));
        dma16(reinterpret_cast<const uint4*>(q) + row * QNCH + u % QNCH, lds_offset(&q_lds[qb][i * 64]));
      }
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(q + (qrow(s) * Hq + kvh * G) * D);
#pragma unroll
      for (int i = 0; i < QPL; ++i) {
        const int u = i * 64 + lane;
        dma16(src + (u < QU4 ? u : QU4 - 1), lds_offset(&q_lds[qb][i * 64]));
      }
    }
  };

  float m[G], l[G], acc[G][EPC];
  auto reset = [&]() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;
    }
  };
  reset();

  // cur is the batch being computed, nxt the one after it, whose K and V
  // are issued during cur's math (q of a new sequence is loaded right
  // before the K of its first batch).
  Batch cur = first, nxt;
  load_q(cur.s, cur.qb);
  issue_k(cur);
  issue_v(cur);

  while (true) {
    const bool has_next = walk.advance(cur, nxt);

    // K of this batch (and its scales, and q, loaded before it) is in LDS
    // once only this batch's V may be outstanding.
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NV) : "memory");
    lds_order();
    // The next sequence's q goes to the other q buffer (last read two
    // sequences ago).
    if (has_next && nxt.s != cur.s) load_q(nxt.s, nxt.qb);
    const int qcur = cur.qb;

    // Scores, lane = row: K row chunks and q chunks (one address for the
    // whole wave, a broadcast read) from LDS, CG chunks at a time.
    const int nvalid = min(cur.seg_hi * 16, cur.L) - cur.pb * 16;  // rows of this batch (1..64)
    const int lo_b = cur.lo - cur.pb * 16;  // rows of this batch before the window (<= 0: none)
    // fp8: this row's K and V scales, read before the next batch's K (and
    // scales) may be issued into the same LDS.
    const float k_row_scale = FP8 ? ks_lds[FP8 ? lane : 0] : 1.0f;
    const float v_row_scale = FP8 ? vs_lds[FP8 ? lane : 0] : 1.0f;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < NCH; c0 += CG) {
      // K and q are read through pointers made opaque per chunk group and
      // tied to the previous group's result, so each group's reads are
      // issued after the previous group's math: only CG chunks of K and
      // G*CG chunks of q are in registers at a time.
      LdsU4* qp = (LdsU4*)(&q_lds[qcur][0]);
      LdsU4* kp = (LdsU4*)(&k_lds[lane * NCH]);
#pragma unroll
      for (int h = 0; h < G; ++h) asm volatile("" : "+v"(qp), "+v"(kp) : "v"(sc[h]));
      u32x4 kr[CG];
#pragma unroll
      for (int c = 0; c < CG; ++c) kr[c] = kp[(c0 + c) ^ Gm::swz(lane)];
      if constexpr (FP8) {
        // 16 codes per chunk -> 8 bf16 pairs (exact), once for all G heads.
        uint32_t kb[CG][8];
#pragma unroll
        for (int c = 0; c < CG; ++c) fp8x16_to_bf16x2(kr[c], kb[c]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            const u32x4 q0 = qp[h * QNCH + 2 * (c0 + c)];
            const u32x4 q1 = qp[h * QNCH + 2 * (c0 + c) + 1];
            float a = sc[h];
            a = dot2_bf16(kb[c][0], q0.x, a);
            a = dot2_bf16(kb[c][1], q0.y, a);
            a = dot2_bf16(kb[c][2], q0.z, a);
            a = dot2_bf16(kb[c][3], q0.w, a);
            a = dot2_bf16(kb[c][4], q1.x, a);
            a = dot2_bf16(kb[c][5], q1.y, a);
            a = dot2_bf16(kb[c][6], q1.z, a);
            sc[h] = dot2_bf16(kb[c][7], q1.w, a);
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            const u32x4 qv = qp[h * QNCH + c0 + c];
            sc[h] = dot_chunk<T>(make_uint4(kr[c].x, kr[c].y, kr[c].z, kr[c].w), qv.x, qv.y, qv.z, qv.w, sc[h]);
          }
        }
      }
      asm volatile("" ::: "memory");
    }
    // All LDS reads of this batch's K are done: the next K may land.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) issue_k(nxt);

    // Online softmax; probabilities to LDS.
    const bool valid = lane < nvalid && lane >= lo_b;
    // fp8: the row's K scale multiplies its scores; its V scale is folded
    // into the probability that P.V uses (the normaliser sums the plain
    // probabilities).  Rows past the end select 0 / -inf, never multiply.
    const float kscale = FP8 ? k_row_scale * scale_log2 : scale_log2;
    const float vscale = v_row_scale;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      bool vis = valid;
      if constexpr (MT) {
        // token j of the pass sees the rows up to its own position:
        // those before L - (fe - 1 - j) of the pass's (trimmed) context
        const int j = h >> fold.lg;
        const int lim = j < fold.fe ? cur.L - (fold.fe - 1 - j) - cur.pb * 16 : 0;
        // (with a window: only the win rows up to the token's own position)
        vis = valid && lane < lim && (fold.win == 0 || lane >= lim - fold.win);
      }
      const float s2 = vis ? sc[h] * kscale : -INFINITY;
      const float mn = fmaxf(m[h], wave_max(s2));
      // (folded rows can see no row of a batch yet: then exponents are
      // taken against 0 so that -inf - -inf never occurs)
      const float mref = MT && mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[h] - mref);
      const float p = fast_exp2(s2 - mref);
      // The normaliser sums the float32 probabilities; for bf16 the P.V
      // product uses them rounded to bf16 (unbiased, round to nearest even).
      const uint32_t pbits = BF16 ? bf16_bits_rne(FP8 ? (valid ? p * vscale : 0.f) : p) : __float_as_uint(p);
      l[h] = l[h] * alpha + p;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha;
      m[h] = mn;
      if constexpr (BF16)
        reinterpret_cast<uint16_t*>(p_lds)[h * 64 + pslot] = static_cast<uint16_t>(pbits);
      else
        p_lds[h * 64 + pslot] = pbits;
    }
    // V of this batch: the next K (NK loads, and before it the next q)
    // may still be outstanding.
    if (has_next)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NK) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_order();
    // This batch's V rows to registers; once read, the buffer takes the
    // next batch's V, which then streams in during this batch's P.V and
    // the next batch's scores.
    uint4 vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = v_lds[i * 64 + lane];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (has_next) issue_v(nxt);
    if (nvalid < 64 || lo_b > 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (i * RPI + grp >= nvalid || i * RPI + grp < lo_b) vr[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    // P.V: lane (grp, chk) accumulates its NI rows into its EPC columns.
    if constexpr (FP8) {
      // Rows (2u, 2u+1) of the group: their codes interleaved byte by byte
      // and widened to bf16 pairs (row 2u low, row 2u+1 high), one pair per
      // column, against the pair of their scaled probabilities.
#pragma unroll
      for (int i8 = 0; i8 < NI; i8 += 8) {
        uint4 pp[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
          pp[h] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p_lds) + h * 64 + grp * NI + i8);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 va = vr[i8 + 2 * u], vb = vr[i8 + 2 * u + 1];
          const uint32_t a4[4] = {va.x, va.y, va.z, va.w}, b4[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
          for (int d4 = 0; d4 < 4; ++d4) {
            const uint32_t x0 = __builtin_amdgcn_perm(b4[d4], a4[d4], 0x05010400u);  // a0 b0 a1 b1
            const uint32_t x1 = __builtin_amdgcn_perm(b4[d4], a4[d4], 0x07030602u);  // a2 b2 a3 b3
            const uint32_t vp[4] = {fp8x2_to_bf16x2<false>(x0), fp8x2_to_bf16x2<true>(x0),
                                    fp8x2_to_bf16x2<false>(x1), fp8x2_to_bf16x2<true>(x1)};
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const uint32_t pw = u == 0 ? pp[h].x : u == 1 ? pp[h].y : u == 2 ? pp[h].z : pp[h].w;
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[h][4 * d4 + e] = dot2_bf16(vp[e], pw, acc[h][4 * d4 + e]);
            }
          }
        }
      }
    } else if constexpr (BF16) {
      // Probabilities of rows (2k, 2k+1) of the group against V pairs.
#pragma unroll
      for (int i8 = 0; i8 < NI; i8 += 8) {
        uint4 pp[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
          pp[h] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p_lds) + h * 64 + grp * NI + i8);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 va = vr[i8 + 2 * u], vb = vr[i8 + 2 * u + 1];
          const uint32_t vp[8] = {pair_lo(va.x, vb.x), pair_hi(va.x, vb.x), pair_lo(va.y, vb.y), pair_hi(va.y, vb.y),
                                  pair_lo(va.z, vb.z), pair_hi(va.z, vb.z), pair_lo(va.w, vb.w), pair_hi(va.w, vb.w)};
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const uint32_t pw = u == 0 ? pp[h].x : u == 1 ? pp[h].y : u == 2 ? pp[h].z : pp[h].w;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = dot2_bf16(vp[e], pw, acc[h][e]);
          }
        }
      }
    } else {
#pragma unroll
      for (int i4 = 0; i4 < NI; i4 += 4) {
        float4 p4[G];
#pragma unroll
        for (int h = 0; h < G; ++h) p4[h] = *reinterpret_cast<const float4*>(&p_lds[h * 64 + grp * NI + i4]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float v[EPC];
          unpack_chunk<EPC>(vr[i4 + u], v);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float p = u == 0 ? p4[h].x : u == 1 ? p4[h].y : u == 2 ? p4[h].z : p4[h].w;
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
          }
        }
      }
    }
    const bool seg_end = cur.pb + 4 >= cur.seg_hi;

    if (seg_end) {
      // End of this wave's part of sequence cur.s: sum the row groups,
      // normalise, write the output (whole sequence) or a partial.
      const int s = cur.s;
      const bool whole = cur.seg_lo == cur.B && cur.seg_hi == cur.P;
      const int slot = (s == s0) ? 0 : 1;
      if (cur.seg_lo == cur.B && kvh == 0 && lane == 0) {
        seq_info[4 * s + 0] = w;
        seq_info[4 * s + 1] = run_wave(cur.cs + (cur.P - cur.B) - 1, per, lead);  // last wave on the sequence
        seq_info[4 * s + 2] = slot;
        seq_info[4 * s + 3] = 0;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          float a = acc[h][e];
          if constexpr (NCH == 8) a += dpp<kDppRor8>(a);  // rows 8 apart share a row of 16
          acc[h][e] = add_xor32(add_xor16(a));
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float lt = wave_sum(l[h]);
        // (a folded row can see no row of this wave's part: a partial of
        // weight 0, zero output, log2-sum-exp -inf)
        const float inv = MT && lt == 0.f ? 0.f : 1.0f / lt;
        const float lse2 = m[h] + fast_log2(lt);
        const bool act = !MT || (h >> fold.lg) < fold.fe;  // idle folded rows write nothing
        const bool mine = act && (h % RPI) == grp;  // one row group writes each head
        if (whole && seq_part) {
          // Cascade: the suffix of a sequence one wave covered is still a
          // partial, to be merged with the shared prefix's.
          // seq_part: bf16 rows [S][Hq][D] (rounded to nearest even), then
          // from float S Hq D on, the log2-sum-exp [S][Hq] as float32.
          const int64_t r = static_cast<int64_t>(s) * Hq + kvh * G + h;
          if (mine) {
            uint2* dst = reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(seq_part) + r * D + chk * EPC);
#pragma unroll
            for (int e = 0; e < EPC; e += 4)
              dst[e / 4] = make_uint2(bf16x2_rne(acc[h][e] * inv, acc[h][e + 1] * inv),
                                      bf16x2_rne(acc[h][e + 2] * inv, acc[h][e + 3] * inv));
          }
          if (lane == 0) seq_part[static_cast<int64_t>(S) * Hq * D + r] = lse2;
        } else if (whole) {
          const int64_t row = MT ? (static_cast<int64_t>(s) * fold.n + fold.tok0 + (h >> fold.lg)) * Hq + kvh * GH +
                                       (h & (GH - 1))
                                 : qrow(s) * Hq + kvh * G + h;
          if (mine) {
            // columns chk*EPC .. +EPC of the output row
            if constexpr (BF16) {
#pragma unroll
              for (int j = 0; j < EPC / 8; ++j) {
                uint4 o;
                o.x = bf16x2_rne(acc[h][8 * j + 0] * inv, acc[h][8 * j + 1] * inv);
                o.y = bf16x2_rne(acc[h][8 * j + 2] * inv, acc[h][8 * j + 3] * inv);
                o.z = bf16x2_rne(acc[h][8 * j + 4] * inv, acc[h][8 * j + 5] * inv);
                o.w = bf16x2_rne(acc[h][8 * j + 6] * inv, acc[h][8 * j + 7] * inv);
                reinterpret_cast<uint4*>(out)[(row * D + chk * EPC) / 8 + j] = o;
              }
            } else {
#pragma unroll
              for (int j = 0; j < EPC / 4; ++j)
                reinterpret_cast<float4*>(out)[(row * D + chk * EPC) / 4 + j] =
                    make_float4(acc[h][4 * j] * inv, acc[h][4 * j + 1] * inv, acc[h][4 * j + 2] * inv,
                                acc[h][4 * j + 3] * inv);
            }
          }
          if (lse_out && act && lane == 0) lse_out[row] = lse2 * kLn2;
        } else {
          const int64_t r = ((static_cast<int64_t>(w) * Hkv + kvh) * 2 + slot) * G + h;
          if (mine) {
            float4* dst = reinterpret_cast<float4*>(part_o + r * D + chk * EPC);
#pragma unroll
            for (int e = 0; e < EPC; e += 4)
              dst[e / 4] = make_float4(acc[h][e] * inv, acc[h][e + 1] * inv, acc[h][e + 2] * inv, acc[h][e + 3] * inv);
          }
          if (lane == 0) part_lse[r] = lse2;
        }
      }
      reset();
    }
    if (!has_next) break;
    cur = nxt;
  }
}

// The stream kernel for waves of 16 query rows on the matrix cores: one
// wave per workgroup, run blockIdx.x of kv-head blockIdx.y (the body and
// its description are in pa_stream.h).
template <typename TKV, int D, bool MT>
__global__ __launch_bounds__(64) void stream_mfma_kernel(
    uint16_t* __restrict__ out, float* __restrict__ lse_out, const uint16_t* __restrict__ q,
    const TKV* __restrict__ k_pool, const TKV* __restrict__ v_pool, const float* __restrict__ k_scales,
    const float* __restrict__ v_scales, const int32_t* __restrict__ block_tables, const int32_t* __restrict__ ctx,
    int max_blocks, int S, int Hkv, int num_pages, float scale_log2, int per, int lead, int total_pages,
    int32_t* __restrict__ seq_info, float* __restrict__ part_o, float* __restrict__ part_lse,
    PageSkip skip, float* __restrict__ seq_part, const int32_t* __restrict__ q_rows, Fold fold) {
  __shared__ StreamMfmaLds<TKV, D> lds;
  stream_mfma_body<TKV, D, MT>(lds, blockIdx.x, blockIdx.y, out, lse_out, q, k_pool, v_pool, k_scales, v_scales,
                               block_tables, ctx, max_blocks, S, Hkv, num_pages, scale_log2, per, lead,
                               total_pages, seq_info, part_o, part_lse, skip, seq_part, q_rows, fold);
}

// Merge the partials of one (sequence, kv-head): the waves w0..w1 that
// shared the sequence each left (o_w, lse_w) per head; out = sum_w a_w o_w /
// sum_w a_w with a_w = 2^(lse_w - max lse), lse = max + log2(sum a_w).  Lane
// j holds wave j's weights; lane d holds output columns; four waves'
// partial rows are loaded together.
// G: partial rows per (wave, kv-head, slot).  A workgroup merges NA of
// them, rows NA * blockIdx.z .. +NA-1 (the grid covers only rows that can
// be active: rows past gqa_ratio of a 16-row wave were never written).
template <typename T, int D, int G, int NA, bool MT>
__global__ __launch_bounds__(64) void merge_kernel(T* __restrict__ out, float* __restrict__ lse_out, int Hkv, int W,
                                                   const int32_t* __restrict__ seq_info,
                                                   const float* __restrict__ part_o,
                                                   const float* __restrict__ part_lse,
                                                   const int32_t* __restrict__ q_rows, Fold fold) {
  constexpr int EPL = D / 64;  // output elements per lane
  const int lane = lane_id();
  const int s = blockIdx.x;
  const int kvh = blockIdx.y;
  const int GH = fold.g;  // q-heads per kv-head
  const int Hq = Hkv * GH;
  // (mixed batch: a prefill chunk's rows are the tile kernel's; its record
  // here is not written by the stream kernel)
  if (q_rows && q_rows[s + 1] - q_rows[s] != 1) return;
  const int w0 = seq_info[4 * s + 0];
  const int w1 = seq_info[4 * s + 1];
  const int slot0 = seq_info[4 * s + 2];
  if (w1 <= w0 || w0 < 0 || w1 >= W || slot0 < 0 || slot0 > 1) return;
  const int n = w1 - w0 + 1;
  const int r0 = NA * blockIdx.z;  // first row of this workgroup
  // Partial row of (wave w0 + j, row r0 + h).
  auto prow = [&](int j, int h) -> int64_t {
    const int slot = j == 0 ? slot0 : 0;
    return ((static_cast<int64_t>(w0 + j) * Hkv + kvh) * 2 + slot) * G + r0 + h;
  };
  float M[NA];
#pragma unroll
  for (int h = 0; h < NA; ++h) M[h] = -INFINITY;
  for (int j = lane; j < n; j += 64) {
#pragma unroll
    for (int h = 0; h < NA; ++h) M[h] = fmaxf(M[h], part_lse[prow(j, h)]);
  }
#pragma unroll
  for (int h = 0; h < NA; ++h) M[h] = wave_max(M[h]);
  float acc[NA][EPL], wsum[NA];
#pragma unroll
  for (int h = 0; h < NA; ++h) {
    wsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int j = j0 + lane;
    float wt[NA];
#pragma unroll
    for (int h = 0; h < NA; ++h) {
      wt[h] = j < n ? fast_exp2(part_lse[prow(min(j, n - 1), h)] - M[h]) : 0.f;
      wsum[h] += wt[h];
    }
    const int cnt = min(64, n - j0);
    for (int jj = 0; jj < cnt; jj += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jx = min(jj + u, cnt - 1);
#pragma unroll
        for (int h = 0; h < NA; ++h) {
          const float* src = part_o + prow(j0 + jx, h) * D + lane * EPL;
          const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt[h]), jx));
          const float a = (jj + u < cnt) ? wj : 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(a, src[e], acc[h][e]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < NA; ++h) {
    const int r = r0 + h;  // row of the wave
    if ((r >> fold.lg) >= fold.fe) continue;  // idle row (past gqa_ratio, or a folded pass's tokens)
    const float ws = wave_sum(wsum[h]);
    const float inv = 1.0f / ws;
    const int64_t row = MT ? (static_cast<int64_t>(s) * fold.n + fold.tok0 + (r >> fold.lg)) * Hq + kvh * GH +
                                 (r & (GH - 1))
                           : (q_rows ? q_rows[s] : s) * static_cast<int64_t>(Hq) + kvh * GH + r;
    if constexpr (sizeof(T) == 2) {
      if constexpr (EPL == 2) {
        reinterpret_cast<uint32_t*>(out)[row * (D / 2) + lane] =
            bf16x2_rne(acc[h][0] * inv, acc[h][1] * inv);
      } else {
        reinterpret_cast<uint16_t*>(out)[row * D + lane] = static_cast<uint16_t>(bf16_bits_rne(acc[h][0] * inv));
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) reinterpret_cast<float*>(out)[row * D + lane * EPL + e] = acc[h][e] * inv;
    }
    if (lse_out && lane == 0) lse_out[row] = (M[h] + fast_log2(ws)) * kLn2;
  }
}

// Resident waves of one kernel on the current device (cached per device),
// at most max_per_cu per compute unit.
template <typename KernelFn>
int resident_waves(KernelFn fn, std::atomic<int>* cache, int max_per_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, blocks = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, 64, 0) != hipSuccess) return 0;
  v = std::max(1, cus * std::min(blocks, max_per_cu));
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <typename T, typename TKV, int D, int G, bool MT = false>
int launch_typed(const DecodeLaunch& a, const int32_t* begin_pages, float* seq_part, const int32_t* q_rows, bool merge,
                 StreamPlan* plan, const Fold* multi = nullptr) {
  static std::atomic<int> occ_cache[64];
  // Waves of 16 bf16 query rows run on the matrix cores.
  constexpr bool kMfma = G == 16 && sizeof(T) == 2;
  auto kern = [] {
    if constexpr (kMfma)
      return stream_mfma_kernel<TKV, D, MT>;
    else
      return stream_decode_kernel<T, TKV, D, G, MT>;
  }();
  // The matrix-core kernel streams best at 4 waves per CU: its fp8 form
  // fits 6, which made shorter runs and more shared-sequence partials and
  // ran 8 % slower (61.9 against 56.7 us on the Llama-shaped fp8 batch);
  // 3 or 2 were slower still.
  constexpr int kWavesPerCu = kMfma ? 4 : 64;
  int64_t per = a.split_pages;
  if (per <= 0) {
    // Fill the GPU once: as many waves as can be resident, spread over the
    // kv-heads, each streaming the same number of pages.
    const int res = resident_waves(kern, occ_cache, kWavesPerCu);
    if (res <= 0) return fail(PA_EHIP, "pa_decode: occupancy query failed");
    const int64_t per_head = std::max<int64_t>(1, std::min<int64_t>(res, kMaxResidentWaves) / a.num_kv_heads);
    per = std::max<int64_t>(kMinPagesPerWave, (a.total_pages + per_head - 1) / per_head);
  }
  const int64_t W = std::max<int64_t>(1, (a.total_pages + per - 1) / per);
  if (W > 0x7ffffffe) return fail(PA_EUNSUPPORTED, "pa_decode: too many waves");
  // Automatic plans of the matrix-core kernel over bf16 pools shift pages
  // from the odd waves of each pair to the even ones (the XCD balance of
  // run_lead); the grid then holds an even number of waves per kv-head (a
  // last, empty one if W is odd), so that wave parity is workgroup parity
  // for every kv-head.  Splits the caller fixes stay equal.
  const int32_t lead = (a.split_pages <= 0 && kMfma && sizeof(TKV) == 2) ? run_lead(per) : 0;
  const int64_t Wg = lead > 0 ? (W + 1) / 2 * 2 : W;
  // partial rows per wave: the kernel's query rows (folded passes hold
  // more rows than q-heads per kv-head)
  const PartialLayout pl = partial_layout(W, a.num_seqs, a.num_kv_heads, G, a.head_dim);
  if (pl.bytes > a.workspace_bytes)
    return fail(PA_EWORKSPACE, "pa_decode: workspace holds " + std::to_string(a.workspace_bytes) +
                                   " bytes, this batch needs " + std::to_string(pl.bytes));
  if (plan) {
    plan->waves = W;
    plan->per = static_cast<int32_t>(per);
    plan->rows = G;
    plan->layout = pl;
  }
  // One token per sequence: row r is q-head r (rows past gqa_ratio idle).
  const Fold fold = multi ? *multi : Fold{1, a.gqa, __builtin_ctz(static_cast<unsigned>(a.gqa)), 0, 1, 0};
  char* ws = static_cast<char*>(a.workspace);
  int32_t* seq_info = reinterpret_cast<int32_t*>(ws + pl.info_offset);
  float* part_lse = reinterpret_cast<float*>(ws + pl.lse_offset);
  float* part_o = reinterpret_cast<float*>(ws + pl.o_offset);
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const float scale_log2 = a.scale * kLog2e;
  PageSkip skip;
  skip.begin_pages = begin_pages;
  skip.window = begin_pages ? 0 : a.window;
  if (a.timed) profile_before(a.stream);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(Wg), a.num_kv_heads), dim3(64), 0, st, static_cast<T*>(a.out),
                     a.lse_out, static_cast<const T*>(a.q), static_cast<const TKV*>(a.k_pool),
                     static_cast<const TKV*>(a.v_pool), a.k_scales, a.v_scales, a.block_tables, a.context_lens,
                     a.max_blocks, a.num_seqs,
                     a.num_kv_heads, static_cast<int>(a.num_pages), scale_log2, static_cast<int>(per), lead,
                     static_cast<int>(a.total_pages), seq_info, part_o, part_lse, skip, seq_part, q_rows, fold);
  if (a.timed) profile_after(a.stream);
  if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_decode: stream kernel launch failed");
  // Unless one wave covers everything, some sequence may be shared; the
  // merge kernel skips the sequences one wave covered.
  if (merge && W > 1) {
    // Rows merged: all of a folded pass's, else the q-heads (gqa_ratio of
    // the matrix-core kernel's 16 rows); up to 4 rows per workgroup (idle
    // rows in the last group are skipped at the write).
    constexpr int NA = G < 4 ? G : 4;
    const int rows = MT ? G : std::min(G, a.gqa);
    hipLaunchKernelGGL((merge_kernel<T, D, G, NA, MT>), dim3(a.num_seqs, a.num_kv_heads, (rows + NA - 1) / NA),
                       dim3(64), 0, st,
                       static_cast<T*>(a.out), a.lse_out, a.num_kv_heads, static_cast<int>(W), seq_info, part_o,
                       part_lse, q_rows, fold);
    if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "pa_decode: merge kernel launch failed");
  }
  return PA_OK;
}

template <typename T, typename TKV, int D>
int launch_g(const DecodeLaunch& a, const int32_t* begin_pages, float* seq_part, const int32_t* q_rows, bool merge,
             StreamPlan* plan) {
  switch (a.gqa) {
    case 1: return launch_typed<T, TKV, D, 1>(a, begin_pages, seq_part, q_rows, merge, plan);
    case 2: return launch_typed<T, TKV, D, 2>(a, begin_pages, seq_part, q_rows, merge, plan);
    case 4:
    case 8:
      // bf16 q (bf16 or fp8 pools): the matrix-core kernel, with 12 or 8
      // of its 16 rows idle, streams faster than the vector kernel's 4 or
      // 8 rows (for 1 or 2 rows the two are even)
      if constexpr (sizeof(T) == 2)
        return launch_typed<T, TKV, D, 16>(a, begin_pages, seq_part, q_rows, merge, plan);
      else if (a.gqa == 4)
        return launch_typed<T, TKV, D, 4>(a, begin_pages, seq_part, q_rows, merge, plan);
      else
        return launch_typed<T, TKV, D, 8>(a, begin_pages, seq_part, q_rows, merge, plan);
    case 16:
      return launch_typed<T, TKV, D, 16>(a, begin_pages, seq_part, q_rows, merge, plan);
  }
  return fail(PA_EUNSUPPORTED, "pa_decode: gqa_ratio not built");
}

// Folded multi-token passes: rows = query rows of work per wave (a power
// of two).  bf16 passes of 4 to 16 rows, and every pass over fp8 pools, run
// on the matrix-core kernel's 16 rows; the rest on the vector kernel.
template <typename T, typename TKV, int D>
int launch_fold_rows(const DecodeLaunch& a, int rows, const Fold& f) {
  if constexpr (sizeof(TKV) == 1) {
    return launch_typed<T, TKV, D, 16, true>(a, nullptr, nullptr, nullptr, true, nullptr, &f);
  } else {
    switch (rows) {
      case 2: return launch_typed<T, TKV, D, 2, true>(a, nullptr, nullptr, nullptr, true, nullptr, &f);
      case 4:
      case 8:
        if constexpr (sizeof(T) == 2)
          return launch_typed<T, TKV, D, 16, true>(a, nullptr, nullptr, nullptr, true, nullptr, &f);
        else if (rows == 4)
          return launch_typed<T, TKV, D, 4, true>(a, nullptr, nullptr, nullptr, true, nullptr, &f);
        else
          return launch_typed<T, TKV, D, 8, true>(a, nullptr, nullptr, nullptr, true, nullptr, &f);
      case 16: return launch_typed<T, TKV, D, 16, true>(a, nullptr, nullptr, nullptr, true, nullptr, &f);
    }
    return fail(PA_EUNSUPPORTED, "pa_decode_multi: fold rows not built");
  }
}

// Profiling ring (thread-local).
struct ProfileRing {
  std::vector<hipEvent_t> ev;  // begin/end pairs
  size_t next = 0;
};
thread_local ProfileRing g_prof;

}  // namespace

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 0;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

int launch_stream(const DecodeLaunch& a, const int32_t* begin_pages, float* seq_part, const int32_t* q_rows, bool merge,
                  StreamPlan* plan) {
  if (a.kv_fp8) {
    if (a.dtype == PA_BF16 && a.head_dim == 128)
      return launch_g<uint16_t, uint8_t, 128>(a, begin_pages, seq_part, q_rows, merge, plan);
  } else if (a.dtype == PA_BF16) {
    if (a.head_dim == 128) return launch_g<uint16_t, uint16_t, 128>(a, begin_pages, seq_part, q_rows, merge, plan);
    if (a.head_dim == 64) return launch_g<uint16_t, uint16_t, 64>(a, begin_pages, seq_part, q_rows, merge, plan);
  } else if (a.dtype == PA_F32) {
    if (a.head_dim == 64) return launch_g<float, float, 64>(a, begin_pages, seq_part, q_rows, merge, plan);
  }
  return fail(PA_EUNSUPPORTED, "pa_decode: shape not built");
}

int launch_decode(const DecodeLaunch& a) { return launch_stream(a, nullptr, nullptr, nullptr, true, nullptr); }

int launch_stream_merge(const DecodeLaunch& a, const int32_t* q_rows, int64_t waves) {
  if (!(a.dtype == PA_BF16 && a.head_dim == 128 && (a.gqa == 4 || a.gqa == 8 || a.gqa == 16)))
    return fail(PA_EUNSUPPORTED, "stream merge: shape not built");
  if (waves <= 1) return PA_OK;
  const PartialLayout pl = partial_layout(waves, a.num_seqs, a.num_kv_heads, 16, a.head_dim);
  char* ws = static_cast<char*>(a.workspace);
  const Fold fold{1, a.gqa, __builtin_ctz(static_cast<unsigned>(a.gqa)), 0, 1, 0};
  constexpr int NA = 4;
  hipLaunchKernelGGL((merge_kernel<uint16_t, 128, 16, NA, false>),
                     dim3(a.num_seqs, a.num_kv_heads, (a.gqa + NA - 1) / NA), dim3(64), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<uint16_t*>(a.out), a.lse_out, a.num_kv_heads,
                     static_cast<int>(waves), reinterpret_cast<const int32_t*>(ws + pl.info_offset),
                     reinterpret_cast<const float*>(ws + pl.o_offset), reinterpret_cast<const float*>(ws + pl.lse_offset),
                     q_rows, fold);
  if (hipGetLastError() != hipSuccess) return fail(PA_EHIP, "stream merge: launch failed");
  return PA_OK;
}

int launch_decode_multi(const DecodeLaunch& a, const MultiPlan& p) {
  if (p.q_len == 1) return launch_decode(a);
  if (static_cast<int>(p.pass_pages.size()) != p.passes) return fail(PA_EINVAL, "pa_decode_multi: bad plan");
  Fold f;
  f.n = p.q_len;
  f.g = a.gqa;
  f.lg = __builtin_ctz(static_cast<unsigned>(a.gqa));
  f.win = a.window;
  // Passes run one after another on the stream and reuse the workspace.
  for (int pass = 0; pass < p.passes; ++pass) {
    f.tok0 = pass * p.fold;
    f.fe = std::min(p.fold, p.q_len - f.tok0);
    f.trim = p.q_len - f.tok0 - f.fe;
    DecodeLaunch b = a;
    b.total_pages = p.pass_pages[pass];
    // a window: the pass's walk covers its earliest token's window (the
    // last window + fe - 1 rows of its context); each row masks its own
    b.window = a.window > 0 ? a.window + f.fe - 1 : 0;
    int rc = PA_EUNSUPPORTED;
    if (a.kv_fp8 && a.dtype == PA_BF16 && a.head_dim == 128)
      rc = launch_fold_rows<uint16_t, uint8_t, 128>(b, p.rows, f);
    else if (a.kv_fp8)
      return fail(PA_EUNSUPPORTED, "pa_decode_multi_fp8: shape not built");
    else if (a.dtype == PA_BF16 && a.head_dim == 128)
      rc = launch_fold_rows<uint16_t, uint16_t, 128>(b, p.rows, f);
    else if (a.dtype == PA_BF16 && a.head_dim == 64)
      rc = launch_fold_rows<uint16_t, uint16_t, 64>(b, p.rows, f);
    else if (a.dtype == PA_F32 && a.head_dim == 64)
      rc = launch_fold_rows<float, float, 64>(b, p.rows, f);
    else
      return fail(PA_EUNSUPPORTED, "pa_decode_multi: shape not built");
    if (rc) return rc;
  }
  return PA_OK;
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
