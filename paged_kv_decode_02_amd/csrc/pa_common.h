// Device helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 pair packed in one dword: element 0 in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two float32 -> a packed bf16 pair (a in the low half), round to nearest
// even, NaN stays NaN: one v_cvt_pk_bf16_f32 on gfx950, no branches.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) { return bf16x2_rne(f, 0.f) & 0xffffu; }

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs (products exact in float32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two e4m3fn codes (bytes 0,1 of w, or bytes 2,3 if HI) -> a packed bf16
// pair, first code in the low half: one v_cvt_scalef32_pk_bf16_fp8 with
// scale 1.  Every e4m3fn value (subnormals, signed zero, NaN) is a bf16
// value, so the conversion is exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// 16 codes (a 16-byte chunk, element 0 in the low byte of x) -> 8 bf16
// pairs in element order.
template <typename U4>
__device__ __forceinline__ void fp8x16_to_bf16x2(const U4& c, uint32_t (&o)[8]) {
  o[0] = fp8x2_to_bf16x2<false>(c.x);
  o[1] = fp8x2_to_bf16x2<true>(c.x);
  o[2] = fp8x2_to_bf16x2<false>(c.y);
  o[3] = fp8x2_to_bf16x2<true>(c.y);
  o[4] = fp8x2_to_bf16x2<false>(c.z);
  o[5] = fp8x2_to_bf16x2<true>(c.z);
  o[6] = fp8x2_to_bf16x2<false>(c.w);
  o[7] = fp8x2_to_bf16x2<true>(c.w);
}

// Vector types for LDS reads and the matrix cores.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4 LdsU4;
typedef __attribute__((address_space(3))) i16x4 LdsI16x4;

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane j of
// the group passes the address of 4 consecutive 16-bit elements, row j/4 and
// columns 4(j%4) .. +3 of a 4 x 16 block; lane j receives column j of that
// block, rows 0..3.  Returned as two packed 32-bit words.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsI16x4*)(lds));
  return __builtin_bit_cast(u32x2, r);
}

// ds_read_b64_tr_b8 (gfx950): within each group of 16 lanes, lane j of
// the group passes the address of 8 consecutive bytes, row j/2 and columns
// 8(j%2) .. +7 of an 8 x 16 block of bytes; lane j receives column j of
// that block, rows 0..7 (row k in byte k).
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 LdsI32x2;
__device__ __forceinline__ u32x2 lds_read_tr8(const void* lds) {
  const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LdsI32x2*)(lds));
  return __builtin_bit_cast(u32x2, r);
}

// D = A B + C on one 16 x 16 x 32 bf16 tile (v_mfma_f32_16x16x32_bf16).
// Lane l holds A row l % 16, B column l % 16, each at k = 8 (l / 16) ..
// +7 (8 bf16 in a u32x4, element 0 in the low half of x), and D/C column
// l % 16, rows 4 (l / 16) .. +3.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// LDS byte offset of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<size_t>((__attribute__((address_space(3))) const void*)(p)));
}

// 16 bytes per lane from global memory straight into LDS, lane i's bytes at
// lds_base + 16 i (global_load_lds_dwordx4; M0 holds the wave's LDS base).
// Issued through inline assembly so that the compiler does not track it: a
// tracked LDS DMA makes the compiler put a wait for *all* outstanding vector
// memory accesses (vmcnt(0)) in front of every later LDS read, which would
// drain every prefetch.  Callers wait for these loads with explicit
// s_waitcnt vmcnt, and order them against LDS reads of the same bytes.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_base) : "memory");
}
// The same from a wave-uniform base (SGPRs) plus a per-lane 32-bit byte
// offset: the address arithmetic that depends on the page stays scalar.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voffset, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voffset), "s"(sbase), "{m0}"(lds_base) : "memory");
}
// The same with 4 bytes per lane (lane i's dword at lds_base + 4 i).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(gptr), "{m0}"(lds_base) : "memory");
}

// Cross-lane steps without LDS: DPP inside rows of 16 lanes, and gfx950's
// v_permlane16_swap / v_permlane32_swap across rows.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8

// a[l] + a[l ^ 16] in every lane l.
__device__ __forceinline__ float add_xor16(float a) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// a[l] + a[l ^ 32] in every lane l.
__device__ __forceinline__ float add_xor32(float a) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float a) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float a) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppRor4>(v));
  v = fmaxf(v, dpp<kDppRor8>(v));
  return max_xor32(max_xor16(v));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppRor4>(v);
  v += dpp<kDppRor8>(v);
  return add_xor32(add_xor16(v));
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Which pages at the start of each sequence a stream walk skips (all
// fields optional; the first that is given decides).
struct PageSkip {
  const int32_t* begin_pages = nullptr;  // per sequence: the first page to walk (cascade: after the prefix)
  int window = 0;                        // sliding window in tokens (0 = none)
};

// First page a sequence's walk covers: begin_pages[s] when given; else, in
// a mixed batch (cu_q = its cumulative query counts), past the end for a
// segment of more than one query token (a prefill chunk, which the tile
// kernel attends) and 0 for a decode token; else the page of the first row
// inside a sliding window (0 without one).
__device__ __forceinline__ int walk_begin(const PageSkip& k, const int32_t* __restrict__ cu_q, int s, int L) {
  if (k.begin_pages) return k.begin_pages[s];
  if (cu_q) return cu_q[s + 1] - cu_q[s] > 1 ? (L + 15) >> 4 : 0;
  return k.window > 0 && L > k.window ? (L - k.window) >> 4 : 0;
}

// Splits of C pages that sequence s needs over pages [begin, pages).
__device__ __forceinline__ int nsplit_of(int L, int begin_pages, int max_blocks, int C) {
  const int64_t pg = (static_cast<int64_t>(L) + 15) >> 4;
  const int pages = static_cast<int>(pg < max_blocks ? pg : max_blocks);
  const int n = pages - begin_pages;
  return n > 0 ? (n + C - 1) / C : 0;
}

struct ItemLoc {
  int s;     // sequence
  int j;     // split index within the sequence
  int ns;    // splits of the sequence
  int base;  // index of the sequence's first item
  int total; // items over all sequences
};

// Work item x -> (sequence, split).  Items are numbered sequence by
// sequence; every wave derives the numbering itself from the device copy
// of the context lengths (one pass over S values, then one over the
// S/64 values of the lane that holds x), so no plan buffer is needed.
// `skip` and `cu_q` (nullable) decide the pages each sequence skips
// (walk_begin).  `trim` rows
// are taken off the end of every context (a multi-token pass that stops
// before a sequence's last new tokens).
__device__ __forceinline__ bool locate_item(const int32_t* __restrict__ ctx, const PageSkip& skip,
                                            const int32_t* __restrict__ cu_q, int S, int max_blocks, int C, int x, ItemLoc& loc,
                                            int trim = 0) {
  const int lane = lane_id();
  const int per = (S + 63) >> 6;
  int tot = 0;
  // Unrolled with clamped indices so that eight independent loads are in
  // flight at once instead of one load-use chain per sequence.
#pragma unroll 8
  for (int i = 0; i < per; ++i) {
    const int s = lane * per + i;
    const int sc = s < S ? s : S - 1;
    const int Lc = ctx[sc] - trim;
    const int n = nsplit_of(Lc, walk_begin(skip, cu_q, sc, Lc), max_blocks, C);
    tot += s < S ? n : 0;
  }
  const int incl = wave_inclusive_scan(tot);
  const int excl = incl - tot;
  loc.total = __shfl(incl, 63, 64);
  const unsigned long long b = __ballot(x >= excl && x < incl);
  if (b == 0ull) return false;
  const int l = __ffsll(b) - 1;
  int base = __shfl(excl, l, 64);
  const int first = l * per;
  for (int r0 = 0; r0 < per; r0 += 64) {
    const int i = r0 + lane;
    const int s = first + i;
    int ns = 0;
    if (i < per && s < S) {
      const int Ls = ctx[s] - trim;
      ns = nsplit_of(Ls, walk_begin(skip, cu_q, s, Ls), max_blocks, C);
    }
    const int inc2 = wave_inclusive_scan(ns);
    const int ex2 = inc2 - ns;
    const unsigned long long b2 = __ballot(ns > 0 && x >= base + ex2 && x < base + inc2);
    if (b2 != 0ull) {
      const int l2 = __ffsll(b2) - 1;
      loc.s = first + r0 + l2;
      loc.ns = __shfl(ns, l2, 64);
      loc.base = base + __shfl(ex2, l2, 64);
      loc.j = x - loc.base;
      return true;
    }
    base += __shfl(inc2, 63, 64);
  }
  return false;
}

// Log-sum-exp merge of n partials (a normalised o row of D elements and its
// log2-sum-exp) for the G heads of one kv-head, this lane's EPL = D / 64
// elements of each row.  lse_at(j, h) gives partial j's log2-sum-exp for
// head h, load_row(j, h, v) this lane's EPL elements of its row.  Partials
// are taken J at a time, their sums and rows loaded together (one round
// trip per J partials, all heads at once), with a running maximum M: a
// partial with lse = -inf weighs 0, and with all n partials in one step
// the result is that of a max pass followed by a sum pass.  The state (M,
// wsum, acc) carries over, so partials of different kinds can be merged by
// successive calls; merge_init sets it up.
template <int G, int D>
__device__ __forceinline__ void merge_init(float (&M)[G], float (&wsum)[G], float (&acc)[G][D / 64]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = -INFINITY;
    wsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc[h][e] = 0.f;
  }
}
// Elements 2 lane, 2 lane + 1 of a bf16 row, widened to float32 (exact).
__device__ __forceinline__ void load_bf16_pair(const uint16_t* row, int lane, float (&v)[2]) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(row + 2 * lane);
  v[0] = bf16_lo(w);
  v[1] = bf16_hi(w);
}
// Partials per step of merge_partials for G rows of D elements.
constexpr int merge_step(int G, int D) { return G * (D / 64) >= 32 ? 1 : 32 / (G * (D / 64)); }
template <int G, int D, typename LseAt, typename LoadRow>
__device__ __forceinline__ void merge_partials(int n, LseAt lse_at, LoadRow load_row, float (&M)[G], float (&wsum)[G],
                                               float (&acc)[G][D / 64]) {
  constexpr int EPL = D / 64;
  constexpr int J = merge_step(G, D);
  for (int j0 = 0; j0 < n; j0 += J) {
    float l[J][G];
    float v[J][G][EPL];
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      const int j = j0 + jj;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (j < n) {
          l[jj][h] = lse_at(j, h);
          load_row(j, h, v[jj][h]);
        } else {
          l[jj][h] = -INFINITY;
#pragma unroll
          for (int e = 0; e < EPL; ++e) v[jj][h][e] = 0.f;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mn = M[h];
#pragma unroll
      for (int jj = 0; jj < J; ++jj) mn = fmaxf(mn, l[jj][h]);
      if (mn == -INFINITY) continue;  // nothing but empty partials so far
      const float alpha = fast_exp2(M[h] - mn);  // M = -inf: 0
      wsum[h] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int jj = 0; jj < J; ++jj) {
        const float a = fast_exp2(l[jj][h] - mn);  // -inf (no visible key) -> 0
        wsum[h] += a;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(a, v[jj][h][e], acc[h][e]);
      }
      M[h] = mn;
    }
  }
}

}  // namespace pa
