// Internal interface between the C-ABI layer (pa_api.cpp), the host-side
// planner/validator (pa_host.cpp) and the HIP kernels (pa_decode.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "pa.h"

namespace pa {

constexpr int kBlockSize = 16;      // rows per page: the only page size built
constexpr int kBatchPages = 4;      // pages one wave consumes per iteration (64 rows)
constexpr int kMinSplitPages = 8;   // smallest automatic split, in pages
constexpr int kTargetWaves = 4096;  // automatic splits aim at about this many waves
constexpr size_t kAlign = 256;

// Error reporting: thread-local message + code.
int fail(int code, const std::string& msg);
void clear_error();

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Number of splits sequence s needs, from its page count after `begin_pages`.
inline int64_t splits_for(int64_t pages, int64_t begin_pages, int64_t split_pages) {
  const int64_t n = pages - begin_pages;
  return n > 0 ? (n + split_pages - 1) / split_pages : 0;
}

// Split size chosen from the batch when the caller passes 0.
int32_t auto_split_pages(int64_t total_pages, int32_t num_kv_heads);

// Workspace carve-up for the split-KV partials.
struct PartialLayout {
  size_t o_offset, lse_offset, bytes;
};
PartialLayout partial_layout(int64_t items, int32_t num_kv_heads, int32_t gqa, int32_t head_dim);
// Largest item count whose partials fit in `bytes`.
int64_t capacity_items(size_t bytes, int32_t num_kv_heads, int32_t gqa, int32_t head_dim);

// Everything the decode launcher needs; all pointers already validated.
struct DecodeLaunch {
  void* out;
  float* lse_out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t gqa;
  int32_t head_dim;
  int64_t num_pages;
  float scale;
  pa_dtype dtype;
  int32_t split_pages;
  int64_t items;      // total (sequence, split) work items, from the host copy
  int64_t capacity;   // partial slots the workspace holds (items index them)
  bool any_multi;     // some sequence has more than one split
  float* part_o;      // workspace partial outputs [items, Hkv, G, D]
  float* part_lse;    // workspace partial log2-sum-exp [items, Hkv, G]
  void* stream;
};

bool decode_supported(pa_dtype dtype, int32_t head_dim, int32_t gqa);
int launch_decode(const DecodeLaunch& a);

// Profiling hook: bracket the dominant kernel of a call.
void profile_before(void* stream);
void profile_after(void* stream);

}  // namespace pa
