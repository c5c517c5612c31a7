// Internal interface between the C-ABI layer (pa_api.cpp), the host-side
// planner/validator (pa_host.cpp) and the HIP kernels (pa_decode.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "pa.h"

namespace pa {

constexpr int kBlockSize = 16;            // rows per page: the only page size built
constexpr int kMinPagesPerWave = 4;       // automatic runs are at least one 4-page batch
constexpr int kMaxResidentWaves = 16384;  // bound on waves resident on one GPU (sizes workspace)
constexpr int kMaxPrefixSplits = 8;       // key splits of a shared prefix (sizes workspace)
constexpr int kPrefixRowsPerBlock = 128;  // query rows one MFMA tile workgroup takes
#ifndef PA_TILE_WG_PER_CU
#define PA_TILE_WG_PER_CU 2
#endif
constexpr int kTileWorkgroupsPerCU = PA_TILE_WG_PER_CU;  // MFMA tile workgroups resident per CU
#ifndef PA_TILE_FP8_WG_PER_CU
#define PA_TILE_FP8_WG_PER_CU 2
#endif
constexpr int kTileFp8WorkgroupsPerCU = PA_TILE_FP8_WG_PER_CU;  // the same over fp8 pools (half the LDS)
constexpr size_t kAlign = 256;
// Automatic plans of the matrix-core stream over bf16 pools: the even wave
// of each pair (2j, 2j + 1) takes this many thousandths of `per` pages
// more, the odd one as many fewer.  Under a full streaming load the XCDs
// of an MI355X (workgroup i runs on XCD i mod 8) do not stream equally
// fast: in most per-wave timelines of the Llama-shaped, long-tail and
// cascade-suffix batches the odd XCDs were 4-9 % slower, so equal runs
// left the even XCDs idle at the end (other runs split the XCDs into other
// halves; there the lead only moves work inside equally fast pairs).
// Leads of 35 and 60 took 1-1.5 % off the Llama-shaped and long-tail
// kernels; over fp8 pools (half the bytes per page) they were 2-3 %
// slower, so those keep equal runs.
#ifndef PA_RUN_LEAD_PERMILLE
#define PA_RUN_LEAD_PERMILLE 50
#endif
constexpr int kRunLeadPermille = PA_RUN_LEAD_PERMILLE;
inline int32_t run_lead(int64_t per) {
  const int64_t l = (per * kRunLeadPermille + 500) / 1000;
  return static_cast<int32_t>(l < per ? l : per - 1);
}

// Error reporting: thread-local message + code.
int fail(int code, const std::string& msg);
void clear_error();

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace carve-up: per-sequence records (first wave, last wave, slot of
// the first wave) written by the stream kernel for the merge kernel, then
// two partial slots per (wave, kv-head): log2-sum-exp and output rows.
struct PartialLayout {
  size_t info_offset, lse_offset, o_offset, bytes;
};
PartialLayout partial_layout(int64_t waves, int64_t num_seqs, int32_t num_kv_heads, int32_t gqa, int32_t head_dim);
// Query rows per wave (and partial rows per wave and kv-head) of the
// stream kernel for `rows` rows of work: 4 or more run on the matrix-core
// kernel's 16 rows (bf16 q; float32 uses fewer, so sizing by this is
// enough for every type).
inline int32_t stream_rows(int32_t rows) { return rows >= 4 ? 16 : rows; }

// Waves per kv-head the decode planner may use for a batch of total_pages
// pages: split_pages > 0 fixes the run length, 0 lets the launcher size runs
// so the resident waves of the GPU are filled once.
int64_t max_waves_per_head(int64_t total_pages, int32_t num_kv_heads, int32_t split_pages);

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
  int32_t split_pages;  // pages per wave run; 0 = automatic
  int64_t total_pages;  // sum over sequences of ceil(L / 16), from the host copy
  void* workspace;
  size_t workspace_bytes;
  void* stream;
  bool timed = true;  // record profiling events around the stream kernel
  // fp8 pools: e4m3fn codes with one float32 scale per (page, kv-head,
  // slot); q and out are then bf16 (dtype == PA_BF16)
  bool kv_fp8 = false;
  const float* k_scales = nullptr;
  const float* v_scales = nullptr;
  // sliding window in tokens (0 = full history); total_pages then counts
  // only the pages from each window's first page on
  int32_t window = 0;
};

// Multi-token decode: q_len new tokens per sequence, causal among them.
// `fold` tokens of every sequence share one pass over its pages, their
// (token, head) rows folded into the wave's query rows (`rows`, the power
// of two >= gqa * fold); passes = ceil(q_len / fold), pass p covering
// tokens p*fold .. and walking each context up to its last token.  The
// workspace is sized for multi_ws_rows partial rows per wave.
constexpr int kMaxFoldRows = 16;  // query rows one wave holds
struct MultiPlan {
  int32_t q_len = 1;
  int32_t fold = 1;
  int32_t rows = 1;
  int32_t passes = 1;
  std::vector<int64_t> pass_pages;  // pages each pass walks (from the host copy of the lengths)
};
// fold, rows and passes only (no lengths): what sizes the workspace.
MultiPlan plan_multi_shape(int32_t q_len, int32_t gqa);
MultiPlan plan_multi(int32_t q_len, int32_t gqa, const int32_t* context_lens_host, int32_t num_seqs,
                     int32_t block_size, int32_t window = 0);
int launch_decode_multi(const DecodeLaunch& a, const MultiPlan& p);
// Partial rows per wave a multi-token call's workspace holds: the stream
// kernel's for one token; 16 for folded passes (every fp8 pass, and bf16
// passes of 4 or more rows, run on the matrix-core kernel's 16 rows).
inline int32_t multi_ws_rows(int32_t q_len, int32_t gqa) { return q_len > 1 ? 16 : stream_rows(gqa); }
bool decode_supported(pa_dtype dtype, int32_t head_dim, int32_t gqa);
// Validation, planning and launch shared by the decode entry points.  With
// plan_sized the workspace is checked against the plan actually made (a
// fixed-size scratch buffer) instead of the largest plan the batch could get.
int decode_call(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                const float* k_scales, const float* v_scales, bool kv_fp8, const int32_t* block_tables,
                int32_t max_blocks, const int32_t* context_lens, const int32_t* context_lens_host, int32_t num_seqs,
                int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim, int32_t block_size, int64_t num_pages,
                float scale, pa_dtype dtype, int32_t split_pages, void* workspace, size_t workspace_bytes,
                void* stream, int32_t window, int32_t q_len, const char* who, bool plan_sized = false);
bool decode_fp8_supported(int32_t head_dim, int32_t gqa);
int launch_decode(const DecodeLaunch& a);

// The stream kernel alone (plus, if `merge`, its merge kernel).  With
// begin_pages (device, per sequence) only pages from there on are walked;
// with seq_part, sequences one wave covers are written there as partials
// (bf16 rows [S][Hq][D], then float32 log2-sum-exps from float S Hq D on)
// instead of to `out`.  The plan actually used comes back in *plan.
struct StreamPlan {
  int64_t waves;
  int32_t per;
  int32_t rows;          // partial rows per (wave, kv-head, slot)
  PartialLayout layout;  // inside a.workspace
};
// q_rows (device, per sequence, nullable) gives the q / out / lse row of
// each sequence when the batch holds more than one token per sequence.
int launch_stream(const DecodeLaunch& a, const int32_t* begin_pages, float* seq_part, const int32_t* q_rows,
                  bool merge, StreamPlan* plan);

// The merge of a matrix-core stream launch (16 partial rows per wave,
// bf16, head_dim 128) over `waves` runs per kv-head; q_rows as launch_stream.
int launch_stream_merge(const DecodeLaunch& a, const int32_t* q_rows, int64_t waves);

// Prefill chunks of a mixed batch, passed by value to the MFMA tile kernel.
constexpr int32_t kMaxChunkSplits = 8;  // key splits of one chunk (sizes workspace)
constexpr int32_t kMinChunkSplitKeys = 1024;
constexpr int kMaxChunkSegments = 64;
struct ChunkList {
  int32_t n;                                // chunk segments (q_len > 1)
  int32_t seg[kMaxChunkSegments];           // their segment indices
  int32_t tok_off[kMaxChunkSegments + 1];   // first chunk-token index of each
  int32_t nks[kMaxChunkSegments];           // key splits of each
  int32_t kps[kMaxChunkSegments];           // keys per split (a multiple of 64)
  int32_t rec[kMaxChunkSegments];           // first partial record (token, kv-head, split) of each
  int32_t ord[kMaxChunkSegments];           // launch order: ord[j] is the j-th chunk launched
  int32_t item_end[kMaxChunkSegments];      // work items (kv-head, split) of launch-order chunks 0..j
};

// Key splits of the prefill chunks: each chunk's keys are cut into splits
// so that one workgroup (a row block against one split) streams about
// total tiles / (CUs * kChunkWorkgroupsPerCU) tiles of 64 keys, and no
// fewer than kMinChunkSplitKeys keys; at most kMaxChunkSplits splits.
#ifndef PA_CHUNK_WG_PER_CU
#define PA_CHUNK_WG_PER_CU 3
#endif
constexpr int kChunkWorkgroupsPerCU = PA_CHUNK_WG_PER_CU;
// In the one-launch mixed kernel the chunk workgroups share the CUs with
// the decode waves: fewer, longer chunk workgroups (one per CU's worth of
// splits) measured faster there (chunked_piggyback 862-864 against 868-876
// us at 3, fp8 629-631 against 640-646 us; 2, 5 and 8 slower), while chunks
// launched on their own keep 3.
#ifndef PA_MIXED_CHUNK_WG_PER_CU
#define PA_MIXED_CHUNK_WG_PER_CU 1
#endif
constexpr int kMixedChunkWorkgroupsPerCU = PA_MIXED_CHUNK_WG_PER_CU;
// The mixed batch runs as one launch (mixed_kernel) when built so, with 4
// or more q-heads per kv-head, decode tokens present and at most
// kMaxChunkSegments chunks; otherwise the chunk tiles and the decode stream
// run one after the other.
#ifndef PA_MIXED_ONE_LAUNCH
#define PA_MIXED_ONE_LAUNCH 1
#endif
inline bool mixed_one_launch(int32_t gqa, int64_t decode_pages, int32_t num_chunks) {
  return PA_MIXED_ONE_LAUNCH && gqa >= 4 && decode_pages > 0 && num_chunks <= kMaxChunkSegments;
}
struct ChunkPlan {
  std::vector<int32_t> nks, kps, rec;
  std::vector<int32_t> tiles;  // tiles of 64 keys per work item (launch order: most first)
  int64_t records = 0;         // partial records (token, kv-head, split) of all chunks
};
ChunkPlan plan_chunks(const std::vector<int32_t>& n_tok, const std::vector<int32_t>& keys, int32_t gqa,
                      int32_t num_kv_heads, int32_t cus,
                      int32_t wg_per_cu);
// Compute units of the current device (0 if the query fails).
int device_cu_count();

// Shared-prefix (cascade) decode.
struct CascadeLayout {
  size_t begin_offset, seq_part_offset, pre_o_offset, pre_lse_offset, stream_offset, bytes;
};
CascadeLayout cascade_layout(int64_t num_seqs, int32_t num_kv_heads, int32_t gqa, int32_t head_dim, int32_t nks,
                             int64_t stream_bytes);
struct CascadeLaunch {
  DecodeLaunch base;             // out, q, pools, tables, lengths, shapes, stream
  const int32_t* group_offsets;  // device [NG+1]
  const int32_t* prefix_lens;    // device [NG]
  int32_t num_groups;
  int32_t row_chunks;  // ceil(max group rows / kPrefixRowsPerBlock)
  int32_t nks;         // key splits per prefix
  int32_t kps;         // keys per split (multiple of 64)
  int64_t suffix_pages;
  CascadeLayout layout;
  void* workspace;
  size_t workspace_bytes;
};
bool cascade_supported(pa_dtype dtype, int32_t head_dim, int32_t gqa);
int launch_cascade(const CascadeLaunch& c);

// Mixed batch: prefill chunks (q_len > 1, causal inside the chunk) and
// decode tokens (q_len = 1) of many sequences in one call.
struct MixedLayout {
  size_t begin_offset, pre_o_offset, pre_lse_offset, stream_offset, bytes;
};
MixedLayout mixed_layout(int64_t num_seqs, int64_t chunk_tokens, int32_t num_kv_heads, int32_t gqa, int32_t head_dim,
                         int32_t nks, int64_t stream_bytes);
struct MixedLaunch {
  DecodeLaunch base;         // num_seqs = segments; out / q rows are tokens
  const int32_t* cu_q_lens;  // device [S+1]
  const int32_t* chunk_seg;  // host [num_chunks]: segments with q_len > 1
  const int32_t* chunk_tok;  // host [num_chunks+1]: first chunk-token index of each
  int32_t num_chunks;
  int32_t row_chunks;  // ceil(max chunk rows / kPrefixRowsPerBlock)
  const ChunkPlan* plan;  // key splits of each chunk
  int64_t decode_pages;
  MixedLayout layout;
  void* workspace;
  size_t workspace_bytes;
};
bool mixed_supported(pa_dtype dtype, int32_t head_dim, int32_t gqa);
int launch_mixed(const MixedLaunch& m);

// KV append.
constexpr int64_t kMaxAppendRowBytes = 512;  // head_dim * element size
struct AppendLaunch {
  void* k_pool;
  void* v_pool;
  const void* k_new;
  const void* v_new;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* cu_q_lens;     // device [S+1]
  const int32_t* context_lens;  // device [S]
  int32_t num_segments;
  int64_t num_tokens;
  int32_t num_kv_heads;
  int32_t row_bytes;  // head_dim * element size, a multiple of 16
  int64_t num_pages;
  void* stream;
};
int launch_append(const AppendLaunch& a);

// KV append into an fp8 cache (codes + one float32 scale per row).
struct AppendFp8Launch {
  void* k_pool;  // [NP, Hkv, 16, D] e4m3fn codes
  void* v_pool;
  float* k_scales;  // [NP, Hkv, 16]
  float* v_scales;
  const void* k_new;  // [T, Hkv, D] new_dtype
  const void* v_new;
  pa_dtype new_dtype;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* cu_q_lens;     // device [S+1]
  const int32_t* context_lens;  // device [S]
  int32_t num_segments;
  int64_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int64_t num_pages;
  void* stream;
};
int launch_append_fp8(const AppendFp8Launch& a);

// Profiling hook: bracket the dominant kernel of a call.
void profile_before(void* stream);
void profile_after(void* stream);

}  // namespace pa
