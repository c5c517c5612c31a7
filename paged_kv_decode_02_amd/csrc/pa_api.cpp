// C-ABI entry points: argument validation and split planning on the host,
// then the launch.  Nothing here touches device memory.
#include <algorithm>
#include <climits>
#include <string>
#include <vector>

#include "pa_internal.h"

using namespace pa;

namespace {

int check_common(const void* out, const void* q, const void* k_pool, const void* v_pool, const int32_t* bt,
                 int32_t max_blocks, const int32_t* ctx, const int32_t* ctx_host, int32_t num_kv_heads,
                 int32_t gqa, int32_t head_dim, int32_t block_size, int64_t num_pages, float scale,
                 pa_dtype dtype, const void* workspace, const char* who) {
  const std::string w(who);
  if (!out || !q || !k_pool || !v_pool || !bt || !ctx || !ctx_host || !workspace)
    return fail(PA_EINVAL, w + ": null pointer argument");
  if (max_blocks < 1 || num_kv_heads < 1 || gqa < 1 || head_dim < 1 || num_pages < 1)
    return fail(PA_EINVAL, w + ": sizes must be >= 1");
  if (!(scale == scale) || scale == 1.0f / 0.0f || scale == -1.0f / 0.0f)
    return fail(PA_EINVAL, w + ": scale is not finite");
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_EUNSUPPORTED, w + ": unknown dtype");
  if (block_size != kBlockSize) return fail(PA_EUNSUPPORTED, w + ": only block_size 16 is built");
  if (num_pages > (int64_t(1) << 31) - 1) return fail(PA_EUNSUPPORTED, w + ": num_pages above 2^31-1");
  return PA_OK;
}

}  // namespace

extern "C" size_t pa_decode_workspace_size(int32_t max_num_seqs, int32_t num_kv_heads, int32_t gqa_ratio,
                                           int32_t head_dim, int64_t max_total_pages, int32_t split_pages) {
  if (max_num_seqs < 0 || num_kv_heads < 1 || gqa_ratio < 1 || head_dim < 1 || max_total_pages < 0 ||
      split_pages < 0)
    return 0;
  const int64_t waves = max_waves_per_head(max_total_pages, num_kv_heads, split_pages);
  return partial_layout(waves, max_num_seqs, num_kv_heads, stream_rows(gqa_ratio), head_dim).bytes;
}

// pa_decode, pa_decode_window, pa_decode_fp8, pa_decode_multi and
// pa_decode_noalloc: validation, page count, workspace check, launch.
int pa::decode_call(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                    const float* k_scales, const float* v_scales, bool kv_fp8, const int32_t* block_tables,
                    int32_t max_blocks, const int32_t* context_lens, const int32_t* context_lens_host,
                    int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim, int32_t block_size,
                    int64_t num_pages, float scale, pa_dtype dtype, int32_t split_pages, void* workspace,
                    size_t workspace_bytes, void* stream, int32_t window, int32_t q_len, const char* who,
                    bool plan_sized) {
  const std::string w(who);
  if (num_seqs < 0) return fail(PA_EINVAL, w + ": num_seqs < 0");
  if (num_seqs == 0) return PA_OK;
  int rc = check_common(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, context_lens_host,
                        num_kv_heads, gqa_ratio, head_dim, block_size, num_pages, scale, dtype, workspace, who);
  if (rc) return rc;
  if (kv_fp8 && (!k_scales || !v_scales)) return fail(PA_EINVAL, w + ": null scale pointer");
  if (split_pages < 0) return fail(PA_EINVAL, w + ": split_pages < 0");
  if (window < 0) return fail(PA_EINVAL, w + ": window < 1");
  if (q_len < 1) return fail(PA_EINVAL, w + ": q_len < 1");
  const bool built = kv_fp8 ? decode_fp8_supported(head_dim, gqa_ratio) : decode_supported(dtype, head_dim, gqa_ratio);
  if (!built)
    return fail(PA_EUNSUPPORTED, w + ": no kernel for head_dim " + std::to_string(head_dim) + "/gqa_ratio " +
                                     std::to_string(gqa_ratio));
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return fail(PA_EINVAL, w + ": workspace not 256B aligned");
  int64_t total_pages = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t L = context_lens_host[s];
    if (L < 1) return fail(PA_EINVAL, w + ": context_lens[" + std::to_string(s) + "] < 1");
    if (L < q_len) return fail(PA_EINVAL, w + ": context_lens[" + std::to_string(s) + "] < q_len");
    if (L > static_cast<int64_t>(max_blocks) * block_size)
      return fail(PA_EINVAL, w + ": context_lens[" + std::to_string(s) + "] exceeds the block table");
    // pages the walk covers: from the first page of the earliest token's
    // window on (a sliding window's earlier entries are placeholders and
    // are never read)
    const int64_t reach = window > 0 ? static_cast<int64_t>(window) + q_len - 1 : 0;
    const int64_t first = reach > 0 && L > reach ? (L - reach) / block_size : 0;
    total_pages += (L + block_size - 1) / block_size - first;
  }
  if (total_pages > (int64_t(1) << 31) - 1) return fail(PA_EUNSUPPORTED, w + ": more than 2^31-1 pages");
  // The workspace must hold the largest plan this batch could get, so that
  // a call never depends on the occupancy the device reports.
  // (multi-token passes keep `rows` query rows per wave; the last pass
  // walks every page)
  // (plan_sized: a fixed scratch buffer is checked against the plan the
  // launcher actually makes instead, before anything is launched)
  const int32_t rows = multi_ws_rows(q_len, gqa_ratio);
  const PartialLayout worst = partial_layout(max_waves_per_head(total_pages, num_kv_heads, split_pages), num_seqs,
                                             num_kv_heads, rows, head_dim);
  if (!plan_sized && worst.bytes > workspace_bytes)
    return fail(PA_EWORKSPACE, w + ": workspace holds " + std::to_string(workspace_bytes) + " bytes, needs " +
                                   std::to_string(worst.bytes));
  DecodeLaunch a;
  a.out = out;
  a.lse_out = lse_out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks = max_blocks;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.gqa = gqa_ratio;
  a.head_dim = head_dim;
  a.num_pages = num_pages;
  a.scale = scale;
  a.dtype = dtype;
  a.split_pages = split_pages;
  a.total_pages = total_pages;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.stream = stream;
  a.kv_fp8 = kv_fp8;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.window = window;
  if (q_len == 1) return launch_decode(a);
  return launch_decode_multi(a, plan_multi(q_len, gqa_ratio, context_lens_host, num_seqs, block_size, window));
}

extern "C" int pa_decode(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                         const int32_t* context_lens_host, int32_t num_seqs, int32_t num_kv_heads,
                         int32_t gqa_ratio, int32_t head_dim, int32_t block_size, int64_t num_pages, float scale,
                         pa_dtype dtype, int32_t split_pages, void* workspace, size_t workspace_bytes,
                         void* stream) {
  clear_error();
  return decode_call(out, lse_out, q, k_pool, v_pool, nullptr, nullptr, false, block_tables, max_blocks, context_lens,
                     context_lens_host, num_seqs, num_kv_heads, gqa_ratio, head_dim, block_size, num_pages, scale,
                     dtype, split_pages, workspace, workspace_bytes, stream, 0, 1, "pa_decode");
}

extern "C" int pa_decode_window(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                                const int32_t* context_lens_host, int32_t num_seqs, int32_t num_kv_heads,
                                int32_t gqa_ratio, int32_t head_dim, int32_t block_size, int64_t num_pages,
                                float scale, pa_dtype dtype, int32_t window, int32_t split_pages, void* workspace,
                                size_t workspace_bytes, void* stream) {
  clear_error();
  if (window < 1) return fail(PA_EINVAL, "pa_decode_window: window < 1");
  return decode_call(out, lse_out, q, k_pool, v_pool, nullptr, nullptr, false, block_tables, max_blocks, context_lens,
                     context_lens_host, num_seqs, num_kv_heads, gqa_ratio, head_dim, block_size, num_pages, scale,
                     dtype, split_pages, workspace, workspace_bytes, stream, window, 1, "pa_decode_window");
}

extern "C" int pa_decode_fp8(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                             const float* k_scales, const float* v_scales, const int32_t* block_tables,
                             int32_t max_blocks, const int32_t* context_lens, const int32_t* context_lens_host,
                             int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim,
                             int32_t block_size, int64_t num_pages, float scale, int32_t split_pages,
                             void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return decode_call(out, lse_out, q, k_pool, v_pool, k_scales, v_scales, true, block_tables, max_blocks,
                     context_lens, context_lens_host, num_seqs, num_kv_heads, gqa_ratio, head_dim, block_size,
                     num_pages, scale, PA_BF16, split_pages, workspace, workspace_bytes, stream, 0, 1, "pa_decode_fp8");
}

extern "C" size_t pa_decode_multi_workspace_size(int32_t max_num_seqs, int32_t q_len, int32_t num_kv_heads,
                                                 int32_t gqa_ratio, int32_t head_dim, int64_t max_total_pages,
                                                 int32_t split_pages) {
  if (max_num_seqs < 0 || q_len < 1 || num_kv_heads < 1 || gqa_ratio < 1 || head_dim < 1 || max_total_pages < 0 ||
      split_pages < 0)
    return 0;
  const int64_t waves = max_waves_per_head(max_total_pages, num_kv_heads, split_pages);
  return partial_layout(waves, max_num_seqs, num_kv_heads, multi_ws_rows(q_len, gqa_ratio), head_dim).bytes;
}

extern "C" int pa_decode_multi(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                               const int32_t* context_lens_host, int32_t num_seqs, int32_t q_len,
                               int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim, int32_t block_size,
                               int64_t num_pages, float scale, pa_dtype dtype, int32_t split_pages, void* workspace,
                               size_t workspace_bytes, void* stream) {
  clear_error();
  return decode_call(out, lse_out, q, k_pool, v_pool, nullptr, nullptr, false, block_tables, max_blocks, context_lens,
                     context_lens_host, num_seqs, num_kv_heads, gqa_ratio, head_dim, block_size, num_pages, scale,
                     dtype, split_pages, workspace, workspace_bytes, stream, 0, q_len, "pa_decode_multi");
}

extern "C" int pa_decode_multi_window(void* out, float* lse_out, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_tables, int32_t max_blocks,
                                      const int32_t* context_lens, const int32_t* context_lens_host, int32_t num_seqs,
                                      int32_t q_len, int32_t window, int32_t num_kv_heads, int32_t gqa_ratio,
                                      int32_t head_dim, int32_t block_size, int64_t num_pages, float scale,
                                      pa_dtype dtype, int32_t split_pages, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  clear_error();
  if (window < 1) return fail(PA_EINVAL, "pa_decode_multi_window: window < 1");
  return decode_call(out, lse_out, q, k_pool, v_pool, nullptr, nullptr, false, block_tables, max_blocks, context_lens,
                     context_lens_host, num_seqs, num_kv_heads, gqa_ratio, head_dim, block_size, num_pages, scale,
                     dtype, split_pages, workspace, workspace_bytes, stream, window, q_len, "pa_decode_multi_window");
}

extern "C" int pa_decode_multi_fp8(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                                   const float* k_scales, const float* v_scales, const int32_t* block_tables,
                                   int32_t max_blocks, const int32_t* context_lens, const int32_t* context_lens_host,
                                   int32_t num_seqs, int32_t q_len, int32_t num_kv_heads, int32_t gqa_ratio,
                                   int32_t head_dim, int32_t block_size, int64_t num_pages, float scale,
                                   int32_t split_pages, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return decode_call(out, lse_out, q, k_pool, v_pool, k_scales, v_scales, true, block_tables, max_blocks,
                     context_lens, context_lens_host, num_seqs, num_kv_heads, gqa_ratio, head_dim, block_size,
                     num_pages, scale, PA_BF16, split_pages, workspace, workspace_bytes, stream, 0, q_len,
                     "pa_decode_multi_fp8");
}

extern "C" size_t pa_prefix_cascade_workspace_size(int32_t max_num_seqs, int32_t num_kv_heads, int32_t gqa_ratio,
                                                   int32_t head_dim, int64_t max_total_pages) {
  if (max_num_seqs < 0 || num_kv_heads < 1 || gqa_ratio < 1 || head_dim < 1 || max_total_pages < 0) return 0;
  const int64_t waves = max_waves_per_head(max_total_pages, num_kv_heads, 0);
  const size_t stream = partial_layout(waves, max_num_seqs, num_kv_heads, stream_rows(gqa_ratio), head_dim).bytes;
  return cascade_layout(max_num_seqs, num_kv_heads, gqa_ratio, head_dim, kMaxPrefixSplits, stream).bytes;
}

namespace {

// pa_prefix_cascade and pa_prefix_cascade_fp8: validation, plans, launch.
int cascade_call(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                 const float* k_scales, const float* v_scales, bool kv_fp8, const int32_t* block_tables,
                 int32_t max_blocks, const int32_t* context_lens, const int32_t* context_lens_host, int32_t num_seqs,
                 int32_t num_groups, const int32_t* group_seq_offsets, const int32_t* group_seq_offsets_host,
                 const int32_t* prefix_lens, const int32_t* prefix_lens_host, int32_t num_kv_heads, int32_t gqa_ratio,
                 int32_t head_dim, int32_t block_size, int64_t num_pages, float scale, pa_dtype dtype,
                 void* workspace, size_t workspace_bytes, void* stream, const char* who) {
  const std::string w(who);
  if (num_seqs < 0 || num_groups < 0) return fail(PA_EINVAL, w + ": negative count");
  if (num_seqs == 0) return PA_OK;
  int rc = check_common(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, context_lens_host,
                        num_kv_heads, gqa_ratio, head_dim, block_size, num_pages, scale, dtype, workspace, who);
  if (rc) return rc;
  if (kv_fp8 && (!k_scales || !v_scales)) return fail(PA_EINVAL, w + ": null scale pointer");
  if (num_groups < 1 || !group_seq_offsets || !group_seq_offsets_host || !prefix_lens || !prefix_lens_host)
    return fail(PA_EINVAL, w + ": groups must be given (device and host copies)");
  if (!cascade_supported(dtype, head_dim, gqa_ratio))
    return fail(PA_EUNSUPPORTED, w + ": built for bf16 q, head_dim 128, gqa_ratio 1/2/4/8/16");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(PA_EINVAL, w + ": workspace not 256B aligned");
  if (group_seq_offsets_host[0] != 0 || group_seq_offsets_host[num_groups] != num_seqs)
    return fail(PA_EINVAL, w + ": groups must cover sequences 0 .. num_seqs-1 in order");
  int64_t suffix_pages = 0;
  int64_t max_rows = 0;
  int32_t max_prefix = 0;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t a = group_seq_offsets_host[g], b = group_seq_offsets_host[g + 1];
    if (b < a) return fail(PA_EINVAL, w + ": group offsets decrease");
    const int32_t P = prefix_lens_host[g];
    if (P < 0 || P % block_size)
      return fail(PA_EINVAL, w + ": prefix_lens[" + std::to_string(g) + "] not a whole number of pages");
    max_prefix = std::max(max_prefix, P);
    max_rows = std::max<int64_t>(max_rows, static_cast<int64_t>(b - a) * gqa_ratio);
    for (int32_t s = a; s < b; ++s) {
      const int64_t L = context_lens_host[s];
      if (L < 1) return fail(PA_EINVAL, w + ": context_lens[" + std::to_string(s) + "] < 1");
      if (L > static_cast<int64_t>(max_blocks) * block_size)
        return fail(PA_EINVAL, w + ": context_lens[" + std::to_string(s) + "] exceeds the block table");
      if (P >= L)
        return fail(PA_EINVAL, w + ": prefix of group " + std::to_string(g) +
                                   " is not shorter than sequence " + std::to_string(s));
      suffix_pages += (L + block_size - 1) / block_size - P / block_size;
    }
  }
  if (suffix_pages > (int64_t(1) << 31) - 1) return fail(PA_EUNSUPPORTED, w + ": too many pages");
  // Prefix plan: two tile workgroups fit on a CU (66 KB of LDS each), so aim
  // at about two per CU (row blocks x key splits), each split a 64-key
  // multiple of the prefix; key splits only when the row blocks alone leave
  // workgroup slots idle.
  const int32_t row_chunks =
      static_cast<int32_t>(std::max<int64_t>(1, (max_rows + kPrefixRowsPerBlock - 1) / kPrefixRowsPerBlock));
  const int64_t units = static_cast<int64_t>(num_groups) * row_chunks * num_kv_heads;
  const int cus = device_cu_count();
  const int64_t slots = static_cast<int64_t>(kv_fp8 ? kTileFp8WorkgroupsPerCU : kTileWorkgroupsPerCU) * (cus > 0 ? cus : 256);
  int32_t nks =
      static_cast<int32_t>(std::min<int64_t>(kMaxPrefixSplits, std::max<int64_t>(1, (slots + units - 1) / units)));
  int32_t kps = 64;
  if (max_prefix > 0) {
    kps = (max_prefix + nks - 1) / nks;
    kps = (kps + 63) / 64 * 64;
    nks = (max_prefix + kps - 1) / kps;
  } else {
    nks = 1;
  }
  const int64_t waves = max_waves_per_head(suffix_pages, num_kv_heads, 0);
  const size_t stream_bytes = partial_layout(waves, num_seqs, num_kv_heads, stream_rows(gqa_ratio), head_dim).bytes;
  const CascadeLayout lay = cascade_layout(num_seqs, num_kv_heads, gqa_ratio, head_dim, nks, stream_bytes);
  if (lay.bytes > workspace_bytes)
    return fail(PA_EWORKSPACE, w + ": workspace holds " + std::to_string(workspace_bytes) +
                                   " bytes, needs " + std::to_string(lay.bytes));
  CascadeLaunch c;
  DecodeLaunch& a = c.base;
  a.out = out;
  a.lse_out = lse_out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks = max_blocks;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.gqa = gqa_ratio;
  a.head_dim = head_dim;
  a.num_pages = num_pages;
  a.scale = scale;
  a.dtype = dtype;
  a.split_pages = 0;
  a.total_pages = suffix_pages;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  a.stream = stream;
  a.kv_fp8 = kv_fp8;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  c.group_offsets = group_seq_offsets;
  c.prefix_lens = prefix_lens;
  c.num_groups = num_groups;
  c.row_chunks = row_chunks;
  c.nks = nks;
  c.kps = kps;
  c.suffix_pages = suffix_pages;
  c.layout = lay;
  c.workspace = workspace;
  c.workspace_bytes = workspace_bytes;
  return launch_cascade(c);
}

}  // namespace

extern "C" int pa_prefix_cascade(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                                 const int32_t* context_lens_host, int32_t num_seqs, int32_t num_groups,
                                 const int32_t* group_seq_offsets, const int32_t* group_seq_offsets_host,
                                 const int32_t* prefix_lens, const int32_t* prefix_lens_host, int32_t num_kv_heads,
                                 int32_t gqa_ratio, int32_t head_dim, int32_t block_size, int64_t num_pages,
                                 float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  clear_error();
  return cascade_call(out, lse_out, q, k_pool, v_pool, nullptr, nullptr, false, block_tables, max_blocks,
                      context_lens, context_lens_host, num_seqs, num_groups, group_seq_offsets,
                      group_seq_offsets_host, prefix_lens, prefix_lens_host, num_kv_heads, gqa_ratio, head_dim,
                      block_size, num_pages, scale, dtype, workspace, workspace_bytes, stream, "pa_prefix_cascade");
}

extern "C" int pa_prefix_cascade_fp8(void* out, float* lse_out, const void* q, const void* k_pool,
                                     const void* v_pool, const float* k_scales, const float* v_scales,
                                     const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                                     const int32_t* context_lens_host, int32_t num_seqs, int32_t num_groups,
                                     const int32_t* group_seq_offsets, const int32_t* group_seq_offsets_host,
                                     const int32_t* prefix_lens, const int32_t* prefix_lens_host,
                                     int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim, int32_t block_size,
                                     int64_t num_pages, float scale, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  clear_error();
  return cascade_call(out, lse_out, q, k_pool, v_pool, k_scales, v_scales, true, block_tables, max_blocks,
                      context_lens, context_lens_host, num_seqs, num_groups, group_seq_offsets,
                      group_seq_offsets_host, prefix_lens, prefix_lens_host, num_kv_heads, gqa_ratio, head_dim,
                      block_size, num_pages, scale, PA_BF16, workspace, workspace_bytes, stream,
                      "pa_prefix_cascade_fp8");
}

extern "C" size_t pa_mixed_chunk_workspace_size(int32_t max_num_tokens, int32_t max_num_segments,
                                                int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim,
                                                int64_t max_total_pages) {
  if (max_num_tokens < 0 || max_num_segments < 0 || num_kv_heads < 1 || gqa_ratio < 1 || head_dim < 1 ||
      max_total_pages < 0)
    return 0;
  const int64_t waves = max_waves_per_head(max_total_pages, num_kv_heads, 0);
  const size_t stream =
      partial_layout(waves, max_num_segments, num_kv_heads, stream_rows(gqa_ratio), head_dim).bytes;
  return mixed_layout(max_num_segments, max_num_tokens, num_kv_heads, gqa_ratio, head_dim, kMaxChunkSplits, stream)
      .bytes;
}

namespace {

int mixed_call(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
               const float* k_scales, const float* v_scales, bool kv_fp8, const int32_t* block_tables,
               int32_t max_blocks, const int32_t* cu_q_lens, const int32_t* cu_q_lens_host,
               const int32_t* context_lens, const int32_t* context_lens_host, int32_t num_segments,
               int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim, int32_t block_size, int64_t num_pages,
               float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream, const char* who) {
  const std::string w(who);
  if (num_segments < 0) return fail(PA_EINVAL, w + ": num_segments < 0");
  if (num_segments == 0) return PA_OK;
  int rc = check_common(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, context_lens_host,
                        num_kv_heads, gqa_ratio, head_dim, block_size, num_pages, scale, dtype, workspace, who);
  if (rc) return rc;
  if (kv_fp8 && (!k_scales || !v_scales)) return fail(PA_EINVAL, w + ": null scale pointer");
  if (!cu_q_lens || !cu_q_lens_host) return fail(PA_EINVAL, w + ": cu_q_lens must be given (device and host)");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return fail(PA_EINVAL, w + ": workspace not 256B aligned");
  if (cu_q_lens_host[0] != 0) return fail(PA_EINVAL, w + ": cu_q_lens[0] != 0");
  std::vector<int32_t> chunk_seg, chunk_tok{0}, chunk_n, chunk_keys;
  int64_t decode_pages = 0;
  int64_t max_rows = 0;
  for (int32_t s = 0; s < num_segments; ++s) {
    const int64_t n = static_cast<int64_t>(cu_q_lens_host[s + 1]) - cu_q_lens_host[s];
    const int64_t L = context_lens_host[s];
    const std::string at = "[" + std::to_string(s) + "]";
    if (n < 1) return fail(PA_EINVAL, w + ": segment" + at + " has no query token");
    if (L < n) return fail(PA_EINVAL, w + ": context_lens" + at + " is shorter than its query tokens");
    if (L > static_cast<int64_t>(max_blocks) * block_size)
      return fail(PA_EINVAL, w + ": context_lens" + at + " exceeds the block table");
    if (n == 1) {
      decode_pages += (L + block_size - 1) / block_size;
    } else {
      chunk_seg.push_back(s);
      chunk_tok.push_back(chunk_tok.back() + static_cast<int32_t>(n));
      chunk_n.push_back(static_cast<int32_t>(n));
      chunk_keys.push_back(static_cast<int32_t>(L));
      max_rows = std::max(max_rows, n * gqa_ratio);
    }
  }
  if (decode_pages > (int64_t(1) << 31) - 1) return fail(PA_EUNSUPPORTED, w + ": too many pages");
  const int32_t num_chunks = static_cast<int32_t>(chunk_seg.size());
  // (over an fp8 cache every shape the chunk tiles take is one the fp8
  // stream kernel takes too)
  const bool built = num_chunks > 0 || kv_fp8 ? mixed_supported(dtype, head_dim, gqa_ratio)
                                              : decode_supported(dtype, head_dim, gqa_ratio);
  if (!built)
    return fail(PA_EUNSUPPORTED, w + ": prefill chunks are built for bf16, head_dim 128, gqa_ratio 1/2/4/8/16");
  // Chunk plan: row blocks of kPrefixRowsPerBlock (token, q-head) rows,
  // each chunk's keys cut into splits of about equal work per workgroup.
  const int32_t row_chunks =
      static_cast<int32_t>(std::max<int64_t>(1, (max_rows + kPrefixRowsPerBlock - 1) / kPrefixRowsPerBlock));
  ChunkPlan plan;
  if (num_chunks > 0) {
    // (The CU count only shapes the splits, never the results; should the
    // query fail, the launch below reports the device error.)
    const int cus = device_cu_count();
    const int32_t wg_per_cu = mixed_one_launch(gqa_ratio, decode_pages, num_chunks) ? kMixedChunkWorkgroupsPerCU
                                                                                    : kChunkWorkgroupsPerCU;
    plan = plan_chunks(chunk_n, chunk_keys, gqa_ratio, num_kv_heads, cus > 0 ? cus : 256, wg_per_cu);
    if (plan.records > INT32_MAX) return fail(PA_EUNSUPPORTED, w + ": too many chunk tokens");
  }
  const int64_t waves = max_waves_per_head(decode_pages, num_kv_heads, 0);
  const size_t stream_bytes =
      partial_layout(waves, num_segments, num_kv_heads, stream_rows(gqa_ratio), head_dim).bytes;
  // (Partial records per kv-head: sum over chunks of tokens x splits.)
  const MixedLayout lay = mixed_layout(num_segments, plan.records / num_kv_heads, num_kv_heads, gqa_ratio, head_dim,
                                       1, stream_bytes);
  if (lay.bytes > workspace_bytes)
    return fail(PA_EWORKSPACE, w + ": workspace holds " + std::to_string(workspace_bytes) + " bytes, needs " +
                                   std::to_string(lay.bytes));
  MixedLaunch m;
  DecodeLaunch& a = m.base;
  a.out = out;
  a.lse_out = lse_out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks = max_blocks;
  a.num_seqs = num_segments;
  a.num_kv_heads = num_kv_heads;
  a.gqa = gqa_ratio;
  a.head_dim = head_dim;
  a.num_pages = num_pages;
  a.scale = scale;
  a.dtype = dtype;
  a.split_pages = 0;
  a.total_pages = decode_pages;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  a.stream = stream;
  a.kv_fp8 = kv_fp8;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  m.cu_q_lens = cu_q_lens;
  m.chunk_seg = chunk_seg.data();
  m.chunk_tok = chunk_tok.data();
  m.num_chunks = num_chunks;
  m.row_chunks = row_chunks;
  m.plan = &plan;
  m.decode_pages = decode_pages;
  m.layout = lay;
  m.workspace = workspace;
  m.workspace_bytes = workspace_bytes;
  return launch_mixed(m);
}

}  // namespace

extern "C" int pa_mixed_chunk(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, int32_t max_blocks, const int32_t* cu_q_lens,
                              const int32_t* cu_q_lens_host, const int32_t* context_lens,
                              const int32_t* context_lens_host, int32_t num_segments, int32_t num_kv_heads,
                              int32_t gqa_ratio, int32_t head_dim, int32_t block_size, int64_t num_pages, float scale,
                              pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return mixed_call(out, lse_out, q, k_pool, v_pool, nullptr, nullptr, false, block_tables, max_blocks, cu_q_lens,
                    cu_q_lens_host, context_lens, context_lens_host, num_segments, num_kv_heads, gqa_ratio, head_dim,
                    block_size, num_pages, scale, dtype, workspace, workspace_bytes, stream, "pa_mixed_chunk");
}

extern "C" int pa_mixed_chunk_fp8(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                                  const float* k_scales, const float* v_scales, const int32_t* block_tables,
                                  int32_t max_blocks, const int32_t* cu_q_lens, const int32_t* cu_q_lens_host,
                                  const int32_t* context_lens, const int32_t* context_lens_host, int32_t num_segments,
                                  int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim, int32_t block_size,
                                  int64_t num_pages, float scale, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  clear_error();
  return mixed_call(out, lse_out, q, k_pool, v_pool, k_scales, v_scales, true, block_tables, max_blocks, cu_q_lens,
                    cu_q_lens_host, context_lens, context_lens_host, num_segments, num_kv_heads, gqa_ratio, head_dim,
                    block_size, num_pages, scale, PA_BF16, workspace, workspace_bytes, stream, "pa_mixed_chunk_fp8");
}

namespace {

// Segments and lengths of a KV append: cu_q_lens[0] = 0, no segment adds a
// negative count, every context holds its new tokens and fits its table.
int check_append_segments(const int32_t* cu_q_lens_host, const int32_t* context_lens_host, int32_t num_segments,
                          int32_t max_blocks, int32_t block_size, const char* who) {
  const std::string w(who);
  if (cu_q_lens_host[0] != 0) return fail(PA_EINVAL, w + ": cu_q_lens[0] != 0");
  for (int32_t s = 0; s < num_segments; ++s) {
    const int64_t n = static_cast<int64_t>(cu_q_lens_host[s + 1]) - cu_q_lens_host[s];
    const int64_t L = context_lens_host[s];
    const std::string at = "[" + std::to_string(s) + "]";
    if (n < 0) return fail(PA_EINVAL, w + ": cu_q_lens decreases at segment" + at);
    if (L < n) return fail(PA_EINVAL, w + ": context_lens" + at + " is shorter than its new tokens");
    if (L > static_cast<int64_t>(max_blocks) * block_size)
      return fail(PA_EINVAL, w + ": context_lens" + at + " exceeds the block table");
  }
  return PA_OK;
}

}  // namespace

extern "C" int pa_kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                            const int32_t* block_tables, int32_t max_blocks, const int32_t* cu_q_lens,
                            const int32_t* cu_q_lens_host, const int32_t* context_lens,
                            const int32_t* context_lens_host, int32_t num_segments, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int64_t num_pages, pa_dtype dtype, void* stream) {
  clear_error();
  if (num_segments < 0) return fail(PA_EINVAL, "pa_kv_append: num_segments < 0");
  if (num_segments == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !block_tables || !cu_q_lens || !cu_q_lens_host || !context_lens ||
      !context_lens_host)
    return fail(PA_EINVAL, "pa_kv_append: null pointer argument");
  if (max_blocks < 1 || num_kv_heads < 1 || head_dim < 1 || num_pages < 1)
    return fail(PA_EINVAL, "pa_kv_append: sizes must be >= 1");
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_EUNSUPPORTED, "pa_kv_append: unknown dtype");
  if (block_size != kBlockSize) return fail(PA_EUNSUPPORTED, "pa_kv_append: only block_size 16 is built");
  const int64_t row_bytes = static_cast<int64_t>(head_dim) * (dtype == PA_F32 ? 4 : 2);
  if (row_bytes % 16 || row_bytes > kMaxAppendRowBytes)
    return fail(PA_EUNSUPPORTED, "pa_kv_append: head_dim * element size must be a multiple of 16 bytes, at most " +
                                     std::to_string(kMaxAppendRowBytes));
  if (num_pages > (int64_t(1) << 31) - 1) return fail(PA_EUNSUPPORTED, "pa_kv_append: num_pages above 2^31-1");
  if (int rc = check_append_segments(cu_q_lens_host, context_lens_host, num_segments, max_blocks, block_size,
                                     "pa_kv_append"))
    return rc;
  const int64_t tokens = cu_q_lens_host[num_segments];
  if (tokens == 0) return PA_OK;
  AppendLaunch a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks;
  a.cu_q_lens = cu_q_lens;
  a.context_lens = context_lens;
  a.num_segments = num_segments;
  a.num_tokens = tokens;
  a.num_kv_heads = num_kv_heads;
  a.row_bytes = static_cast<int32_t>(row_bytes);
  a.num_pages = num_pages;
  a.stream = stream;
  return launch_append(a);
}

extern "C" int pa_kv_append_fp8(void* k_pool, void* v_pool, float* k_scales, float* v_scales, const void* k_new,
                                const void* v_new, const int32_t* block_tables, int32_t max_blocks,
                                const int32_t* cu_q_lens, const int32_t* cu_q_lens_host, const int32_t* context_lens,
                                const int32_t* context_lens_host, int32_t num_segments, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int64_t num_pages, pa_dtype new_dtype,
                                void* stream) {
  clear_error();
  if (num_segments < 0) return fail(PA_EINVAL, "pa_kv_append_fp8: num_segments < 0");
  if (num_segments == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_scales || !v_scales || !k_new || !v_new || !block_tables || !cu_q_lens ||
      !cu_q_lens_host || !context_lens || !context_lens_host)
    return fail(PA_EINVAL, "pa_kv_append_fp8: null pointer argument");
  if (max_blocks < 1 || num_kv_heads < 1 || head_dim < 1 || num_pages < 1)
    return fail(PA_EINVAL, "pa_kv_append_fp8: sizes must be >= 1");
  if (new_dtype != PA_F32 && new_dtype != PA_BF16) return fail(PA_EUNSUPPORTED, "pa_kv_append_fp8: unknown dtype");
  if (block_size != kBlockSize) return fail(PA_EUNSUPPORTED, "pa_kv_append_fp8: only block_size 16 is built");
  if (head_dim != 64 && head_dim != 128) return fail(PA_EUNSUPPORTED, "pa_kv_append_fp8: head_dim must be 64 or 128");
  if (num_pages > (int64_t(1) << 31) - 1) return fail(PA_EUNSUPPORTED, "pa_kv_append_fp8: num_pages above 2^31-1");
  if (int rc = check_append_segments(cu_q_lens_host, context_lens_host, num_segments, max_blocks, block_size,
                                     "pa_kv_append_fp8"))
    return rc;
  const int64_t tokens = cu_q_lens_host[num_segments];
  if (tokens == 0) return PA_OK;
  AppendFp8Launch a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_dtype = new_dtype;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks;
  a.cu_q_lens = cu_q_lens;
  a.context_lens = context_lens;
  a.num_segments = num_segments;
  a.num_tokens = tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_pages = num_pages;
  a.stream = stream;
  return launch_append_fp8(a);
}
