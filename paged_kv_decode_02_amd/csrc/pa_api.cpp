// C-ABI entry points: argument validation and split planning on the host,
// then the launch.  Nothing here touches device memory.
#include <string>

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
  return partial_layout(waves, max_num_seqs, num_kv_heads, gqa_ratio, head_dim).bytes;
}

extern "C" int pa_decode(void* out, float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                         const int32_t* context_lens_host, int32_t num_seqs, int32_t num_kv_heads,
                         int32_t gqa_ratio, int32_t head_dim, int32_t block_size, int64_t num_pages, float scale,
                         pa_dtype dtype, int32_t split_pages, void* workspace, size_t workspace_bytes,
                         void* stream) {
  clear_error();
  if (num_seqs < 0) return fail(PA_EINVAL, "pa_decode: num_seqs < 0");
  if (num_seqs == 0) return PA_OK;
  int rc = check_common(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, context_lens_host,
                        num_kv_heads, gqa_ratio, head_dim, block_size, num_pages, scale, dtype, workspace,
                        "pa_decode");
  if (rc) return rc;
  if (split_pages < 0) return fail(PA_EINVAL, "pa_decode: split_pages < 0");
  if (!decode_supported(dtype, head_dim, gqa_ratio))
    return fail(PA_EUNSUPPORTED, "pa_decode: no kernel for dtype/head_dim " + std::to_string(head_dim) +
                                     "/gqa_ratio " + std::to_string(gqa_ratio));
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return fail(PA_EINVAL, "pa_decode: workspace not 256B aligned");
  int64_t total_pages = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t L = context_lens_host[s];
    if (L < 1) return fail(PA_EINVAL, "pa_decode: context_lens[" + std::to_string(s) + "] < 1");
    if (L > static_cast<int64_t>(max_blocks) * block_size)
      return fail(PA_EINVAL, "pa_decode: context_lens[" + std::to_string(s) + "] exceeds the block table");
    total_pages += (L + block_size - 1) / block_size;
  }
  if (total_pages > (int64_t(1) << 31) - 1) return fail(PA_EUNSUPPORTED, "pa_decode: more than 2^31-1 pages");
  // The workspace must hold the largest plan this batch could get, so that
  // a call never depends on the occupancy the device reports.
  const PartialLayout worst = partial_layout(max_waves_per_head(total_pages, num_kv_heads, split_pages), num_seqs,
                                             num_kv_heads, gqa_ratio, head_dim);
  if (worst.bytes > workspace_bytes)
    return fail(PA_EWORKSPACE, "pa_decode: workspace holds " + std::to_string(workspace_bytes) + " bytes, needs " +
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
  return launch_decode(a);
}
