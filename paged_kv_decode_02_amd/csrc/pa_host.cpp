// Host-side pieces of libpa: error state, split planning, workspace layout
// and the block-table checker.  Plain C++ (no HIP), so it can also be built
// with g++ and host sanitizers.
#include <algorithm>
#include <climits>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

namespace pa {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

void clear_error() { g_last_error.clear(); }

PartialLayout partial_layout(int64_t waves, int64_t num_seqs, int32_t num_kv_heads, int32_t gqa, int32_t head_dim) {
  PartialLayout l;
  const size_t rows = static_cast<size_t>(waves) * num_kv_heads * 2 * gqa;
  l.info_offset = 0;
  l.lse_offset = align_up(static_cast<size_t>(num_seqs) * 4 * sizeof(int32_t));
  l.o_offset = l.lse_offset + align_up(rows * sizeof(float));
  l.bytes = l.o_offset + align_up(rows * head_dim * sizeof(float));
  return l;
}

int64_t max_waves_per_head(int64_t total_pages, int32_t num_kv_heads, int32_t split_pages) {
  if (split_pages > 0) return (total_pages + split_pages - 1) / split_pages;
  const int64_t by_gpu = (kMaxResidentWaves + num_kv_heads - 1) / num_kv_heads;
  const int64_t by_pages = (total_pages + kMinPagesPerWave - 1) / kMinPagesPerWave;
  return std::max<int64_t>(1, std::min(by_gpu, by_pages));
}

CascadeLayout cascade_layout(int64_t num_seqs, int32_t num_kv_heads, int32_t gqa, int32_t head_dim, int32_t nks,
                             int64_t stream_bytes) {
  CascadeLayout l;
  const size_t rows = static_cast<size_t>(num_seqs) * num_kv_heads * gqa;  // (sequence, q-head)
  l.begin_offset = 0;
  l.seq_part_offset = align_up(static_cast<size_t>(num_seqs) * sizeof(int32_t));
  l.pre_o_offset = l.seq_part_offset + align_up(rows * (head_dim + 1) * sizeof(float));
  l.pre_lse_offset = l.pre_o_offset + align_up(rows * nks * head_dim * sizeof(float));
  l.stream_offset = l.pre_lse_offset + align_up(rows * nks * sizeof(float));
  l.bytes = l.stream_offset + align_up(static_cast<size_t>(stream_bytes));
  return l;
}

MixedLayout mixed_layout(int64_t num_seqs, int64_t chunk_tokens, int32_t num_kv_heads, int32_t gqa, int32_t head_dim,
                         int32_t nks, int64_t stream_bytes) {
  MixedLayout l;
  const size_t rows = static_cast<size_t>(chunk_tokens) * num_kv_heads * gqa;  // (chunk token, q-head)
  l.begin_offset = 0;
  l.pre_o_offset = align_up(static_cast<size_t>(num_seqs) * sizeof(int32_t));
  l.pre_lse_offset = l.pre_o_offset + align_up(rows * nks * head_dim * sizeof(float));
  l.stream_offset = l.pre_lse_offset + align_up(rows * nks * sizeof(float));
  l.bytes = l.stream_offset + align_up(static_cast<size_t>(stream_bytes));
  return l;
}

ChunkPlan plan_chunks(const std::vector<int32_t>& n_tok, const std::vector<int32_t>& keys, int32_t gqa,
                      int32_t num_kv_heads, int32_t cus) {
  const size_t n = n_tok.size();
  // Tiles of 64 keys the chunks' row blocks stream in all: the last token
  // of a row block bounds the keys it sees (causal inside the chunk).
  int64_t total = 0;
  for (size_t u = 0; u < n; ++u) {
    const int64_t rows = static_cast<int64_t>(n_tok[u]) * gqa;
    const int64_t L = keys[u];
    for (int64_t r0 = 0; r0 < rows; r0 += kPrefixRowsPerBlock) {
      const int64_t i_max = (std::min<int64_t>(rows, r0 + kPrefixRowsPerBlock) - 1) / gqa;
      const int64_t k_end = std::min<int64_t>(L, L - n_tok[u] + i_max + 1);
      total += (k_end + 63) / 64;
    }
  }
  total *= num_kv_heads;
  const int64_t slots = static_cast<int64_t>(std::max(cus, 1)) * kChunkWorkgroupsPerCU;
  const int64_t per_wg = std::max<int64_t>(kMinChunkSplitKeys / 64, (total + slots - 1) / slots);
  ChunkPlan p;
  p.nks.resize(n);
  p.kps.resize(n);
  p.rec.resize(n);
  p.tiles.resize(n);
  for (size_t u = 0; u < n; ++u) {
    const int64_t L = keys[u];
    const int64_t kt = (L + 63) / 64;
    int64_t nks = std::min<int64_t>(kMaxChunkSplits, std::max<int64_t>(1, (kt + per_wg - 1) / per_wg));
    const int64_t kps = ((L + nks - 1) / nks + 63) / 64 * 64;
    nks = (L + kps - 1) / kps;
    p.nks[u] = static_cast<int32_t>(nks);
    p.kps[u] = static_cast<int32_t>(kps);
    p.tiles[u] = static_cast<int32_t>((std::min<int64_t>(kps, L) + 63) / 64);
    p.rec[u] = static_cast<int32_t>(std::min<int64_t>(p.records, INT32_MAX));
    p.records += static_cast<int64_t>(n_tok[u]) * num_kv_heads * nks;
  }
  return p;
}

}  // namespace pa

using namespace pa;

extern "C" const char* pa_last_error(void) { return g_last_error.c_str(); }

extern "C" int pa_check_block_tables(const int32_t* bt, int32_t max_blocks, const int32_t* ctx, int32_t num_seqs,
                                     int32_t block_size, int64_t num_pages, int32_t num_groups,
                                     const int32_t* group_offsets, const int32_t* prefix_lens) {
  clear_error();
  if (num_seqs < 0 || max_blocks < 0 || block_size < 1 || num_pages < 0 || num_groups < 0)
    return fail(PA_EINVAL, "pa_check_block_tables: negative size");
  if (num_seqs == 0) return PA_OK;
  if (!bt || !ctx) return fail(PA_EINVAL, "pa_check_block_tables: null table or lengths");
  if (num_groups > 0 && (!group_offsets || !prefix_lens))
    return fail(PA_EINVAL, "pa_check_block_tables: groups given without offsets/prefix lengths");
  std::vector<int64_t> prefix_pages(num_seqs, 0);
  // page -> owner: >= 0 sequence id, < 0 encodes -(group + 1)
  std::unordered_map<int64_t, int64_t> owner;
  if (num_groups > 0) {
    if (group_offsets[0] < 0 || group_offsets[num_groups] > num_seqs)
      return fail(PA_EINVAL, "group offsets outside [0, num_seqs]");
    for (int32_t g = 0; g < num_groups; ++g) {
      const int32_t a = group_offsets[g], b = group_offsets[g + 1];
      if (b < a) return fail(PA_EINVAL, "group " + std::to_string(g) + ": offsets decrease");
      const int32_t P = prefix_lens[g];
      if (P < 0 || P % block_size)
        return fail(PA_EINVAL, "group " + std::to_string(g) + ": prefix length not a whole number of pages");
      const int64_t np = P / block_size;
      if (np > max_blocks) return fail(PA_EINVAL, "group " + std::to_string(g) + ": prefix longer than the table");
      for (int32_t s = a; s < b; ++s) {
        if (P >= ctx[s])
          return fail(PA_EINVAL, "group " + std::to_string(g) + ": prefix not shorter than sequence " +
                                     std::to_string(s));
        if (std::memcmp(bt + static_cast<int64_t>(s) * max_blocks, bt + static_cast<int64_t>(a) * max_blocks,
                        np * sizeof(int32_t)) != 0)
          return fail(PA_EINVAL, "group " + std::to_string(g) + ": sequence " + std::to_string(s) +
                                     " does not share the prefix pages");
        prefix_pages[s] = np;
      }
      for (int64_t j = 0; j < np && b > a; ++j) {
        const int64_t p = bt[static_cast<int64_t>(a) * max_blocks + j];
        if (p < 0 || p >= num_pages)
          return fail(PA_EINVAL, "group " + std::to_string(g) + ": prefix entry out of range");
        if (!owner.emplace(p, -(g + 1)).second)
          return fail(PA_EINVAL, "page " + std::to_string(p) + " named by two groups' prefixes");
      }
    }
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t L = ctx[s];
    if (L < 1) return fail(PA_EINVAL, "sequence " + std::to_string(s) + ": empty context");
    const int64_t n = (L + block_size - 1) / block_size;
    if (n > max_blocks) return fail(PA_EINVAL, "sequence " + std::to_string(s) + ": table too short");
    for (int64_t j = prefix_pages[s]; j < n; ++j) {
      const int64_t p = bt[static_cast<int64_t>(s) * max_blocks + j];
      if (p < 0 || p >= num_pages)
        return fail(PA_EINVAL, "sequence " + std::to_string(s) + ": entry " + std::to_string(j) + " out of range");
      if (!owner.emplace(p, s).second)
        return fail(PA_EINVAL, "sequence " + std::to_string(s) + ": page " + std::to_string(p) +
                                   " is also named elsewhere");
    }
  }
  return PA_OK;
}
