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

// Shapes the kernels are built for.
bool decode_fp8_supported(int32_t head_dim, int32_t gqa) {
  return head_dim == 128 && (gqa == 1 || gqa == 2 || gqa == 4 || gqa == 8 || gqa == 16);
}

bool decode_supported(pa_dtype dtype, int32_t head_dim, int32_t gqa) {
  const bool g_ok = gqa == 1 || gqa == 2 || gqa == 4 || gqa == 8 || gqa == 16;
  if (!g_ok) return false;
  if (dtype == PA_BF16) return head_dim == 64 || head_dim == 128;
  if (dtype == PA_F32) return head_dim == 64;
  return false;
}

bool cascade_supported(pa_dtype dtype, int32_t head_dim, int32_t gqa) {
  return dtype == PA_BF16 && head_dim == 128 && (gqa == 1 || gqa == 2 || gqa == 4 || gqa == 8 || gqa == 16);
}

bool mixed_supported(pa_dtype dtype, int32_t head_dim, int32_t gqa) { return cascade_supported(dtype, head_dim, gqa); }

int64_t max_waves_per_head(int64_t total_pages, int32_t num_kv_heads, int32_t split_pages) {
  if (split_pages > 0) return (total_pages + split_pages - 1) / split_pages;
  const int64_t by_gpu = (kMaxResidentWaves + num_kv_heads - 1) / num_kv_heads;
  const int64_t by_pages = (total_pages + kMinPagesPerWave - 1) / kMinPagesPerWave;
  return std::max<int64_t>(1, std::min(by_gpu, by_pages));
}

MultiPlan plan_multi_shape(int32_t q_len, int32_t gqa) {
  MultiPlan p;
  p.q_len = std::max(1, q_len);
  if (p.q_len == 1) {
    p.rows = gqa;  // plain decode
    return p;
  }
  // The fold factor of the TokenSpeed deep-dive (section 7.2) against the
  // wave's 16 rows; the page's divisibility condition is dropped: a pass
  // addresses its q rows token by token, so the last pass may hold fewer.
  p.fold = std::max(1, std::min(p.q_len, kMaxFoldRows / std::max(1, gqa)));
  int32_t rows = 2;
  while (rows < gqa * p.fold) rows <<= 1;
  p.rows = rows;
  p.passes = (p.q_len + p.fold - 1) / p.fold;
  return p;
}

MultiPlan plan_multi(int32_t q_len, int32_t gqa, const int32_t* context_lens_host, int32_t num_seqs,
                     int32_t block_size, int32_t window) {
  MultiPlan p = plan_multi_shape(q_len, gqa);
  for (int32_t pass = 0; pass < p.passes; ++pass) {
    const int64_t tok0 = static_cast<int64_t>(pass) * p.fold;
    const int64_t fe = std::min<int64_t>(p.fold, p.q_len - tok0);  // tokens of the pass
    const int64_t trim = p.q_len - tok0 - fe;
    // with a window, the pass walks from its earliest token's window on:
    // the last window + fe - 1 rows of its context
    const int64_t walk = window > 0 ? window + fe - 1 : 0;
    int64_t pages = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int64_t L = static_cast<int64_t>(context_lens_host[s]) - trim;
      const int64_t first = walk > 0 && L > walk ? (L - walk) / block_size : 0;
      pages += (L + block_size - 1) / block_size - first;
    }
    p.pass_pages.push_back(pages);
  }
  return p;
}

CascadeLayout cascade_layout(int64_t num_seqs, int32_t num_kv_heads, int32_t gqa, int32_t head_dim, int32_t nks,
                             int64_t stream_bytes) {
  CascadeLayout l;
  const size_t rows = static_cast<size_t>(num_seqs) * num_kv_heads * gqa;  // (sequence, q-head)
  l.begin_offset = 0;
  l.seq_part_offset = align_up(static_cast<size_t>(num_seqs) * sizeof(int32_t));
  // (seq_part and pre_o hold bf16 rows in float-sized slots: room to spare)
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
                      int32_t num_kv_heads, int32_t cus, int32_t wg_per_cu) {
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
  const int64_t slots = static_cast<int64_t>(std::max(cus, 1)) * std::max(wg_per_cu, 1);
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

// Shared-prefix detection (the greedy search the Tokasaurus page runs before
// each forward pass to find shared prefixes among live sequences).  Blocks of
// a shared prefix are stored once and named by every table sharing it, so two
// sequences share their first d pages exactly when their first d table
// entries are equal; a sequence may share at most d pages with d * block_size
// < its context length.  Each round takes the longest prefix still held by
// at least min_group sequences not yet grouped (ties: the prefix with more
// such holders, then the one whose first holder in table order comes first),
// and makes those holders a group.
//
// Instead of a trie of every page, the tables are sorted lexicographically
// (each up to its own depth limit) and the longest common prefixes of
// neighbours give the LCP intervals: a run of sorted rows [l, r] whose common
// prefix is d pages.  Every prefix held by two or more sequences is a trie
// node whose members are such a run, and among the nodes with the same
// members the deepest (the interval) ranks first, so only intervals are
// candidates.  Counts of ungrouped members come from a Fenwick tree over the
// sorted positions; a candidate's depth is fixed and its count only ever
// decreases, so a max-heap with lazy re-keying finds each round's best
// without rescanning.
namespace {
struct Fenwick {
  std::vector<int32_t> t;
  explicit Fenwick(int32_t n) : t(n + 1, 0) {}
  void add(int32_t i, int32_t v) {
    for (++i; i < static_cast<int32_t>(t.size()); i += i & -i) t[i] += v;
  }
  int32_t prefix(int32_t i) const {  // sum over [0, i)
    int32_t r = 0;
    for (; i > 0; i -= i & -i) r += t[i];
    return r;
  }
};
}  // namespace

extern "C" int pa_detect_prefix_groups(const int32_t* bt, int32_t max_blocks, const int32_t* ctx, int32_t num_seqs,
                                       int32_t block_size, int32_t min_group, int32_t min_prefix_pages,
                                       int32_t* order_out, int32_t* group_offsets_out, int32_t* prefix_lens_out,
                                       int32_t* num_groups_out) {
  clear_error();
  if (num_seqs < 0 || max_blocks < 0 || block_size < 1)
    return fail(PA_EINVAL, "pa_detect_prefix_groups: negative size or block_size < 1");
  if (!num_groups_out) return fail(PA_EINVAL, "pa_detect_prefix_groups: null num_groups_out");
  *num_groups_out = 0;
  if (num_seqs == 0) return PA_OK;
  if (!bt || !ctx || !order_out || !group_offsets_out || !prefix_lens_out)
    return fail(PA_EINVAL, "pa_detect_prefix_groups: null pointer argument");
  const int32_t S = num_seqs;
  const int32_t mg = std::max(2, min_group);
  const int32_t mp = std::max(1, min_prefix_pages);
  std::vector<int32_t> dmax(S);
  for (int32_t s = 0; s < S; ++s) {
    const int64_t L = ctx[s];
    if (L < 1 || L > static_cast<int64_t>(max_blocks) * block_size)
      return fail(PA_EINVAL, "pa_detect_prefix_groups: context_lens[" + std::to_string(s) + "] out of range");
    dmax[s] = static_cast<int32_t>((L - 1) / block_size);
  }
  auto row = [&](int32_t s) { return bt + static_cast<int64_t>(s) * max_blocks; };
  // common prefix of two sequences within both depth limits
  auto lcp = [&](int32_t a, int32_t b) {
    const int32_t n = std::min(dmax[a], dmax[b]);
    const int32_t* ra = row(a);
    const int32_t* rb = row(b);
    int32_t d = 0;
    while (d < n && ra[d] == rb[d]) ++d;
    return d;
  };
  std::vector<int32_t> idx(S);
  for (int32_t s = 0; s < S; ++s) idx[s] = s;
  std::sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) {
    const int32_t d = lcp(a, b);
    const int32_t n = std::min(dmax[a], dmax[b]);
    if (d < n) return row(a)[d] < row(b)[d];
    if (dmax[a] != dmax[b]) return dmax[a] < dmax[b];
    return a < b;
  });
  // LCP intervals (depth, sorted range [l, r]) by the usual stack walk over
  // the neighbours' common prefixes.
  struct Interval {
    int32_t depth, l, r, first;  // first: smallest original index in the run
  };
  std::vector<Interval> iv;
  {
    std::vector<std::pair<int32_t, int32_t>> st;  // (depth, left end)
    st.emplace_back(0, 0);
    for (int32_t i = 1; i <= S; ++i) {
      const int32_t h = i < S ? lcp(idx[i - 1], idx[i]) : 0;
      int32_t lb = i - 1;
      while (st.back().first > h) {
        const auto top = st.back();
        st.pop_back();
        iv.push_back(Interval{top.first, top.second, i - 1, 0});
        lb = top.second;
      }
      if (st.back().first < h) st.emplace_back(h, lb);
    }
  }
  for (Interval& x : iv) {
    x.first = S;
    for (int32_t p = x.l; p <= x.r; ++p) x.first = std::min(x.first, idx[p]);
  }
  Fenwick left(S);  // 1 at each sorted position not yet grouped
  for (int32_t p = 0; p < S; ++p) left.add(p, 1);
  auto remaining = [&](const Interval& x) { return left.prefix(x.r + 1) - left.prefix(x.l); };
  struct Cand {
    int32_t depth, count, first, id;
    bool operator<(const Cand& o) const {
      if (depth != o.depth) return depth < o.depth;
      if (count != o.count) return count < o.count;
      return first > o.first;  // the earlier first holder ranks higher
    }
  };
  auto cand_of = [&](int32_t i) { return Cand{iv[i].depth, remaining(iv[i]), iv[i].first, i}; };
  auto eligible = [&](int32_t i) {
    const int32_t n = remaining(iv[i]);
    return n >= mg && iv[i].depth >= mp;
  };
  std::vector<Cand> heap;
  for (int32_t i = 0; i < static_cast<int32_t>(iv.size()); ++i)
    if (eligible(i)) heap.push_back(cand_of(i));
  std::make_heap(heap.begin(), heap.end());
  std::vector<char> assigned(S, 0);
  int32_t placed = 0, groups = 0;
  group_offsets_out[0] = 0;
  while (!heap.empty()) {
    std::pop_heap(heap.begin(), heap.end());
    const Cand top = heap.back();
    heap.pop_back();
    if (!eligible(top.id)) continue;
    const Cand now = cand_of(top.id);
    if (now.count != top.count) {  // stale: members were grouped since it was pushed
      heap.push_back(now);
      std::push_heap(heap.begin(), heap.end());
      continue;
    }
    const Interval& x = iv[top.id];
    const int32_t first = placed;
    for (int32_t p = x.l; p <= x.r; ++p) {
      if (assigned[idx[p]]) continue;
      assigned[idx[p]] = 1;
      left.add(p, -1);
      order_out[placed++] = idx[p];
    }
    std::sort(order_out + first, order_out + placed);  // members by original index
    prefix_lens_out[groups] = x.depth * block_size;
    group_offsets_out[++groups] = placed;
  }
  if (placed < S) {
    for (int32_t s = 0; s < S; ++s)
      if (!assigned[s]) order_out[placed++] = s;
    prefix_lens_out[groups] = 0;
    group_offsets_out[++groups] = placed;
  }
  *num_groups_out = groups;
  return PA_OK;
}
