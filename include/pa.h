/*
 * pa.h -- attention over a paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpa.so.  Every pointer is a raw address; the header says for
 * each one whether it is device memory (HBM) or host memory.  No call
 * allocates memory (the measurement hook pa_profile_enable at the end
 * aside): the caller owns q, the pools, the tables, the outputs and the
 * workspace.  Kernels are launched asynchronously on the HIP stream
 * passed as `stream` (a hipStream_t, NULL = the default stream); device
 * buffers must stay alive until the stream reaches the call.  Host arrays
 * (the `*_host` twins) are read synchronously before the call returns, so
 * planning never waits for the device.
 *
 * The problem statement these calls follow:
 *  - KV cache split into fixed-size blocks (pages); a sequence's rows are
 *    found through its block table; blocks of a shared prefix may be named
 *    by many tables (SwiftLLM page, section 3.1 "PagedAttention and KV
 *    cache management").
 *  - The attention layer is handed the block tables and per-sequence
 *    context lengths (SwiftLLM page, section 5.1).
 *  - Split-KV decode: each split writes a partial output and its
 *    log-sum-exp to a workspace, and a second pass reduces the partials by
 *    their LSE (TokenSpeed deep-dive, sections 7 and 7.1).
 *  - Page size is a property of the kernel, passed explicitly, never
 *    derived (TokenSpeed deep-dive, section 4.3); no argument has a
 *    default and an idle step passes zero-length arrays (section 8.2).
 *
 * Layouts (all row-major, C order):
 *  q          [T, Hq, D]   dtype        T = number of query tokens
 *  out        [T, Hq, D]   dtype
 *  lse_out    [T, Hq]      float32, natural log (may be NULL)
 *  k_pool     [num_pages, Hkv, block_size, D]   dtype
 *  v_pool     [num_pages, Hkv, block_size, D]   dtype
 *  block_tables [num_seqs, max_blocks_per_seq] int32; entry j of row s is
 *             the physical page holding rows [16j, 16j+16) of sequence s.
 *  context_lens [num_seqs] int32: rows of sequence s in the pool,
 *             including this step's own tokens.
 * Hq = num_kv_heads * gqa_ratio; q-head h reads kv-head h / gqa_ratio.
 *
 * Semantics: query token i of a sequence with L rows and n query tokens
 * sees rows [0, L - n + i] (decode: n = 1, all L rows):
 *     out = sum_t softmax_t(scale * <q, k_t>) v_t,
 *     lse = ln sum_t exp(scale * <q, k_t>).
 * Arithmetic is float32 (bf16 products are exact in float32); bf16
 * outputs are rounded to nearest even.
 *
 * Errors: every call returns PA_OK or a negative code, never throws, and
 * on error launches nothing; pa_last_error() then holds a message.
 * Table *contents* in device memory are not checked on the hot call
 * (pa_check_block_tables does that on host copies); kernels clamp every
 * page id into [0, num_pages), so a bad table gives wrong numbers, never an
 * out-of-bounds access.  `context_lens` and `context_lens_host` must hold
 * the same values; if they do not, results are undefined but every access
 * still stays inside the buffers passed.
 *
 * Thread safety: calls are reentrant (pa_profile_enable / _collect aside:
 * they keep per-thread state).  Two calls that share a workspace must be
 * ordered on one stream.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

enum {
  PA_OK = 0,
  PA_EINVAL = -1,       /* bad argument (null pointer, size, length) */
  PA_EUNSUPPORTED = -2, /* valid but not built: head_dim, block_size, gqa_ratio, dtype */
  PA_EWORKSPACE = -3,   /* workspace too small for this call's plan */
  PA_EHIP = -4          /* a HIP runtime call failed */
};

/* Supported shapes: block_size 16; head_dim 64 or 128 (bf16) and 64
 * (float32); gqa_ratio 1, 2, 4, 8 or 16 for decode.  With bf16 q and 4 or
 * more q-heads per kv-head a wave's 16 query rows run on the matrix cores
 * (16 x 16 x 32 bf16 MFMA tiles); otherwise on the vector ALUs.  Results
 * are the same attention either way, within the stated tolerances. */

/* ---------------------------------------------------------------------------
 * Decode: one query token per sequence (T = num_seqs).
 *
 * For each kv-head the pages of all sequences are laid end to end and cut
 * into runs of `split_pages` pages (0 = sized so the GPU's resident waves
 * are filled once); each wave streams one run and computes the G =
 * gqa_ratio q-heads that share the kv-head from one pass over K and V.  A
 * sequence covered by one run is written directly; the partials of a
 * sequence shared by several runs are merged by their LSE.
 *
 * workspace: device memory of at least pa_decode_workspace_size(...) bytes
 *   for the largest batch it will serve; 256-byte aligned.  Its contents
 *   need no initialisation and are scratch between calls.
 * Returns PA_OK; PA_EINVAL for null pointers (lse_out may be NULL), sizes
 *   < 1 (num_seqs == 0 is a no-op returning PA_OK), a context length < 1
 *   or > max_blocks_per_seq * block_size, or split_pages < 0;
 *   PA_EUNSUPPORTED for shapes not built; PA_EWORKSPACE if the plan needs
 *   more workspace than workspace_bytes; PA_EHIP if a launch fails.
 * ------------------------------------------------------------------------- */
size_t pa_decode_workspace_size(int32_t max_num_seqs, int32_t num_kv_heads, int32_t gqa_ratio,
                                int32_t head_dim, int64_t max_total_pages, int32_t split_pages);

int pa_decode(void* out,                      /* device [S, Hq, D] dtype */
              float* lse_out,                 /* device [S, Hq] or NULL */
              const void* q,                  /* device [S, Hq, D] dtype */
              const void* k_pool,             /* device [NP, Hkv, BS, D] dtype */
              const void* v_pool,             /* device [NP, Hkv, BS, D] dtype */
              const int32_t* block_tables,    /* device [S, max_blocks_per_seq] */
              int32_t max_blocks_per_seq,
              const int32_t* context_lens,    /* device [S] */
              const int32_t* context_lens_host, /* host [S], same values */
              int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim,
              int32_t block_size, int64_t num_pages, float scale, pa_dtype dtype,
              int32_t split_pages,            /* pages per split; 0 = automatic */
              void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Decode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels, plan and results as pa_decode
 * (bit for bit), minus the workspace: the scratch lives in a file-scope
 * device array of PA_NOALLOC_SCRATCH_BYTES bytes, one copy per GPU, held
 * until the process ends.  The call allocates nothing (its first call on a
 * device looks the array's address up; nothing is allocated then either).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other host threads) race; calls ordered on one stream
 * are safe.  The scratch needs no clearing between calls.
 * Returns as pa_decode; PA_EWORKSPACE when the batch's plan needs more than
 * PA_NOALLOC_SCRATCH_BYTES (many sequences shared by many waves: a smaller
 * split_pages needs more), checked before anything is launched; PA_EHIP if
 * there is no current device.
 * ------------------------------------------------------------------------- */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)

int pa_decode_noalloc(void* out,                   /* device [S, Hq, D] dtype */
                      float* lse_out,              /* device [S, Hq] or NULL */
                      const void* q,               /* device [S, Hq, D] dtype */
                      const void* k_pool,          /* device [NP, Hkv, BS, D] dtype */
                      const void* v_pool,          /* device [NP, Hkv, BS, D] dtype */
                      const int32_t* block_tables, /* device [S, max_blocks_per_seq] */
                      int32_t max_blocks_per_seq,
                      const int32_t* context_lens,      /* device [S] */
                      const int32_t* context_lens_host, /* host [S], same values */
                      int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim,
                      int32_t block_size, int64_t num_pages, float scale, pa_dtype dtype,
                      int32_t split_pages, /* pages per split; 0 = automatic */
                      void* stream);

/* ---------------------------------------------------------------------------
 * Sliding-window decode: pa_decode where the query of a sequence with L rows
 * sees only rows [max(0, L - window), L).  A sliding-window KV group
 * declares its window in tokens (TokenSpeed deep-dive section 4.1, the
 * attention kinds); its block table keeps the real blocks at the back and
 * placeholder entries at the front for blocks that fell out of the window
 * (tokenspeed 딥다이브 section 6-3).  Only entries from (L - window) / 16 on
 * are read, so placeholders may name any page (page 0 by convention) and
 * are never dereferenced; the rows of the window's first page before
 * L - window are masked.  Work is planned over the window's pages only.
 *
 * window: tokens, >= 1 (PA_EINVAL otherwise); a window >= L is plain decode.
 * Everything else as pa_decode (same workspace size for the same batch).
 * ------------------------------------------------------------------------- */
int pa_decode_window(void* out,                 /* device [S, Hq, D] dtype */
                     float* lse_out,            /* device [S, Hq] or NULL */
                     const void* q,             /* device [S, Hq, D] dtype */
                     const void* k_pool,        /* device [NP, Hkv, BS, D] dtype */
                     const void* v_pool,        /* device [NP, Hkv, BS, D] dtype */
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* context_lens_host,
                     int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim,
                     int32_t block_size, int64_t num_pages, float scale, pa_dtype dtype,
                     int32_t window,            /* tokens, >= 1 */
                     int32_t split_pages, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Decode over an fp8 KV cache: pa_decode with K and V stored as OCP e4m3fn
 * codes (one byte each: 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals, NaN = 0x7f/0xff, largest finite value 448) and one float32
 * scale per (page, kv-head, slot) for K and one for V.  A stored row reads
 * back as code value * scale -- the token-group FP8 recipe of the tokenspeed
 * 딥다이브 page (section 6-4), with a group = one kv-head's row of one
 * token.  q and out are bf16; scores use the K scale of each row, P.V the
 * V scale folded into the probability (rounded to bf16 for P.V, like the
 * bf16 path); lse_out, split planning and the workspace (the same size as
 * pa_decode_workspace_size gives) are as for pa_decode.
 *
 *  k_pool, v_pool   [NP, Hkv, 16, D] uint8 codes (device)
 *  k_scales, v_scales [NP, Hkv, 16] float32 (device)
 * Built for head_dim 128 and gqa_ratio 1, 2, 4, 8, 16.  Errors as pa_decode;
 * PA_EINVAL also for a NULL scale pointer.
 * ------------------------------------------------------------------------- */
int pa_decode_fp8(void* out,                  /* device [S, Hq, D] bf16 */
                  float* lse_out,             /* device [S, Hq] or NULL */
                  const void* q,              /* device [S, Hq, D] bf16 */
                  const void* k_pool,         /* device [NP, Hkv, BS, D] e4m3fn codes */
                  const void* v_pool,         /* device [NP, Hkv, BS, D] e4m3fn codes */
                  const float* k_scales,      /* device [NP, Hkv, BS] */
                  const float* v_scales,      /* device [NP, Hkv, BS] */
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, const int32_t* context_lens_host,
                  int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim,
                  int32_t block_size, int64_t num_pages, float scale, int32_t split_pages,
                  void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Multi-token decode: every sequence brings q_len >= 1 new tokens at once
 * (T = num_seqs * q_len; token i of sequence s is q / out / lse row
 * s * q_len + i), causal among them: with L = context_lens[s] rows, the
 * new tokens counted, token i sits at position L - q_len + i and sees rows
 * 0 .. L - q_len + i.  The tokens are folded into the query rows a wave
 * computes from one pass over K and V, next to the gqa_ratio heads: the
 * fold_sq_factor of the TokenSpeed deep-dive (section 7.2), with a wave's
 * 16 rows in place of the page's 128-row tile.  fold = min(q_len,
 * 16 / gqa_ratio) tokens share a pass; ceil(q_len / fold) passes run one
 * after another on `stream` (unlike the page, q_len need not be a multiple
 * of the fold: the last pass may hold fewer tokens).  q_len == 1 is
 * pa_decode exactly.  Results equal pa_mixed_chunk's on a batch of
 * segments of q_len tokens each.
 *
 * workspace: at least pa_decode_multi_workspace_size(...) bytes for the
 *   largest batch it will serve (max_total_pages = sum of ceil(L / 16));
 *   256-byte aligned, no initialisation, scratch between calls.
 * Built for bf16 (head_dim 64, 128) and float32 (head_dim 64), gqa_ratio
 * 1, 2, 4, 8, 16.  Errors as pa_decode, plus PA_EINVAL for q_len < 1 or a
 * context length < q_len.
 * ------------------------------------------------------------------------- */
size_t pa_decode_multi_workspace_size(int32_t max_num_seqs, int32_t q_len, int32_t num_kv_heads, int32_t gqa_ratio,
                                      int32_t head_dim, int64_t max_total_pages, int32_t split_pages);

int pa_decode_multi(void* out,                 /* device [S * q_len, Hq, D] dtype */
                    float* lse_out,            /* device [S * q_len, Hq] or NULL */
                    const void* q,             /* device [S * q_len, Hq, D] dtype */
                    const void* k_pool,        /* device [NP, Hkv, BS, D] dtype */
                    const void* v_pool,        /* device [NP, Hkv, BS, D] dtype */
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, const int32_t* context_lens_host,
                    int32_t num_seqs, int32_t q_len, int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim,
                    int32_t block_size, int64_t num_pages, float scale, pa_dtype dtype, int32_t split_pages,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Multi-token decode over a sliding-window cache: pa_decode_multi's tokens
 * and fold, each token with its own window of `window` tokens (TokenSpeed
 * deep-dive section 4.1, sliding_window_tokens): with L = context_lens[s],
 * token i sits at position p = L - q_len + i and sees rows
 * max(0, p + 1 - window) .. p.  Table entries before the first page of the
 * earliest token's window, (L - q_len + 1 - window) / block_size, may be
 * placeholders (tokenspeed 딥다이브 section 6-3): they are never read.
 * Workspace: pa_decode_multi_workspace_size.  Built as pa_decode_multi.
 * Errors as pa_decode_multi, plus PA_EINVAL for window < 1.  q_len == 1 is
 * pa_decode_window exactly; a window of at least every context length is
 * pa_decode_multi exactly.
 * ------------------------------------------------------------------------- */
int pa_decode_multi_window(void* out,                 /* device [S * q_len, Hq, D] dtype */
                           float* lse_out,            /* device [S * q_len, Hq] or NULL */
                           const void* q,             /* device [S * q_len, Hq, D] dtype */
                           const void* k_pool,        /* device [NP, Hkv, BS, D] dtype */
                           const void* v_pool,        /* device [NP, Hkv, BS, D] dtype */
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, const int32_t* context_lens_host,
                           int32_t num_seqs, int32_t q_len, int32_t window, int32_t num_kv_heads,
                           int32_t gqa_ratio, int32_t head_dim, int32_t block_size, int64_t num_pages, float scale,
                           pa_dtype dtype, int32_t split_pages, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ---------------------------------------------------------------------------
 * Multi-token decode over an fp8 cache: pa_decode_multi's tokens, rows and
 * causal limits (token i of a sequence with L rows sees rows 0 ..
 * L - q_len + i) over pa_decode_fp8's pools (e4m3fn codes with one float32
 * scale per (page, kv-head, slot) for K and one for V, tokenspeed 딥다이브
 * section 6-4); q and out bf16.  Every folded pass runs on the matrix cores.
 * Workspace: pa_decode_multi_workspace_size.  Built for head_dim 128 and
 * gqa_ratio 1, 2, 4, 8, 16.  Errors as pa_decode_multi, plus PA_EINVAL for
 * a NULL scale pointer.  q_len == 1 is pa_decode_fp8 exactly.
 * ------------------------------------------------------------------------- */
int pa_decode_multi_fp8(void* out,                 /* device [S * q_len, Hq, D] bf16 */
                        float* lse_out,            /* device [S * q_len, Hq] or NULL */
                        const void* q,             /* device [S * q_len, Hq, D] bf16 */
                        const void* k_pool,        /* device [NP, Hkv, BS, D] e4m3fn codes */
                        const void* v_pool,        /* device [NP, Hkv, BS, D] e4m3fn codes */
                        const float* k_scales,     /* device [NP, Hkv, BS] */
                        const float* v_scales,     /* device [NP, Hkv, BS] */
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, const int32_t* context_lens_host,
                        int32_t num_seqs, int32_t q_len, int32_t num_kv_heads, int32_t gqa_ratio,
                        int32_t head_dim, int32_t block_size, int64_t num_pages, float scale,
                        int32_t split_pages, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Shared-prefix (cascade) decode: one query token per sequence, sequences in
 * groups whose block tables start with the same prefix pages (shared blocks,
 * SwiftLLM page section 3.1); the result equals pa_decode on the same
 * inputs.  The prefix is attended once per group with MFMA -- the group's
 * (member, q-head) rows against the prefix keys form one dense product
 * (Tokasaurus page, "dynamic prefix identification": Hydragen / cascade
 * attention) -- each member's suffix is decoded as in pa_decode, and the two
 * are merged by log-sum-exp.
 *
 * Groups: sequences [group_seq_offsets[g], group_seq_offsets[g+1]) for
 * g < num_groups, covering 0 .. num_seqs-1 in order; prefix_lens[g] is a
 * multiple of block_size (0 allowed), shorter than every member's context,
 * and every member's first prefix_lens[g]/block_size table entries are the
 * same pages (not checked on this call; see pa_check_block_tables).  Device
 * arrays and their host twins must hold the same values.
 * Built for bf16, head_dim 128, gqa_ratio 1, 2, 4, 8, 16.
 * Errors as pa_decode, plus PA_EINVAL for malformed groups.
 * ------------------------------------------------------------------------- */
size_t pa_prefix_cascade_workspace_size(int32_t max_num_seqs, int32_t num_kv_heads, int32_t gqa_ratio,
                                        int32_t head_dim, int64_t max_total_pages);

int pa_prefix_cascade(void* out,                       /* device [S, Hq, D] */
                      float* lse_out,                  /* device [S, Hq] or NULL */
                      const void* q,                   /* device [S, Hq, D] */
                      const void* k_pool, const void* v_pool, /* device [NP, Hkv, BS, D] */
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens,      /* device [S] */
                      const int32_t* context_lens_host, /* host [S] */
                      int32_t num_seqs, int32_t num_groups,
                      const int32_t* group_seq_offsets,      /* device [G+1] */
                      const int32_t* group_seq_offsets_host, /* host [G+1] */
                      const int32_t* prefix_lens,            /* device [G] */
                      const int32_t* prefix_lens_host,       /* host [G] */
                      int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim, int32_t block_size,
                      int64_t num_pages, float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ---------------------------------------------------------------------------
 * Shared-prefix (cascade) decode over an fp8 cache: pa_prefix_cascade's
 * groups, prefixes and result (decode over each member's whole table) over
 * pa_decode_fp8's pools -- e4m3fn codes with one float32 scale per (page,
 * kv-head, slot) for K and one for V (tokenspeed 딥다이브 section 6-4); q and
 * out bf16.  The prefix tiles read the codes, widen them exactly to bf16 for
 * the matrix cores, and apply each key's K scale to its scores and its V
 * scale to the probability P.V takes; the suffix runs on the fp8 stream
 * kernel.  Workspace: pa_prefix_cascade_workspace_size.  Built for
 * head_dim 128, gqa_ratio 1, 2, 4, 8, 16.  Errors as pa_prefix_cascade, plus
 * PA_EINVAL for a NULL scale pointer.
 * ------------------------------------------------------------------------- */
int pa_prefix_cascade_fp8(void* out,                       /* device [S, Hq, D] bf16 */
                          float* lse_out,                  /* device [S, Hq] or NULL */
                          const void* q,                   /* device [S, Hq, D] bf16 */
                          const void* k_pool, const void* v_pool, /* device [NP, Hkv, BS, D] e4m3fn codes */
                          const float* k_scales, const float* v_scales, /* device [NP, Hkv, BS] */
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens,      /* device [S] */
                          const int32_t* context_lens_host, /* host [S] */
                          int32_t num_seqs, int32_t num_groups,
                          const int32_t* group_seq_offsets,      /* device [G+1] */
                          const int32_t* group_seq_offsets_host, /* host [G+1] */
                          const int32_t* prefix_lens,            /* device [G] */
                          const int32_t* prefix_lens_host,       /* host [G] */
                          int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim, int32_t block_size,
                          int64_t num_pages, float scale, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Mixed batch: prefill chunks and decode tokens in one call (decode tokens
 * of many sequences piggybacked on prefill chunks: SwiftLLM page, section
 * 3.3, SARATHI-style piggybacking; prefill admitted in bounded chunks, each attending
 * to the cached prefix plus itself: TokenSpeed deep-dive section 5.1, with
 * the per-segment lengths passed as device + host copies and no defaults,
 * section 8.2).
 *
 * Segment s has q_len = cu_q_lens[s+1] - cu_q_lens[s] >= 1 query tokens at
 * rows cu_q_lens[s] .. cu_q_lens[s+1]-1 of q / out / lse_out (T =
 * cu_q_lens[num_segments] rows), and context_lens[s] >= q_len rows in the
 * pool, its own new rows included (they are written to the pool before the
 * call).  Its token i sees rows [0, context_lens[s] - q_len + i]: causal
 * inside the chunk; q_len = 1 is a decode token and sees every row.
 * Chunks (q_len > 1) run as MFMA tiles of (token, q-head) rows against the
 * segment's keys, split along the keys and merged by log-sum-exp; decode
 * tokens run on pa_decode's stream wave.  With 4 or more q-heads per
 * kv-head, a batch holding both runs them in one launch (chunk workgroups
 * and decode workgroups side by side, the decode split planned for that
 * launch), so its decode rows equal pa_decode's within the stated
 * tolerances; a batch without chunks takes pa_decode's plan, bit for bit.
 * Chunks are built for bf16, head_dim 128, gqa_ratio 1, 2, 4, 8, 16; a
 * batch without chunks takes every pa_decode shape.
 * Returns as pa_decode, plus PA_EINVAL for cu_q_lens[0] != 0, a segment
 * with no query token or with context_lens[s] < q_len.
 * ------------------------------------------------------------------------- */
size_t pa_mixed_chunk_workspace_size(int32_t max_num_tokens, int32_t max_num_segments, int32_t num_kv_heads,
                                     int32_t gqa_ratio, int32_t head_dim, int64_t max_total_pages);

int pa_mixed_chunk(void* out,                      /* device [T, Hq, D] dtype */
                   float* lse_out,                 /* device [T, Hq] or NULL */
                   const void* q,                  /* device [T, Hq, D] dtype */
                   const void* k_pool, const void* v_pool, /* device [NP, Hkv, BS, D] */
                   const int32_t* block_tables,    /* device [S, max_blocks_per_seq] */
                   int32_t max_blocks_per_seq,
                   const int32_t* cu_q_lens,       /* device [S+1] */
                   const int32_t* cu_q_lens_host,  /* host [S+1], same values */
                   const int32_t* context_lens,    /* device [S] */
                   const int32_t* context_lens_host, /* host [S], same values */
                   int32_t num_segments, int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim,
                   int32_t block_size, int64_t num_pages, float scale, pa_dtype dtype, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Mixed batch over an fp8 cache: pa_mixed_chunk's segments, causal rule and
 * result over pa_decode_fp8's pools -- e4m3fn codes with one float32 scale
 * per (page, kv-head, slot) for K and one for V (tokenspeed 딥다이브 section
 * 6-4); q and out bf16.  The chunk tiles read 64-key code tiles, widen them
 * exactly to bf16 for the matrix cores and apply each key's K scale to its
 * scores and its V scale to the probability P.V takes; decode tokens run on
 * the fp8 stream wave, in the same launch as the chunks with 4 or more
 * q-heads per kv-head.  A batch without chunks takes pa_decode_fp8's plan.
 * Workspace: pa_mixed_chunk_workspace_size.  Built for head_dim 128,
 * gqa_ratio 1, 2, 4, 8, 16.  Errors as pa_mixed_chunk, plus PA_EINVAL for a
 * NULL scale pointer.
 * ------------------------------------------------------------------------- */
int pa_mixed_chunk_fp8(void* out,                      /* device [T, Hq, D] bf16 */
                       float* lse_out,                 /* device [T, Hq] or NULL */
                       const void* q,                  /* device [T, Hq, D] bf16 */
                       const void* k_pool, const void* v_pool, /* device [NP, Hkv, BS, D] e4m3fn codes */
                       const float* k_scales, const float* v_scales, /* device [NP, Hkv, BS] */
                       const int32_t* block_tables,    /* device [S, max_blocks_per_seq] */
                       int32_t max_blocks_per_seq,
                       const int32_t* cu_q_lens,       /* device [S+1] */
                       const int32_t* cu_q_lens_host,  /* host [S+1], same values */
                       const int32_t* context_lens,    /* device [S] */
                       const int32_t* context_lens_host, /* host [S], same values */
                       int32_t num_segments, int32_t num_kv_heads, int32_t gqa_ratio, int32_t head_dim,
                       int32_t block_size, int64_t num_pages, float scale, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ---------------------------------------------------------------------------
 * KV append: write this step's new K/V rows into the paged cache, the step
 * that runs before attention each decode or prefill step.  The block table
 * names where a sequence's rows live, its blocks being handed out as the
 * sequence grows (SwiftLLM page, section 3.1); the segments and lengths are
 * those of pa_mixed_chunk (device + host copies, no defaults: TokenSpeed
 * deep-dive section 8.2).
 *
 * Segment s adds n = cu_q_lens[s+1] - cu_q_lens[s] >= 0 tokens, rows
 * cu_q_lens[s] .. cu_q_lens[s+1]-1 of k_new / v_new, and holds
 * context_lens[s] >= n rows counting them.  Its new token i is row
 * pos = context_lens[s] - n + i: for every kv-head g,
 *   k_pool[block_tables[s][pos / block_size]][g][pos % block_size][:] =
 *       k_new[cu_q_lens[s] + i][g][:]
 * and the same for V; values are copied bit for bit, every other pool row
 * is left as it is.  A table entry outside [0, num_pages) is not written
 * through (device-side tables are not checked on this path; see
 * pa_check_block_tables).  Segments must not map two tokens to one row.
 * k_pool / v_pool are written in place; k_new / v_new are read only; the
 * launch is asynchronous on `stream`; nothing is allocated.
 * head_dim * element size must be a multiple of 16 bytes and at most 512;
 * block_size 16; dtype PA_F32 or PA_BF16.
 * Returns PA_OK (num_segments == 0 or no new token: no launch), PA_EINVAL
 * (null pointer, non-positive sizes, cu_q_lens[0] != 0, n < 0,
 * context_lens[s] < n or > max_blocks_per_seq * block_size),
 * PA_EUNSUPPORTED (shape or dtype), PA_EHIP (launch).
 * ------------------------------------------------------------------------- */
int pa_kv_append(void* k_pool, void* v_pool,        /* device [NP, Hkv, BS, D] dtype, updated in place */
                 const void* k_new, const void* v_new, /* device [T, Hkv, D] dtype */
                 const int32_t* block_tables,       /* device [S, max_blocks_per_seq] */
                 int32_t max_blocks_per_seq,
                 const int32_t* cu_q_lens,          /* device [S+1] */
                 const int32_t* cu_q_lens_host,     /* host [S+1], same values */
                 const int32_t* context_lens,       /* device [S] */
                 const int32_t* context_lens_host,  /* host [S], same values */
                 int32_t num_segments, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                 int64_t num_pages, pa_dtype dtype, void* stream);

/* ---------------------------------------------------------------------------
 * KV append into an fp8 cache: pa_kv_append's placement (segments, rows,
 * table entries outside the pool not written through), with each new K row
 * and each new V row of each kv-head quantised on its own by the
 * token-group FP8 recipe of the tokenspeed 딥다이브 page (section 6-4):
 *   scale = max(max_d |x_d|, 1e-10) / 448,
 *   code_d = e4m3fn(clamp(x_d / scale, -448, 448)),
 * in float32 with correctly rounded division, rounding to the nearest
 * e4m3fn value (ties to even).  The codes go to the row of k_pool / v_pool
 * and the scale to the same (page, kv-head, slot) of k_scales / v_scales --
 * the layout pa_decode_fp8 reads.
 *
 *  k_pool, v_pool     [NP, Hkv, 16, D] uint8 codes, updated in place
 *  k_scales, v_scales [NP, Hkv, 16] float32, updated in place
 *  k_new, v_new       [T, Hkv, D] new_dtype (PA_BF16 or PA_F32)
 * head_dim 64 or 128; errors as pa_kv_append (PA_EINVAL also for a NULL
 * scale pointer).
 * ------------------------------------------------------------------------- */
int pa_kv_append_fp8(void* k_pool, void* v_pool, float* k_scales, float* v_scales, const void* k_new,
                     const void* v_new, const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* cu_q_lens, const int32_t* cu_q_lens_host, const int32_t* context_lens,
                     const int32_t* context_lens_host, int32_t num_segments, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int64_t num_pages, pa_dtype new_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Host-side table check (host copies only, no device access).
 * Every sequence needs ceil(L/block_size) entries in [0, num_pages); a page
 * may appear in more than one table only as a declared shared prefix: for
 * each group g, sequences [group_seq_offsets[g], group_seq_offsets[g+1])
 * must all start with the same prefix_lens[g] / block_size pages, and
 * prefix_lens[g] must be a multiple of block_size and shorter than every
 * member's context.  num_groups = 0 (offsets/prefix NULL) means no sharing.
 * Returns PA_OK or PA_EINVAL with the first problem in pa_last_error().
 * ------------------------------------------------------------------------- */
int pa_check_block_tables(const int32_t* block_tables_host, int32_t max_blocks_per_seq,
                          const int32_t* context_lens_host, int32_t num_seqs, int32_t block_size,
                          int64_t num_pages, int32_t num_groups, const int32_t* group_seq_offsets_host,
                          const int32_t* prefix_lens_host);

/* ---------------------------------------------------------------------------
 * Shared-prefix detection for pa_prefix_cascade (host only, no device
 * access): the greedy search the Tokasaurus page runs before each forward
 * pass ("dynamic prefix identification").  Shared-prefix blocks are stored
 * once and named by every table that shares them (SwiftLLM page section
 * 3.1), so sequences share their first d pages when their first d table
 * entries are equal.  Each round picks, over a trie of the tables' page ids,
 * the longest prefix (the page's rule) among prefixes of >= min_prefix_pages
 * pages, shorter than every member's context and held by >= min_group (at
 * least 2) sequences not yet grouped (ties: the prefix with more such
 * sequences, then the one met first when the tables are read in order);
 * those sequences become a group.  The rest form a last group with prefix
 * 0.
 *
 * Outputs (host, caller-owned): order_out[num_seqs] -- original sequence
 * index at each position, group by group (groups in the order found,
 * members by original index); group_offsets_out[num_seqs + 1] and
 * prefix_lens_out[num_seqs] -- pa_prefix_cascade's groups over the sequences
 * taken in that order; *num_groups_out.  Returns PA_OK, or PA_EINVAL for
 * null pointers, negative sizes or a context length < 1 or beyond the
 * table.
 * ------------------------------------------------------------------------- */
int pa_detect_prefix_groups(const int32_t* block_tables_host, int32_t max_blocks_per_seq,
                            const int32_t* context_lens_host, int32_t num_seqs, int32_t block_size,
                            int32_t min_group, int32_t min_prefix_pages, int32_t* order_out,
                            int32_t* group_offsets_out, int32_t* prefix_lens_out, int32_t* num_groups_out);

/* Message for the last non-OK return on this thread ("" if none). */
const char* pa_last_error(void);

/* ---------------------------------------------------------------------------
 * Profiling hook (measurement only; changes no result).  A test and
 * benchmark hook, not part of the hot path: pa_profile_enable allocates
 * HIP events and both calls keep thread-local state, so they are neither
 * allocation-free nor reentrant.
 * pa_profile_enable(n) creates n pairs of HIP timing events on this thread;
 * every later call records one pair around each of its dominant kernels on
 * its stream: the stream kernel of the decode entry points (one pair per
 * pass of a multi-token call); the prefix kernel of pa_prefix_cascade and
 * pa_prefix_cascade_fp8; for pa_mixed_chunk and pa_mixed_chunk_fp8, the
 * one-launch mixed kernel, or, when the batch runs as separate launches,
 * the chunk kernel(s) (if it has chunks) and then the decode stream kernel
 * (if it has decode tokens).  pa_profile_collect() waits for those events,
 * writes up to `cap` durations in milliseconds to `ms_out`, returns how
 * many it wrote and rewinds the ring.  pa_profile_enable(0) frees the
 * events and stops recording.  Returns a negative code on error.
 * ------------------------------------------------------------------------- */
int pa_profile_enable(int32_t num_pairs);
int pa_profile_collect(float* ms_out, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
