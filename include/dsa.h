/*
 * dsa.h -- C ABI of libdsa.so: one DSA sparse decode step on an MI355X (gfx950).
 *
 * The step (page "[ROCm] Support decode context parallel (DCP) for GLM-5 /
 * DeepSeek-V3.2", sgl-project/sglang PR #42618, sections Motivation and
 * Modifications):
 *   1. dsa_index_scores      fp8 indexer score of every visible cached token
 *                            (the bf16 queries quantized as dsa_quantize_q does)
 *   2. dsa_topk              exact top-k per row: per-split local top-k, then an
 *                            exact merge of the candidates
 *   3. dsa_sparse_mla_decode absorbed-MLA attention over the selected paged fp8
 *                            rows, split along the selected list into
 *                            (partial output, natural-log LSE) pairs
 *   4. dsa_lse_merge         merge of the split partials by their LSE
 * dsa_index_topk runs steps 1 and 2 for decode rows with the top-k's
 * candidate filter in the indexer's epilogue (same results as the two calls).
 * dsa_quantize_q exposes the query quantization of step 1 on its own.
 * dsa_cache_write is the step before the path: it stores new tokens' MLA rows
 * and index keys in the paged caches the four steps read.
 * dsa_lse_merge_project is the step after it: step 4 followed by the value
 * projection W_UV, in one launch.
 *
 * Conventions shared by every entry point:
 *  - Every array pointer is DEVICE memory owned by the caller.  The library
 *    never allocates, never frees, never synchronises and never falls back to
 *    another path.  Calls are enqueued on `stream` in order and return before
 *    the work runs; they are stateless and may be called from several threads.
 *  - All arrays are dense row-major with the shapes given per call.
 *  - The return value is the HOST validation status: DSA_OK (0) when the work
 *    was enqueued, a negative DSA_ERR_* otherwise, in which case nothing was
 *    enqueued.  dsa_status_string() names every code.
 *  - Kernels check what only the device can see (page ids, row geometry,
 *    top-k indices).  A violation ORs a DSA_DEV_* bit into the caller's int32
 *    `status` word (device memory, not cleared by the library) and nothing is
 *    read out of bounds.  Each call writes a row whose geometry it finds
 *    inconsistent as empty (dsa_index_scores: scores -inf; dsa_topk: count
 *    0; dsa_sparse_mla_decode: output 0, lse -inf); a call checks what its
 *    arguments show (only dsa_index_scores sees kv_lens).  A token on an
 *    invalid page scores -inf; a selected entry outside its row's span or on
 *    an invalid page is left out of the attention (the row attends the
 *    others).  Once a bit is set, the step's results are not to be used.
 *  - Page pool layout: NP pages of P tokens.  Indexer keys: k_code uint8
 *    [NP, P, 128] (E4M3FN codes) and k_scale float32 [NP, P].  MLA rows:
 *    kv_cache uint8 [NP, P, 640], one 640-byte row per token: bytes
 *    0..575 the E4M3FN codes (512 latent then 64 rope), bytes 576..579 the
 *    token's fp32 scale (little-endian), bytes 580..639 unused.  A token's
 *    value is code * its scale.  The scale shares the row so that a gathered
 *    token costs exactly the five 128-byte lines of its row.
 *  - Block table: page_table int32 [batch, max_pages]; logical slot t of
 *    request b lives at physical row page_table[b][t / P] * P + t % P.
 *    Entries past a request's span are -1 (page "DeepSeek V4 DSpark
 *    Internals", kernel mapping).
 *  - Rows are query tokens: row r belongs to request row_req[r] and sees the
 *    slots [0, row_vis[r]) of it (causal rows of MTP verify and prefill see
 *    fewer than kv_len).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 12

/* Host validation status (return value of every entry point). */
enum {
    DSA_OK = 0,
    DSA_ERR_NULL = -1,        /* a required pointer is NULL */
    DSA_ERR_SHAPE = -2,       /* a size, stride or count is out of range or inconsistent */
    DSA_ERR_UNSUPPORTED = -3, /* valid but not built: head count, head dim, page size */
    DSA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than the size query */
    DSA_ERR_LAUNCH = -5,      /* the HIP runtime refused a launch */
    DSA_ERR_SCRATCH = -6      /* dsa_topk_noalloc: the call needs more than DSA_NOALLOC_SCRATCH_BYTES */
};

/* Bits ORed by kernels into the caller's device status word. */
enum {
    DSA_DEV_PAGE_OOB = 1,   /* a slot inside a row's span maps to a page id < 0 or >= num_pages */
    DSA_DEV_TOPK_OOB = 2,   /* a selected index is < 0 or >= row_vis, or top-k count out of range */
    DSA_DEV_ROW_RANGE = 4,  /* row_req out of [0, batch), or row_vis < 0, > kv_len,
                               > max_pages * page_size or > score_stride */
    DSA_DEV_GROUP = 8,      /* rows of one scoring group belong to different requests */
    DSA_DEV_NAN = 16,       /* a NaN score reached the top-k (ordered, but reported) */
    DSA_DEV_WRITE = 32,     /* a new token's request, slot or position is out of range */
    DSA_DEV_SCALE = 64      /* a key or MLA row read for a row has a scale that is not a
                               positive finite number; that token is left out (score -inf,
                               not attended) */
};

/*
 * dsa_cache_write -- new tokens into the paged caches (subject page,
 * Modifications: writes and the fused rope + KV-cache write; Future work:
 * the write location computed once per step inside the write kernel).
 * Token i of request tok_req[i] is stored at logical slot t = tok_slot[i]
 * (its position), physical row page_table[b][t / P] * P + t % P:
 *   MLA row: the 512 latent entries, then the 64 rope entries with pair
 *     (2j, 2j+1) of a token at position t turned by c = rope_cos[t][j],
 *     s = rope_sin[t][j]:  y0 = x0*c - x1*s,  y1 = x0*s + x1*c  (each product
 *     and the sum rounded to fp32 on its own); no rotation when both tables
 *     are NULL.  Codes E4M3FN of clamp(x / scale, +-448) rounded to nearest
 *     even, scale = max|x| / 448 in fp32 (1 for an all-zero row), into bytes
 *     0..575 of the row, the scale at bytes 576..579; bytes 580..639 are not
 *     written.
 *   index key: its 128 entries, unrotated, quantized the same way into
 *     k_code[row] with k_scale[row].
 *   latent [n_tok, 512], rope [n_tok, 64], index_k [n_tok, 128] bf16 bit
 *     patterns, 16-byte aligned rows; rope_cos, rope_sin [max_pos, 32] f32 or
 *     both NULL; tok_req, tok_slot [n_tok] i32; page_table [batch, max_pages].
 *   kv_cache [num_pages, page_size, 640] u8, k_code [num_pages, page_size,
 *     128] u8, k_scale [num_pages, page_size] f32: written in place.
 * A token whose request is out of [0, batch), whose slot is out of
 * [0, max_pages * page_size) or whose position is >= max_pos (with tables)
 * writes nothing and sets DSA_DEV_WRITE; one whose page id is out of
 * [0, num_pages) writes nothing and sets DSA_DEV_PAGE_OOB.  Two tokens with
 * the same destination leave either one's row.  n_tok == 0 enqueues nothing
 * and reads no array (its pointers may be NULL).
 */
int dsa_cache_write(const uint16_t* latent, const uint16_t* rope, const uint16_t* index_k,
                    const float* rope_cos, const float* rope_sin, int32_t max_pos,
                    const int32_t* tok_req, const int32_t* tok_slot, int32_t n_tok,
                    const int32_t* page_table, int32_t batch, int32_t num_pages, int32_t max_pages,
                    int32_t page_size, uint8_t* kv_cache, uint8_t* k_code, float* k_scale,
                    int32_t* status, hipStream_t stream);

/*
 * dsa_lse_merge_project -- the LSE merge of step 4 followed by the value
 * projection of absorbed MLA (subject page, Future work: projecting V before
 * the LSE merge; the projection is linear and the merge weights add to one,
 * so merging first and projecting once gives the same values):
 *   latent[r,h] = merge of part_o[r,h,:] by part_lse[r,h,:] as dsa_lse_merge,
 *                 then rounded to bf16 (nearest even)
 *   out[r,h,d]  = sum_k latent[r,h,k] * w_uv[h][d][k]   (fp32 accumulation,
 *                 rounded to bf16)
 *   out_lse[r,h] as dsa_lse_merge (may be NULL).
 *   part_o [n_rows, n_heads, n_splits, d_latent] bf16 bit patterns (16-byte aligned),
 *   part_lse [n_rows, n_heads, n_splits] f32, w_uv [n_heads, d_v, d_latent]
 *   bf16 (16-byte aligned; each output dimension's weights one contiguous
 *   row), out [n_rows, n_heads, d_v] bf16.
 * A row no split saw gives out = 0 and lse = -inf.
 * Supported: d_latent == 512, d_v == 128, 1 <= n_splits <= 64.
 */
int dsa_lse_merge_project(const uint16_t* part_o, const float* part_lse, int32_t n_rows, int32_t n_heads,
                          int32_t n_splits, int32_t d_latent, const uint16_t* w_uv, int32_t d_v,
                          uint16_t* out, float* out_lse, hipStream_t stream);

/*
 * DSA_ABI_VERSION of the built library; loaders refuse a mismatch.  The
 * version check follows the narrow native ABI of page "Harden DeepSeek V4
 * DSpark DP2 serving" (section 4.1: the loader requires an exact ABI version
 * and geometry; section 4.3 warning: a missing library or a wrong ABI aborts
 * the path, with no fallback).
 */
int dsa_abi_version(void);

/*
 * Static, never-NULL name of a DSA_OK / DSA_ERR_* code ("unknown" otherwise),
 * so that a binding can turn every native error into an exception with a
 * readable message (same page, section 4.1: any native error becomes a Python
 * exception).
 */
const char* dsa_status_string(int status);

/*
 * dsa_quantize_q -- input side of the fp8 indexer.
 * The subject page's indexer scores fp8 keys; the query arrives as bf16, so it
 * is brought to fp8 E4M3FN with one power-of-two scale per (row, head):
 * scale = 2^ceil(log2(amax / 448)) (scale 1 for an all-zero head) and
 * code = round-to-nearest-even(q / scale).  dsa_index_scores quantizes its
 * queries the same way, bit for bit.
 *   q_bf16   [n_rows, n_heads, head_dim] bf16 bit patterns
 *   q_code   [n_rows, n_heads, head_dim] uint8 out
 *   q_scale  [n_rows, n_heads] float32 out
 * Supported: head_dim == 128, n_heads >= 1.  n_rows == 0 enqueues nothing.
 */
int dsa_quantize_q(const uint16_t* q_bf16, int32_t n_rows, int32_t n_heads, int32_t head_dim,
                   uint8_t* q_code, float* q_scale, hipStream_t stream);

/*
 * dsa_index_scores -- fp8 lightning-indexer scores (subject page,
 * Modifications, indexer decode: the index-K cache is scored per token).
 *   scores[r][t] = k_scale[t] * sum_h (head_w[r][h] * q_scale[r][h])
 *                  * relu( dec(q_code[r][h]) . dec(k_code[t]) )     for t < row_vis[r]
 * with (q_code, q_scale) = dsa_quantize_q of q,
 *   scores[r][t] = -inf                      for row_vis[r] <= t < score_stride
 * which equals sum_h w_h * relu(q_h . k_t) for positive scales.
 *   q [n_rows, 64, 128] bf16 bit patterns, head_w [n_rows, 64] f32
 *   k_code [num_pages, page_size, 128] uint8, k_scale [num_pages, page_size] f32
 *   page_table [batch, max_pages] i32, kv_lens [batch] i32
 *   row_req [n_rows] i32, row_vis [n_rows] i32
 *   scores [n_rows, score_stride] f32 out
 * group_rows (1..8, dividing n_rows): that many consecutive rows are scored
 * against one stream of keys (MTP verify and prefill rows of one request);
 * all rows of a group must share a request, else DSA_DEV_GROUP.
 * flags: 0, or DSA_INDEX_WHOLE_ROWS with group_rows == 1: the caller knows
 * (from the lengths it holds on the host) that every row's span is at least
 * three quarters of score_stride, so the launch streams keys on the whole
 * chip to its end; the keys are then read as whole 128-byte rows with the
 * non-temporal hint (faster there, slower for ragged rows).  The scores are
 * the same either way.  Other bits: DSA_ERR_SHAPE.
 * Supported: n_heads == 64, head_dim == 128, page_size a power of two in
 * [16, 1024].  All scales must be finite and > 0.
 */
#define DSA_INDEX_WHOLE_ROWS 1
int dsa_index_scores(const uint16_t* q, const float* head_w,
                     const uint8_t* k_code, const float* k_scale, const int32_t* page_table,
                     const int32_t* kv_lens, const int32_t* row_req, const int32_t* row_vis,
                     int32_t n_rows, int32_t batch, int32_t num_pages, int32_t max_pages,
                     int32_t page_size, int32_t n_heads, int32_t head_dim, int32_t group_rows,
                     int32_t flags, float* scores, int32_t score_stride, int32_t* status,
                     hipStream_t stream);

/*
 * dsa_index_topk -- steps 1 and 2 for decode rows (one row per scoring
 * group): the scores of dsa_index_scores with group_rows = 1, and the top-k
 * of dsa_topk over them, bit for bit (subject page, Modifications, indexer
 * decode: local top-k per shard merged into the exact global top-k).
 * The indexer scores each row in chunks of tokens, one workgroup each; while
 * a chunk's scores are still on chip, the workgroup keeps its candidates:
 * every visible score at or above a cut of its own, placed near the rank of
 * the chunk's expected share of the row's top top_k plus four standard
 * deviations.  A merge per row then selects the top top_k of the
 * candidates, after checking that at least top_k of them lie at or above the
 * highest chunk cut, which makes them hold the row's top top_k; a row that
 * fails the check (scores far from exchangeable across chunks, many equal
 * scores) is selected from its scores instead (slower, same result).
 *   arguments as dsa_index_scores (group_rows fixed to 1) and dsa_topk;
 *   scores [n_rows, score_stride] f32 out (as dsa_index_scores)
 *   topk_idx [n_rows, top_k] i32 out, topk_count [n_rows] i32 out (as dsa_topk)
 *   workspace: dsa_index_topk_workspace_size(n_rows, score_stride, top_k)
 *   bytes of device memory, 4-byte aligned, else DSA_ERR_WORKSPACE; its
 *   contents need no initialisation and are not results.
 * phases: DSA_PHASE_SCORE | DSA_PHASE_SELECT runs both (the normal call);
 * DSA_PHASE_SCORE alone writes the scores and the candidates in the
 * workspace; DSA_PHASE_SELECT alone runs the merge over the candidates and
 * scores a previous DSA_PHASE_SCORE call with the same arguments left there
 * (the two halves can be timed or scheduled apart).  Other values:
 * DSA_ERR_SHAPE.
 * Device status bits: those of dsa_index_scores and dsa_topk (DSA_DEV_NAN
 * for a NaN score inside a row's span).
 * Limits: 1 <= top_k <= 8192; the indexer's chunks per row (score_stride
 * over its chunk length of 1024 to 8192 tokens) at most 1024.
 */
#define DSA_PHASE_SCORE 1
#define DSA_PHASE_SELECT 2
size_t dsa_index_topk_workspace_size(int32_t n_rows, int32_t score_stride, int32_t top_k);
int dsa_index_topk(const uint16_t* q, const float* head_w, const uint8_t* k_code, const float* k_scale,
                   const int32_t* page_table, const int32_t* kv_lens, const int32_t* row_req,
                   const int32_t* row_vis, int32_t n_rows, int32_t batch, int32_t num_pages, int32_t max_pages,
                   int32_t page_size, int32_t n_heads, int32_t head_dim, float* scores, int32_t score_stride,
                   int32_t top_k, int32_t phases, void* workspace, size_t workspace_bytes,
                   int32_t* topk_idx, int32_t* topk_count, int32_t* status, hipStream_t stream);

/*
 * Workspace bytes dsa_topk needs for n_splits > 1: room for top_k candidate
 * keys and slots per split and row; per split and row a count, the cut, the
 * top of the kept-key histogram and a 512-bin histogram (all 32-bit).  0 when
 * n_splits == 1.  The contents are internal to the call.  The caller
 * reserves the workspace once, up front, and a call with a smaller one is
 * rejected (DSA_ERR_WORKSPACE) rather than served by an allocation (page
 * "Harden DeepSeek V4 DSpark DP2 serving", section 6.3: workspaces reserved
 * before graph capture, whose slices reject capacity or geometry changes).
 */
size_t dsa_topk_workspace_size(int32_t n_rows, int32_t top_k, int32_t n_splits);

/*
 * dsa_topk -- exact top-k per row under the total order (score descending,
 * slot ascending), so equal scores keep the lower slot (subject page,
 * Motivation: the top 2048 of the whole sequence; Modifications, indexer
 * decode: local top-k per shard merged into the exact global top-k).
 * n_splits == 1 selects directly, one workgroup per row.  n_splits > 1 cuts
 * row r's slots [0, row_vis[r]) into n_splits contiguous ranges of
 * ceil(row_vis/n_splits) rounded up to a multiple of 4 (the last ranges may
 * be short or empty), one workgroup each.  Each range keeps its candidates:
 * the scores at or above one cut that every range of the row derives alike
 * from a strided sample of the whole row, or its own top top_k when more
 * than top_k of its scores pass the cut.  One merge per row selects the top
 * top_k of the candidates, which is the row's top top_k whenever at least
 * top_k are kept; when the cut kept fewer, the merge selects from the row's
 * scores directly (slower, same result).
 * Score rows whose start is 16-byte aligned (score_stride a multiple of 4)
 * are read in 16-byte loads; nothing outside [0, row_vis) of a row is used,
 * and nothing past the row's score_stride entries is read.
 *   scores [n_rows, score_stride] f32 (only [0, row_vis) is read)
 *   topk_idx [n_rows, top_k] i32 out: selected slots in ascending order, then -1
 *   topk_count [n_rows] i32 out: min(top_k, row_vis)
 * Limits: 1 <= top_k <= 8192; ceil(score_stride / n_splits) <= 32768;
 * n_splits * top_k <= 32768 when n_splits > 1; n_splits <= 64.
 */
int dsa_topk(const float* scores, int32_t score_stride, const int32_t* row_vis, int32_t n_rows,
             int32_t top_k, int32_t n_splits, void* workspace, size_t workspace_bytes,
             int32_t* topk_idx, int32_t* topk_count, int32_t* status, hipStream_t stream);

/*
 * dsa_topk_rows -- dsa_topk that also emits, for each selected slot, its
 * physical row in the paged caches (subject page, Modifications, indexer
 * decode: the merge emits the KV rows directly, so the attention needs no
 * per-layer page-table transform).  The selection, topk_idx and topk_count
 * are dsa_topk's, bit for bit; in addition
 *   topk_rows [n_rows, top_k] i32 out: page_table[b][t / page_size] *
 *     page_size + t % page_size for each selected slot t of row r (b =
 *     row_req[r]), -1 after topk_count[r].
 * A slot whose page id lies outside [0, num_pages) gets -1 and
 * DSA_DEV_PAGE_OOB; a row whose request lies outside [0, batch), or whose
 * span exceeds max_pages * page_size, gets -1 rows and DSA_DEV_ROW_RANGE.
 * The block-table row of each request is read once per row.
 *   row_req [n_rows] i32, page_table [batch, max_pages] i32 (as for the
 *   attention); other arguments, limits and the workspace as dsa_topk.
 */
int dsa_topk_rows(const float* scores, int32_t score_stride, const int32_t* row_vis, const int32_t* row_req,
                  const int32_t* page_table, int32_t batch, int32_t num_pages, int32_t max_pages, int32_t page_size,
                  int32_t n_rows, int32_t top_k, int32_t n_splits, void* workspace, size_t workspace_bytes,
                  int32_t* topk_idx, int32_t* topk_count, int32_t* topk_rows, int32_t* status, hipStream_t stream);

/*
 * dsa_topk_noalloc -- dsa_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, rules and results as dsa_topk, without the
 * workspace: the candidates of a split call (n_splits > 1) live in a fixed
 * array of DSA_NOALLOC_SCRATCH_BYTES that the library holds in device memory,
 * one per GPU, from the first call on that GPU until the process ends.  The
 * call allocates nothing.
 * Limit: dsa_topk_workspace_size(n_rows, top_k, n_splits) must not exceed
 * DSA_NOALLOC_SCRATCH_BYTES, else DSA_ERR_SCRATCH and nothing is enqueued
 * (16 MiB holds n_rows * n_splits * top_k up to 2^21 candidates).  The array
 * keeps the last call's contents; nothing in it needs to start at zero.
 * Every call on one GPU shares that GPU's array: calls that may overlap on one
 * GPU (other streams, other threads) race and must be ordered by the caller.
 * DSA_ERR_LAUNCH if the array's device address cannot be looked up.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int dsa_topk_noalloc(const float* scores, int32_t score_stride, const int32_t* row_vis, int32_t n_rows,
                     int32_t top_k, int32_t n_splits, int32_t* topk_idx, int32_t* topk_count,
                     int32_t* status, hipStream_t stream);

/*
 * dsa_sparse_mla_decode -- split-K absorbed-MLA attention over each row's
 * selected slots (subject page, Modifications, sparse decode: the split-K
 * kernel attends the selected slots and also returns the LSE; the per-row
 * selected count bounds the work; a lone split writes the final output and
 * natural-log LSE directly).
 * For row r, head h, split s over entries [s*c, min(n, (s+1)*c)) of
 * topk_idx[r] with n = topk_count[r], c = ceil(top_k / n_splits) (fixed by
 * top_k, so a split's range is known before the count is read; when
 * n < top_k the last splits may be empty):
 *   x_t   = dec(codes of row t) * scale of row t       (576 wide)
 *   l_t   = sm_scale * (q[r][h] . x_t)     (q the exact bf16 values)
 *   o_s   = sum_t e^{l_t - m} x_t[0:512] / sum_t e^{l_t - m},  lse_s = m + ln sum_t e^{l_t - m}
 * Empty split: o_s = 0, lse_s = -inf.
 *   q [n_rows, n_heads, 576] bf16 bit patterns
 *   kv_cache [num_pages, page_size, 640] uint8 (layout above)
 *   page_table [batch, max_pages] i32, row_req / row_vis [n_rows] i32
 *   topk_idx [n_rows, top_k] i32, topk_count [n_rows] i32
 * n_splits == 1: writes out [n_rows, n_heads, 512] bf16 (round to nearest
 *   even) and, if out_lse != NULL, out_lse [n_rows, n_heads] f32; part_* unused.
 * n_splits > 1: writes part_o [n_rows, n_heads, n_splits, 512] bf16 bit
 *   patterns (o_s rounded to nearest even; 4-byte aligned, else
 *   DSA_ERR_SHAPE) and part_lse [n_rows, n_heads, n_splits] f32; out /
 *   out_lse unused (dsa_lse_merge finishes the row).
 * Supported: n_heads in {16, 32}, page_size a power of two in [16, 1024],
 * 1 <= n_splits <= 64, 1 <= top_k <= 8192.
 */
int dsa_sparse_mla_decode(const uint16_t* q, const uint8_t* kv_cache, const int32_t* page_table,
                          const int32_t* row_req, const int32_t* row_vis, const int32_t* topk_idx,
                          const int32_t* topk_count, int32_t n_rows,
                          int32_t batch, int32_t num_pages, int32_t max_pages, int32_t page_size,
                          int32_t n_heads, int32_t top_k, int32_t n_splits, float sm_scale,
                          uint16_t* part_o, float* part_lse, uint16_t* out, float* out_lse,
                          int32_t* status, hipStream_t stream);

/*
 * dsa_sparse_mla_decode_rows -- dsa_sparse_mla_decode over lists of physical
 * rows (dsa_topk_rows' topk_rows) instead of slots: no block table is read,
 * so the gathers start as soon as a split's entries arrive (subject page,
 * Modifications, indexer decode: the merge emits the KV rows directly).
 * Row r attends the rows topk_rows[r][0 .. topk_count[r]) with the same
 * splits, arithmetic and outputs as dsa_sparse_mla_decode; given the rows
 * dsa_topk_rows emits for a selection, the results equal
 * dsa_sparse_mla_decode's on that selection, bit for bit.  An entry of -1
 * (a slot on an invalid page, already reported by the top-k) is left out; an
 * entry below -1 or at or past num_pages * page_size is left out and sets
 * DSA_DEV_TOPK_OOB; a count above top_k or row_vis[r] empties the row
 * (DSA_DEV_TOPK_OOB).
 *   q, kv_cache, outputs, limits: as dsa_sparse_mla_decode
 *   row_vis [n_rows] i32 (bounds the count), topk_rows [n_rows, top_k] i32,
 *   topk_count [n_rows] i32
 */
int dsa_sparse_mla_decode_rows(const uint16_t* q, const uint8_t* kv_cache, const int32_t* row_vis,
                               const int32_t* topk_rows, const int32_t* topk_count, int32_t n_rows,
                               int32_t num_pages, int32_t page_size, int32_t n_heads, int32_t top_k,
                               int32_t n_splits, float sm_scale, uint16_t* part_o, float* part_lse, uint16_t* out,
                               float* out_lse, int32_t* status, hipStream_t stream);

/*
 * dsa_sparse_mla_decode_shared -- dsa_sparse_mla_decode where rows share
 * selected lists (subject page, Modifications, "MTP / EAGLE", and the
 * chain-EAGLE commit note: the index can be shared across MTP iterations,
 * an option the page switches off only under DCP).  The chain of draft rows
 * of one request runs the indexer and the top-k once, for its first row,
 * and every row of the chain attends that list with its own query.
 * Row r attends list l = row_list[r]: the first topk_count[l] entries of
 * topk_idx[l], exactly as dsa_sparse_mla_decode attends row r's own list
 * (same splits, outputs, checks).  An entry outside row r's span is left out
 * (DSA_DEV_TOPK_OOB); a list count above row r's span, or l outside
 * [0, n_lists), writes row r empty (DSA_DEV_TOPK_OOB / DSA_DEV_ROW_RANGE).
 *   row_list [n_rows] i32; topk_idx [n_lists, top_k] i32; topk_count
 *   [n_lists] i32; every other argument as dsa_sparse_mla_decode.
 * When n_lists divides n_rows into chains of 2..16 consecutive rows, each
 * chain's work runs on one XCD of the chip, so the rows it shares are read
 * from HBM about once; any row_list gives the same results.
 */
int dsa_sparse_mla_decode_shared(const uint16_t* q, const uint8_t* kv_cache, const int32_t* page_table,
                                 const int32_t* row_req, const int32_t* row_vis, const int32_t* row_list,
                                 const int32_t* topk_idx, const int32_t* topk_count, int32_t n_lists,
                                 int32_t n_rows, int32_t batch, int32_t num_pages, int32_t max_pages,
                                 int32_t page_size, int32_t n_heads, int32_t top_k, int32_t n_splits,
                                 float sm_scale, uint16_t* part_o, float* part_lse, uint16_t* out, float* out_lse,
                                 int32_t* status, hipStream_t stream);

/*
 * dsa_lse_merge -- merge split partials by their natural-log LSE (subject
 * page, split-K commit note: the reduce can also store the natural-log LSE).
 *   lse = ln sum_s e^{lse_s};  out = sum_s e^{lse_s - lse} o_s
 * Splits with lse_s = -inf are skipped; a row with no finite lse_s gets
 * out = 0 and lse = -inf.
 *   part_o [n_rows, n_heads, n_splits, d_v] bf16 bit patterns, part_lse [n_rows, n_heads, n_splits] f32
 *   out [n_rows, n_heads, d_v] bf16 (round to nearest even)
 *   part_o and out 16-byte aligned, else DSA_ERR_SHAPE
 *   out_lse [n_rows, n_heads] f32, may be NULL
 * Supported: d_v == 512, 1 <= n_splits <= 64.
 */
int dsa_lse_merge(const uint16_t* part_o, const float* part_lse, int32_t n_rows, int32_t n_heads,
                  int32_t n_splits, int32_t d_v, uint16_t* out, float* out_lse, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
