// C ABI of libdsa.so: host-side validation, then the launchers.
//
// Every check here runs before any HIP call, so a rejected call touches
// neither the device nor the stream.  Rules follow include/dsa.h.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "dsa.h"
#include "launch.h"

namespace {

constexpr int32_t kMaxRows = 65535;   // one workgroup row per query row in the grid's y dimension

bool is_pow2_in(int32_t v, int32_t lo, int32_t hi) {
    return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

int log2i(int32_t v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

int launch_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH; }

int check_page_geometry(int32_t batch, int32_t num_pages, int32_t max_pages, int32_t page_size) {
    if (batch < 1 || num_pages < 1 || max_pages < 1) return DSA_ERR_SHAPE;
    if (page_size < 1) return DSA_ERR_SHAPE;
    if (!is_pow2_in(page_size, 16, 1024)) return DSA_ERR_UNSUPPORTED;
    if ((int64_t)max_pages * page_size > INT32_MAX) return DSA_ERR_SHAPE;
    if ((int64_t)num_pages * page_size > INT32_MAX) return DSA_ERR_SHAPE;
    return DSA_OK;
}

size_t topk_ws_keys(int32_t n_rows, int32_t top_k, int32_t n_splits) {
    return (size_t)n_rows * n_splits * top_k * sizeof(uint32_t);
}

// Validation and launch shared by the attention entry points: row r attends
// list row_list[r] of [n_lists, top_k] (row_list NULL: list r, n_lists ==
// n_rows).
int mla_checked(const uint16_t* q, const uint8_t* kv_cache, const int32_t* page_table, const int32_t* row_req,
                const int32_t* row_vis, const int32_t* row_list, const int32_t* topk_idx,
                const int32_t* topk_count, int32_t n_lists, int32_t n_rows, int32_t batch, int32_t num_pages,
                int32_t max_pages, int32_t page_size, int32_t n_heads, int32_t top_k, int32_t n_splits,
                float sm_scale, uint16_t* part_o, float* part_lse, uint16_t* out, float* out_lse, int32_t* status,
                hipStream_t stream, const int32_t* topk_rows = nullptr) {
    if (n_rows < 0 || n_rows > kMaxRows || n_heads < 1) return DSA_ERR_SHAPE;
    if (top_k < 1 || top_k > dsa::kTopkMaxK) return DSA_ERR_SHAPE;
    if (n_splits < 1 || n_splits > dsa::kMaxSplits) return DSA_ERR_SHAPE;
    if (!isfinite(sm_scale)) return DSA_ERR_SHAPE;
    if (n_heads != 16 && n_heads != 32) return DSA_ERR_UNSUPPORTED;
    int rc = check_page_geometry(batch, num_pages, max_pages, page_size);
    if (rc != DSA_OK) return rc;
    if (topk_rows != nullptr) {   // physical rows: no block table is read
        if (!q || !kv_cache || !row_vis || !topk_count || !status) return DSA_ERR_NULL;
    } else if (!q || !kv_cache || !page_table || !row_req || !row_vis || !topk_idx || !topk_count || !status) {
        return DSA_ERR_NULL;
    }
    if (n_splits == 1 ? !out : (!part_o || !part_lse)) return DSA_ERR_NULL;
    if (n_splits > 1 && (reinterpret_cast<uintptr_t>(part_o) & 3) != 0) return DSA_ERR_SHAPE;   // 4-byte stores
    if (n_rows == 0) return DSA_OK;
    dsa::MlaArgs a{};
    a.topk_rows = topk_rows;
    a.q = q; a.kv_cache = kv_cache; a.page_table = page_table;
    a.row_req = row_req; a.row_vis = row_vis; a.topk_idx = topk_idx; a.topk_count = topk_count;
    a.n_rows = n_rows; a.batch = batch; a.num_pages = num_pages; a.max_pages = max_pages;
    a.page_size = page_size; a.log2_page = log2i(page_size); a.n_heads = n_heads;
    a.top_k = top_k; a.n_splits = n_splits; a.sm_scale = sm_scale;
    a.part_o = part_o; a.part_lse = part_lse; a.out = out; a.out_lse = out_lse; a.status = status;
    a.row_list = row_list;
    a.n_lists = n_lists;
    // Chains of consecutive rows that share a list go to one XCD each (a
    // placement only: every row reads its own list index).
    const int32_t per = n_lists > 0 ? n_rows / n_lists : 0;
    a.chain = (row_list != nullptr && per > 1 && per <= 16 && n_rows % n_lists == 0) ? per : 1;
    return launch_status(dsa::launch_sparse_mla(a, stream));
}

// Validation of an indexer call (the rules of dsa_index_scores) and its
// arguments, filled into `a`; nothing is launched.
int index_checked(const uint16_t* q, const float* head_w, const uint8_t* k_code, const float* k_scale,
                  const int32_t* page_table, const int32_t* kv_lens, const int32_t* row_req,
                  const int32_t* row_vis, int32_t n_rows, int32_t batch, int32_t num_pages, int32_t max_pages,
                  int32_t page_size, int32_t n_heads, int32_t head_dim, int32_t group_rows, float* scores,
                  int32_t score_stride, int32_t* status, dsa::IndexArgs& a) {
    if (n_rows < 0 || n_rows > kMaxRows || score_stride < 1) return DSA_ERR_SHAPE;
    if (n_heads < 1 || head_dim < 1) return DSA_ERR_SHAPE;
    if (n_heads != 64 || head_dim != 128) return DSA_ERR_UNSUPPORTED;
    int rc = check_page_geometry(batch, num_pages, max_pages, page_size);
    if (rc != DSA_OK) return rc;
    if (group_rows < 1 || group_rows > 8) return DSA_ERR_SHAPE;
    if (n_rows % group_rows != 0) return DSA_ERR_SHAPE;
    if (!q || !head_w || !k_code || !k_scale || !page_table || !kv_lens ||
        !row_req || !row_vis || !scores || !status)
        return DSA_ERR_NULL;
    a.q = q; a.head_w = head_w;
    a.k_code = k_code; a.k_scale = k_scale; a.page_table = page_table; a.kv_lens = kv_lens;
    a.row_req = row_req; a.row_vis = row_vis;
    a.n_rows = n_rows; a.batch = batch; a.num_pages = num_pages; a.max_pages = max_pages;
    a.page_size = page_size; a.log2_page = log2i(page_size); a.group_rows = group_rows;
    a.scores = scores; a.score_stride = score_stride; a.status = status;
    a.cand_key = nullptr;
    return DSA_OK;
}

// Chunks per row of the decode indexer launch and the candidates' block
// length per chunk (a chunk keeps at most min(chunk, top_k) of them).
constexpr int32_t kMaxIndexChunks = 1024;
struct IndexTopkGeometry {
    int64_t n_chunks;
    int32_t cap;
};
IndexTopkGeometry index_topk_geometry(int32_t n_rows, int32_t score_stride, int32_t top_k) {
    const int chunk = dsa::index_chunk(n_rows, score_stride);
    return {((int64_t)score_stride + chunk - 1) / chunk, std::min(chunk, top_k)};
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_string(int status) {
    switch (status) {
        case DSA_OK: return "DSA_OK";
        case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
        case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: a size, stride or count is out of range";
        case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: head count, head dim or page size not built";
        case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
        case DSA_ERR_LAUNCH: return "DSA_ERR_LAUNCH: the HIP runtime refused a launch";
        case DSA_ERR_SCRATCH:
            return "DSA_ERR_SCRATCH: the call needs more scratch than the library's fixed buffer holds";
        default: return "unknown";
    }
}

int dsa_quantize_q(const uint16_t* q_bf16, int32_t n_rows, int32_t n_heads, int32_t head_dim,
                   uint8_t* q_code, float* q_scale, hipStream_t stream) {
    if (n_rows < 0 || n_heads < 1 || head_dim < 1) return DSA_ERR_SHAPE;
    if (head_dim != 128) return DSA_ERR_UNSUPPORTED;
    if ((int64_t)n_rows * n_heads > INT32_MAX / 4) return DSA_ERR_SHAPE;
    if (n_rows == 0) return DSA_OK;
    if (!q_bf16 || !q_code || !q_scale) return DSA_ERR_NULL;
    return launch_status(dsa::launch_quantize_q(q_bf16, n_rows * n_heads, q_code, q_scale, stream));
}

int dsa_index_scores(const uint16_t* q, const float* head_w,
                     const uint8_t* k_code, const float* k_scale, const int32_t* page_table,
                     const int32_t* kv_lens, const int32_t* row_req, const int32_t* row_vis,
                     int32_t n_rows, int32_t batch, int32_t num_pages, int32_t max_pages,
                     int32_t page_size, int32_t n_heads, int32_t head_dim, int32_t group_rows,
                     int32_t flags, float* scores, int32_t score_stride, int32_t* status,
                     hipStream_t stream) {
    dsa::IndexArgs a{};
    const int rc = index_checked(q, head_w, k_code, k_scale, page_table, kv_lens, row_req, row_vis, n_rows, batch,
                                 num_pages, max_pages, page_size, n_heads, head_dim, group_rows, scores,
                                 score_stride, status, a);
    if (rc != DSA_OK) return rc;
    if ((flags & ~DSA_INDEX_WHOLE_ROWS) != 0 || ((flags & DSA_INDEX_WHOLE_ROWS) && group_rows != 1))
        return DSA_ERR_SHAPE;
    if (n_rows == 0) return DSA_OK;
    a.whole_rows = (flags & DSA_INDEX_WHOLE_ROWS) ? 1 : 0;
    return launch_status(dsa::launch_index_scores(a, stream));
}

size_t dsa_index_topk_workspace_size(int32_t n_rows, int32_t score_stride, int32_t top_k) {
    if (n_rows <= 0 || score_stride < 1 || top_k < 1) return 0;
    const IndexTopkGeometry g = index_topk_geometry(n_rows, score_stride, top_k);
    // keys and slots [n_rows, n_chunks, cap]; counts and cuts [n_rows, n_chunks]
    return (size_t)n_rows * g.n_chunks * (2 * (size_t)g.cap + 2) * sizeof(int32_t);
}

int dsa_index_topk(const uint16_t* q, const float* head_w, const uint8_t* k_code, const float* k_scale,
                   const int32_t* page_table, const int32_t* kv_lens, const int32_t* row_req,
                   const int32_t* row_vis, int32_t n_rows, int32_t batch, int32_t num_pages, int32_t max_pages,
                   int32_t page_size, int32_t n_heads, int32_t head_dim, float* scores, int32_t score_stride,
                   int32_t top_k, int32_t phases, void* workspace, size_t workspace_bytes, int32_t* topk_idx,
                   int32_t* topk_count, int32_t* status, hipStream_t stream) {
    if (phases < 1 || phases > (DSA_PHASE_SCORE | DSA_PHASE_SELECT)) return DSA_ERR_SHAPE;
    dsa::IndexArgs a{};
    int rc = index_checked(q, head_w, k_code, k_scale, page_table, kv_lens, row_req, row_vis, n_rows, batch,
                           num_pages, max_pages, page_size, n_heads, head_dim, 1, scores, score_stride, status, a);
    if (rc != DSA_OK) return rc;
    if (top_k < 1 || top_k > dsa::kTopkMaxK) return DSA_ERR_SHAPE;
    const IndexTopkGeometry g = index_topk_geometry(std::max(n_rows, 1), score_stride, top_k);
    if (g.n_chunks > kMaxIndexChunks) return DSA_ERR_SHAPE;
    if (!topk_idx || !topk_count) return DSA_ERR_NULL;
    if (n_rows == 0) return DSA_OK;
    const size_t need = dsa_index_topk_workspace_size(n_rows, score_stride, top_k);
    if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 3) != 0) return DSA_ERR_WORKSPACE;
    const size_t blocks = (size_t)n_rows * g.n_chunks;
    char* ws = static_cast<char*>(workspace);
    a.cand_key = reinterpret_cast<uint32_t*>(ws);
    a.cand_slot = reinterpret_cast<int32_t*>(ws + blocks * g.cap * sizeof(uint32_t));
    a.cand_count = a.cand_slot + blocks * g.cap;
    a.cand_cut = a.cand_count + blocks;
    a.top_k = top_k;
    a.cand_cap = g.cap;
    dsa::TopkArgs t{};
    t.scores = scores; t.score_stride = score_stride; t.row_vis = row_vis;
    t.n_rows = n_rows; t.top_k = top_k; t.n_splits = g.n_chunks;
    t.cand_key = a.cand_key; t.cand_slot = a.cand_slot; t.cand_count = a.cand_count; t.cand_cut = a.cand_cut;
    t.cand_top = nullptr; t.cand_hist = nullptr; t.cand_cap = g.cap;
    t.topk_idx = topk_idx; t.topk_count = topk_count; t.status = status;
    if (phases & DSA_PHASE_SCORE) {
        rc = launch_status(dsa::launch_index_scores(a, stream));
        if (rc != DSA_OK) return rc;
    }
    if (phases & DSA_PHASE_SELECT) rc = launch_status(dsa::launch_topk_merge_cuts(t, stream));
    return rc;
}

int dsa_cache_write(const uint16_t* latent, const uint16_t* rope, const uint16_t* index_k,
                    const float* rope_cos, const float* rope_sin, int32_t max_pos,
                    const int32_t* tok_req, const int32_t* tok_slot, int32_t n_tok,
                    const int32_t* page_table, int32_t batch, int32_t num_pages, int32_t max_pages,
                    int32_t page_size, uint8_t* kv_cache, uint8_t* k_code, float* k_scale,
                    int32_t* status, hipStream_t stream) {
    if (n_tok < 0 || n_tok > kMaxRows) return DSA_ERR_SHAPE;
    int rc = check_page_geometry(batch, num_pages, max_pages, page_size);
    if (rc != DSA_OK) return rc;
    if ((rope_cos == nullptr) != (rope_sin == nullptr)) return DSA_ERR_NULL;
    if (rope_cos != nullptr && max_pos < 1) return DSA_ERR_SHAPE;
    if (n_tok == 0) return DSA_OK;   // nothing to enqueue; no array is read
    if (!latent || !rope || !index_k || !tok_req || !tok_slot || !page_table || !kv_cache || !k_code ||
        !k_scale || !status)
        return DSA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(latent) & 15) != 0 || (reinterpret_cast<uintptr_t>(rope) & 3) != 0 ||
        (reinterpret_cast<uintptr_t>(index_k) & 3) != 0 || (reinterpret_cast<uintptr_t>(kv_cache) & 7) != 0 ||
        (reinterpret_cast<uintptr_t>(k_code) & 1) != 0 || (reinterpret_cast<uintptr_t>(k_scale) & 3) != 0)
        return DSA_ERR_SHAPE;
    dsa::CacheWriteArgs a;
    a.latent = latent; a.rope = rope; a.index_k = index_k;
    a.rope_cos = rope_cos; a.rope_sin = rope_sin; a.max_pos = max_pos;
    a.tok_req = tok_req; a.tok_slot = tok_slot; a.n_tok = n_tok;
    a.batch = batch; a.num_pages = num_pages; a.max_pages = max_pages;
    a.page_size = page_size; a.log2_page = log2i(page_size);
    a.page_table = page_table; a.kv_cache = kv_cache; a.k_code = k_code; a.k_scale = k_scale;
    a.status = status;
    return launch_status(dsa::launch_cache_write(a, stream));
}

int dsa_lse_merge_project(const uint16_t* part_o, const float* part_lse, int32_t n_rows, int32_t n_heads,
                          int32_t n_splits, int32_t d_latent, const uint16_t* w_uv, int32_t d_v,
                          uint16_t* out, float* out_lse, hipStream_t stream) {
    if (n_rows < 0 || n_rows > kMaxRows * 8 || n_heads < 1 || n_heads > 65535) return DSA_ERR_SHAPE;
    if (n_splits < 1 || n_splits > dsa::kMaxSplits) return DSA_ERR_SHAPE;
    if (d_latent != 512 || d_v != 128) return DSA_ERR_UNSUPPORTED;
    if (!part_o || !part_lse || !w_uv || !out) return DSA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(part_o) & 15) != 0 || (reinterpret_cast<uintptr_t>(w_uv) & 15) != 0)
        return DSA_ERR_SHAPE;
    if (n_rows == 0) return DSA_OK;
    dsa::MergeProjectArgs a;
    a.part_o = part_o; a.part_lse = part_lse; a.w_uv = w_uv;
    a.n_rows = n_rows; a.n_heads = n_heads; a.n_splits = n_splits;
    a.out = out; a.out_lse = out_lse;
    return launch_status(dsa::launch_merge_project(a, stream));
}

size_t dsa_topk_workspace_size(int32_t n_rows, int32_t top_k, int32_t n_splits) {
    if (n_rows <= 0 || top_k <= 0 || n_splits <= 1) return 0;
    // keys and slots [n_rows, n_splits, top_k]; counts, cuts and histogram
    // tops [n_rows, n_splits]; kept-key histograms [n_rows, n_splits, 512]
    return 2 * topk_ws_keys(n_rows, top_k, n_splits) + (size_t)n_rows * n_splits * (3 + 512) * sizeof(int32_t);
}

int dsa_topk(const float* scores, int32_t score_stride, const int32_t* row_vis, int32_t n_rows,
             int32_t top_k, int32_t n_splits, void* workspace, size_t workspace_bytes,
             int32_t* topk_idx, int32_t* topk_count, int32_t* status, hipStream_t stream) {
    const int rc = dsa::topk_validate(scores, score_stride, row_vis, n_rows, top_k, n_splits, topk_idx,
                                      topk_count, status);
    if (rc != DSA_OK || n_rows == 0) return rc;
    return dsa::topk_launch(scores, score_stride, row_vis, n_rows, top_k, n_splits, workspace, workspace_bytes,
                            topk_idx, topk_count, status, stream);
}

int dsa_topk_rows(const float* scores, int32_t score_stride, const int32_t* row_vis, const int32_t* row_req,
                  const int32_t* page_table, int32_t batch, int32_t num_pages, int32_t max_pages, int32_t page_size,
                  int32_t n_rows, int32_t top_k, int32_t n_splits, void* workspace, size_t workspace_bytes,
                  int32_t* topk_idx, int32_t* topk_count, int32_t* topk_rows, int32_t* status, hipStream_t stream) {
    int rc = dsa::topk_validate(scores, score_stride, row_vis, n_rows, top_k, n_splits, topk_idx, topk_count,
                                status);
    if (rc != DSA_OK) return rc;
    rc = check_page_geometry(batch, num_pages, max_pages, page_size);
    if (rc != DSA_OK) return rc;
    if (!row_req || !page_table || !topk_rows) return DSA_ERR_NULL;
    if (n_rows == 0) return DSA_OK;
    dsa::TopkArgs r{};
    r.topk_rows = topk_rows; r.row_req = row_req; r.page_table = page_table;
    r.batch = batch; r.num_pages = num_pages; r.max_pages = max_pages;
    r.page_size = page_size; r.log2_page = log2i(page_size);
    return dsa::topk_launch(scores, score_stride, row_vis, n_rows, top_k, n_splits, workspace, workspace_bytes,
                            topk_idx, topk_count, status, stream, &r);
}

int dsa_sparse_mla_decode_rows(const uint16_t* q, const uint8_t* kv_cache, const int32_t* row_vis,
                               const int32_t* topk_rows, const int32_t* topk_count, int32_t n_rows,
                               int32_t num_pages, int32_t page_size, int32_t n_heads, int32_t top_k,
                               int32_t n_splits, float sm_scale, uint16_t* part_o, float* part_lse, uint16_t* out,
                               float* out_lse, int32_t* status, hipStream_t stream) {
    if (!topk_rows) return DSA_ERR_NULL;
    // One request of one page: the geometry a physical-row list needs.
    return mla_checked(q, kv_cache, nullptr, nullptr, row_vis, nullptr, nullptr, topk_count, n_rows, n_rows, 1,
                       num_pages, 1, page_size, n_heads, top_k, n_splits, sm_scale, part_o, part_lse, out, out_lse,
                       status, stream, topk_rows);
}

int dsa_sparse_mla_decode(const uint16_t* q, const uint8_t* kv_cache, const int32_t* page_table,
                          const int32_t* row_req, const int32_t* row_vis, const int32_t* topk_idx,
                          const int32_t* topk_count, int32_t n_rows,
                          int32_t batch, int32_t num_pages, int32_t max_pages, int32_t page_size,
                          int32_t n_heads, int32_t top_k, int32_t n_splits, float sm_scale,
                          uint16_t* part_o, float* part_lse, uint16_t* out, float* out_lse,
                          int32_t* status, hipStream_t stream) {
    return mla_checked(q, kv_cache, page_table, row_req, row_vis, nullptr, topk_idx, topk_count, n_rows, n_rows,
                       batch, num_pages, max_pages, page_size, n_heads, top_k, n_splits, sm_scale, part_o,
                       part_lse, out, out_lse, status, stream);
}

int dsa_sparse_mla_decode_shared(const uint16_t* q, const uint8_t* kv_cache, const int32_t* page_table,
                                 const int32_t* row_req, const int32_t* row_vis, const int32_t* row_list,
                                 const int32_t* topk_idx, const int32_t* topk_count, int32_t n_lists,
                                 int32_t n_rows, int32_t batch, int32_t num_pages, int32_t max_pages,
                                 int32_t page_size, int32_t n_heads, int32_t top_k, int32_t n_splits,
                                 float sm_scale, uint16_t* part_o, float* part_lse, uint16_t* out, float* out_lse,
                                 int32_t* status, hipStream_t stream) {
    if (n_lists < 1 || n_lists > kMaxRows) return DSA_ERR_SHAPE;
    if (!row_list) return DSA_ERR_NULL;
    return mla_checked(q, kv_cache, page_table, row_req, row_vis, row_list, topk_idx, topk_count, n_lists, n_rows,
                       batch, num_pages, max_pages, page_size, n_heads, top_k, n_splits, sm_scale, part_o,
                       part_lse, out, out_lse, status, stream);
}

int dsa_lse_merge(const uint16_t* part_o, const float* part_lse, int32_t n_rows, int32_t n_heads,
                  int32_t n_splits, int32_t d_v, uint16_t* out, float* out_lse, hipStream_t stream) {
    if (n_rows < 0 || n_heads < 1 || d_v < 1) return DSA_ERR_SHAPE;
    if (n_splits < 1 || n_splits > dsa::kMaxSplits) return DSA_ERR_SHAPE;
    if ((int64_t)n_rows * n_heads > INT32_MAX / 256) return DSA_ERR_SHAPE;
    if (d_v != 512) return DSA_ERR_UNSUPPORTED;
    if (!part_o || !part_lse || !out) return DSA_ERR_NULL;
    if (((reinterpret_cast<uintptr_t>(part_o) | reinterpret_cast<uintptr_t>(out)) & 15) != 0) return DSA_ERR_SHAPE;
    if (n_rows == 0) return DSA_OK;
    dsa::MergeArgs a;
    a.part_o = part_o; a.part_lse = part_lse; a.n_rows = n_rows; a.n_heads = n_heads;
    a.n_splits = n_splits; a.out = out; a.out_lse = out_lse;
    return launch_status(dsa::launch_lse_merge(a, stream));
}

}  // extern "C"

namespace dsa {

int topk_validate(const float* scores, int32_t score_stride, const int32_t* row_vis, int32_t n_rows,
                  int32_t top_k, int32_t n_splits, const int32_t* topk_idx, const int32_t* topk_count,
                  const int32_t* status) {
    if (n_rows < 0 || n_rows > kMaxRows || score_stride < 1) return DSA_ERR_SHAPE;
    if (top_k < 1 || top_k > kTopkMaxK) return DSA_ERR_SHAPE;
    if (n_splits < 1 || n_splits > kMaxSplits) return DSA_ERR_SHAPE;
    if (((int64_t)score_stride + n_splits - 1) / n_splits > kTopkMaxList) return DSA_ERR_SHAPE;
    if (n_splits > 1 && (int64_t)n_splits * top_k > kTopkMaxList) return DSA_ERR_SHAPE;
    if (!scores || !row_vis || !topk_idx || !topk_count || !status) return DSA_ERR_NULL;
    return DSA_OK;
}

int topk_launch(const float* scores, int32_t score_stride, const int32_t* row_vis, int32_t n_rows,
                int32_t top_k, int32_t n_splits, void* workspace, size_t workspace_bytes, int32_t* topk_idx,
                int32_t* topk_count, int32_t* status, hipStream_t stream, const TopkArgs* rows) {
    TopkArgs a{};
    if (rows != nullptr) {
        a.topk_rows = rows->topk_rows; a.row_req = rows->row_req; a.page_table = rows->page_table;
        a.batch = rows->batch; a.num_pages = rows->num_pages; a.max_pages = rows->max_pages;
        a.page_size = rows->page_size; a.log2_page = rows->log2_page;
    }
    a.scores = scores; a.score_stride = score_stride; a.row_vis = row_vis;
    a.n_rows = n_rows; a.top_k = top_k; a.n_splits = n_splits;
    a.cand_key = nullptr; a.cand_slot = nullptr; a.cand_count = nullptr; a.cand_cut = nullptr;
    a.cand_top = nullptr; a.cand_hist = nullptr;
    if (n_splits > 1) {
        const size_t need = dsa_topk_workspace_size(n_rows, top_k, n_splits);
        if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 3) != 0) return DSA_ERR_WORKSPACE;
        char* ws = static_cast<char*>(workspace);
        const size_t kb = topk_ws_keys(n_rows, top_k, n_splits);
        a.cand_key = reinterpret_cast<uint32_t*>(ws);
        a.cand_slot = reinterpret_cast<int32_t*>(ws + kb);
        a.cand_count = reinterpret_cast<int32_t*>(ws + 2 * kb);
        a.cand_cut = a.cand_count + (size_t)n_rows * n_splits;
        a.cand_top = a.cand_cut + (size_t)n_rows * n_splits;
        a.cand_hist = a.cand_top + (size_t)n_rows * n_splits;
    }
    a.topk_idx = topk_idx; a.topk_count = topk_count; a.status = status;
    return launch_status(launch_topk(a, stream));
}

}  // namespace dsa
