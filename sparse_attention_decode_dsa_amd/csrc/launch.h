// Internal launchers: the C ABI in dsa_api.cpp validates its arguments and
// then calls these, which only compute grid shapes and enqueue kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct IndexArgs {
    const uint16_t* q;        // [n_rows, 64, 128] bf16
    const float* head_w;
    const uint8_t* k_code;
    const float* k_scale;
    const int32_t* page_table;
    const int32_t* kv_lens;
    const int32_t* row_req;
    const int32_t* row_vis;
    int32_t n_rows, batch, num_pages, max_pages, page_size, log2_page, group_rows;
    float* scores;
    int32_t score_stride;
    int32_t* status;
    int32_t chunk;     // chunked launch: tokens per workgroup (set by the launcher)
    int32_t whole_rows;   // decode launch: whole-row key loads with the non-temporal hint
    // Top-k candidates kept by the decode launch (one row a group), or
    // cand_key == nullptr for scores only.  Chunk j of row r writes to block
    // r * n_chunks + j: up to cand_cap keys and slots, their count (-1: more
    // than cand_cap) and its cut.
    uint32_t* cand_key;
    int32_t* cand_slot;
    int32_t* cand_count;
    int32_t* cand_cut;
    int32_t top_k, cand_cap;
};

struct TopkArgs {
    const float* scores;
    int32_t score_stride;
    const int32_t* row_vis;
    int32_t n_rows, top_k, n_splits;
    uint32_t* cand_key;   // [n_rows, n_splits, top_k]: each split's kept keys, at the front of its block
    int32_t* cand_slot;   // [n_rows, n_splits, top_k]: their slots
    int32_t* cand_count;  // [n_rows, n_splits]: how many each split kept
    int32_t* cand_cut;    // [n_rows, n_splits]: the row's cut key, as each split used it
    int32_t* cand_top;    // [n_rows, n_splits]: the key from which the kept-key histogram's last bin starts
    int32_t* cand_hist;   // [n_rows, n_splits, 512]: histogram of each split's kept keys
    int32_t cand_cap;     // candidates' block length per split (the merge of the indexer's candidates)
    int32_t* topk_idx;
    int32_t* topk_count;
    int32_t* status;
    // Physical rows of the selected slots (nullptr: not asked for), through
    // row r's request row_req[r] and the block table.
    int32_t* topk_rows;
    const int32_t* row_req;
    const int32_t* page_table;
    int32_t batch, num_pages, max_pages, page_size, log2_page;
};

struct MlaArgs {
    const uint16_t* q;         // [n_rows, n_heads, 576] bf16
    const uint8_t* kv_cache;   // [num_pages, page_size, 640]: codes, fp32 scale, pad
    const int32_t* page_table;
    const int32_t* row_req;
    const int32_t* row_vis;
    const int32_t* topk_idx;
    const int32_t* topk_count;
    // Physical rows of the list entries instead of slots (nullptr: topk_idx
    // holds slots, resolved through the block table).
    const int32_t* topk_rows;
    int32_t n_rows, batch, num_pages, max_pages, page_size, log2_page, n_heads, top_k, n_splits;
    float sm_scale;
    uint16_t* part_o;          // bf16 bit patterns
    float* part_lse;
    uint16_t* out;
    float* out_lse;
    int32_t* status;
    // Shared lists (MTP IndexShare): row r attends list row_list[r] of
    // [n_lists, top_k]; nullptr: row r attends list r.  chain: the rows come
    // in chains of that many consecutive rows sharing one list (1: none
    // shared), and the launch places each chain's work units on one XCD (set
    // by the launcher).
    const int32_t* row_list;
    int32_t n_lists;
    int32_t chain;
};

struct CacheWriteArgs {
    const uint16_t* latent;    // [n_tok, 512] bf16
    const uint16_t* rope;      // [n_tok, 64] bf16, before rotation
    const uint16_t* index_k;   // [n_tok, 128] bf16
    const float* rope_cos;     // [max_pos, 32] or null (no rotation)
    const float* rope_sin;
    int32_t max_pos;
    const int32_t* tok_req;
    const int32_t* tok_slot;
    int32_t n_tok, batch, num_pages, max_pages, page_size, log2_page;
    const int32_t* page_table;
    uint8_t* kv_cache;         // [num_pages, page_size, 640]
    uint8_t* k_code;           // [num_pages, page_size, 128]
    float* k_scale;            // [num_pages, page_size]
    int32_t* status;
};

struct MergeProjectArgs {
    const uint16_t* part_o;    // [n_rows, n_heads, n_splits, 512] bf16
    const float* part_lse;     // [n_rows, n_heads, n_splits]
    const uint16_t* w_uv;      // [n_heads, 128, 512] bf16
    int32_t n_rows, n_heads, n_splits;
    uint16_t* out;             // [n_rows, n_heads, 128] bf16
    float* out_lse;            // [n_rows, n_heads] or null
};

struct MergeArgs {
    const uint16_t* part_o;    // bf16
    const float* part_lse;
    int32_t n_rows, n_heads, n_splits;
    uint16_t* out;
    float* out_lse;
};

// Largest list one top-k workgroup selects from (its keys live in LDS).
constexpr int kTopkMaxList = 32768;
constexpr int kTopkMaxK = 8192;
constexpr int kMaxSplits = 64;

// Host validation of a top-k call (the rules of dsa_topk, without the
// workspace), and its launch with a given workspace (checked against the
// size dsa_topk_workspace_size gives).  Both return DSA_OK or a DSA_ERR_*.
int topk_validate(const float* scores, int32_t score_stride, const int32_t* row_vis, int32_t n_rows,
                  int32_t top_k, int32_t n_splits, const int32_t* topk_idx, const int32_t* topk_count,
                  const int32_t* status);
int topk_launch(const float* scores, int32_t score_stride, const int32_t* row_vis, int32_t n_rows,
                int32_t top_k, int32_t n_splits, void* workspace, size_t workspace_bytes, int32_t* topk_idx,
                int32_t* topk_count, int32_t* status, hipStream_t stream, const TopkArgs* rows = nullptr);

hipError_t launch_quantize_q(const uint16_t* q, int32_t n_pairs, uint8_t* code, float* scale,
                             hipStream_t stream);
hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream);
// Tokens per workgroup of the chunked indexer launch for `groups` row groups.
int index_chunk(int groups, int score_stride);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
// Merge of the candidates the decode indexer kept (a.n_splits = its chunks
// per row, a.cand_cap their block length; no histograms).
hipError_t launch_topk_merge_cuts(const TopkArgs& a, hipStream_t stream);
hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream);
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);
hipError_t launch_merge_project(const MergeProjectArgs& a, hipStream_t stream);

}  // namespace dsa
