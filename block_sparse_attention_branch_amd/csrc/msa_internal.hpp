// msa_internal.hpp - host-side launch interface between the C ABI layer
// (msa_api.hip) and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// Largest page-table width (pages per sequence) the decode calls accept.
constexpr int kMaxDecodePages = 16384;
// Pages of one sequence scored by one workgroup of the decode index scan.
constexpr int kKiDecodePagesPerWg = 16;

// ---------------------------------------------------------------- index
// Tiles of 256 (query, group) rows; the block range [0, hi) of a tile is cut
// into chunks of `chunk_blocks` blocks; every (tile, chunk) is one workgroup.
struct KiPrefillArgs {
  const void* q_idx;        // [n_q, h_kv, d_idx]
  const void* k_idx;        // contiguous [n_kv, d_idx] or pages [*, 128, d_idx]
  const uint8_t* k_idx_scale;  // MXFP8 caches: [n_kv or pages * 128, d_idx / 32]
  const int32_t* page_table;  // NULL or [max_pages] of the one sequence
  int32_t n_rows;           // n_q * h_kv
  int32_t h_kv;
  int32_t q_start;
  int32_t n_kv;
  int32_t chunk_blocks;
  int32_t n_chunks;         // chunks of the longest tile
  int32_t grid_chunks;      // chunk slots in the grid (n_chunks rounded up to 8 when xcd_major)
  int32_t xcd_major;        // chunk c runs on XCD c % 8 (all its tiles share that L2)
  int32_t n_tiles;
  float idx_scale;
  int32_t force_local;
  int32_t pool;             // msa_pool: 0 max, 1 mean
  int32_t top_k;
  int32_t need_diag;        // diagonal block must be scored
  int32_t* block_idx;       // [n_rows, top_k]
  float* block_score;       // nullable
  uint64_t* part_keys;      // [n_rows, n_chunks, 16] when n_chunks > 1
  float* part_diag;         // [n_rows]
};

struct KiDecodeArgs {
  const void* q_idx;        // [batch, h_kv, d_idx]
  const void* k_idx;        // pages [*, 128, d_idx]
  const uint8_t* k_idx_scale;  // MXFP8 caches: [pages, 128, d_idx / 32]
  const int32_t* page_table;  // [batch, max_pages]
  const int32_t* seq_lens;  // [batch]
  int32_t batch;
  int32_t h_kv;
  int32_t max_pages;
  int32_t pages_per_wg;
  float idx_scale;
  int32_t force_local;
  int32_t pool;             // msa_pool: 0 max, 1 mean
  int32_t top_k;
  int32_t need_diag;
  float* scores;            // workspace [batch, h_kv, max_pages]
  int32_t* block_idx;       // [batch, h_kv, top_k]
  float* block_score;       // nullable
};

// Host-side tiling rule of the prefill index kernel, shared with the
// workspace-size query so both agree.
struct KiPlan {
  int32_t n_rows, n_tiles, chunk_blocks, n_chunks, grid_chunks, xcd_major;
};
KiPlan ki_prefill_plan(int32_t n_q, int32_t h_kv, int32_t q_start, int32_t need_diag);

// Index projections + RoPE + index-key cache append.
struct KxArgs {
  const void* x;            // [n_tok, d_model]
  const void* w_q;          // [h_kv, d_idx, d_model]
  const void* w_k;          // [d_idx, d_model]
  const int32_t* positions; // [n_tok]
  const int32_t* seq;       // [n_tok] nullable (paged: page_table row of each token)
  const int32_t* page_table;
  void* k_cache;            // contiguous [n_kv, d_idx] or pages [*, 128, d_idx]
  void* q_out;              // [n_tok, h_kv, d_idx]
  int32_t n_tok, d_model, h_kv, rope_dim, n_kv, max_pages;
  float rope_base;
  float* part;              // split > 1: fp32 partial sums [split, n_tok, h_kv + 1, d_idx]
  int32_t split, k_per_split;
};
// Short calls split d_model over `split` slices of k_per_split (a multiple of
// 16) so that enough workgroups stream the weights; total = workspace bytes.
struct KxPlan {
  int32_t split, k_per_split;
  size_t total;
};
KxPlan kx_plan(int32_t n_tok, int32_t d_model, int32_t h_kv, int32_t d_idx);
hipError_t launch_index_project(int d_idx, const KxArgs& a, hipStream_t st);

hipError_t launch_ki_prefill(int dtype, int d_idx, const KiPrefillArgs& a, hipStream_t st);
hipError_t launch_ki_decode(int dtype, int d_idx, const KiDecodeArgs& a, hipStream_t st);
bool ki_supported(int dtype, int d_idx);

// ------------------------------------------------------- main branch
struct AttnArgs {
  const void* q;             // prefill [n_q, h_q, d] / decode [batch, h_q, d]
  const void* k;             // contiguous [n_kv, h_kv, d] or pages [*, h_kv, 128, d]
  const void* v;
  const uint8_t* k_scale;    // MXFP8 caches: E8M0 scales, the cache layout with d / 32 columns
  const uint8_t* v_scale;
  const int32_t* page_table; // NULL = contiguous
  const int32_t* seq_lens;   // decode only
  const int32_t* block_idx;  // [rows, h_kv, top_k]
  void* o;
  float* lse;                // nullable
  int32_t n_q, q_start, n_kv, batch, max_pages;
  int32_t h_q, h_kv, group, top_k;
  float sm_scale;
  // prefill schedule / decode split workspace
  void* ws;
  size_t ws_bytes;
};

// Prefill schedule geometry (windows of query tokens, KV-outer items).
struct PrefillPlan {
  int32_t window;           // query tokens per window
  int32_t n_windows;
  int32_t merge_windows;    // consecutive windows whose partials one merge launch combines
  int32_t stream_partials;  // partials are written with streaming stores (they outgrow the caches)
  int32_t n_blocks;         // KV blocks addressable by the call
  int32_t chunk;            // max tokens per KV-outer work item
  int64_t n_cells;          // n_windows * h_kv * n_blocks
  size_t off_count, off_fill, off_cell_off, off_item_off, off_entries, off_items,
      off_part_o, off_part_lse, off_scan, total;
  int64_t max_items;
  size_t off_bitmap;        // ordered schedules only
  int32_t bitmap_words;     // 0: entries are scattered in arrival order
};
PrefillPlan prefill_plan(int dtype, int32_t n_q, int32_t q_start, int32_t n_kv, int32_t h_q,
                         int32_t h_kv, int32_t d_h, int32_t top_k);
// Schedule arrays only (windows of `window` tokens, items of at most `chunk`
// tokens); `total` ends after them.  `ordered`: each cell lists its tokens in
// increasing order (built through a per-cell token bitmap), so that sums over
// a cell's rows do not depend on thread timing; the slot field of such
// entries is 0.
void schedule_layout(PrefillPlan& p, int32_t n_q, int32_t q_start, int32_t h_kv, int32_t top_k, int32_t window,
                     int32_t chunk, bool ordered = false);
hipError_t launch_sparse_prefill(int dtype, int d_h, const AttnArgs& a, const PrefillPlan& pl,
                                 hipStream_t st);
// Test hook: largest block count whose schedule counters are kept in LDS
// (< 0 restores the built-in limits; 0 forces the global-atomic path).
void set_schedule_lds_limit(int max_blocks);
bool attn_supported(int dtype, int d_h);

struct DecodePlan {
  int32_t split;            // workgroups per (sequence, group)
  int32_t waves;            // waves per workgroup (8, or 4 when the keys are split)
  size_t off_part_o, off_part_lse, total;
};
DecodePlan decode_plan(int32_t batch, int32_t h_q, int32_t h_kv, int32_t d_h, int32_t top_k);
hipError_t launch_sparse_decode(int dtype, int d_h, const AttnArgs& a, const DecodePlan& pl,
                                hipStream_t st);
bool decode_supported(int dtype, int d_h);

hipError_t launch_dense_prefill(int dtype, int d_h, const AttnArgs& a, hipStream_t st);

// ------------------------------------------------------- training path
struct BackwardArgs {
  AttnArgs attn;            // q, k, v, block_idx, o (the forward's output), lse, workspace
  const void* d_o;          // [n_q, h_q, d]
  void* dq;                 // [n_q, h_q, d]
  void* dk;                 // [n_kv, h_kv, d]
  void* dv;
  // KL-alignment term: kl != 0 asks for it
  int32_t kl, d_idx;
  const void* q_idx;        // [n_q, h_kv, d_idx]
  const void* k_idx;        // [n_kv, d_idx]
  float idx_scale, kl_scale;
  float* kl_out;            // [n_q, h_kv], nullable
  void* dq_idx;             // [n_q, h_kv, d_idx]
  void* dk_idx;             // [n_kv, d_idx]
};
struct BackwardPlan {
  PrefillPlan q;            // dQ pass schedule (windows), at off_q
  PrefillPlan kv;           // dK/dV pass schedule (one window), at off_kv
  size_t off_q, off_kv, off_dsum, off_part_dq, off_part_dkv;
  size_t off_pmain, off_part_kl, off_lse_idx, off_part_dki;  // with the KL term only
  size_t total;
};
BackwardPlan backward_plan(int32_t n_q, int32_t q_start, int32_t n_kv, int32_t h_q, int32_t h_kv, int32_t d_h,
                           int32_t top_k, int32_t d_idx, bool with_kl);
hipError_t launch_sparse_prefill_backward(int d_h, const BackwardArgs& a, const BackwardPlan& pl, hipStream_t st);
bool backward_supported(int dtype, int d_h);
bool dense_supported(int dtype, int d_h);

}  // namespace msa
