// msa_attn.hip - main branch of MiniMax Sparse Attention on gfx950.
//
// Eq. (8) of the "MiniMax Sparse Attention" digest (titansim.online, §4.3):
// every query head of KV group r attends, with exact softmax, to the causally
// visible keys of the blocks its group selected.
//
// Prefill is KV-outer (digest §4.4.2): the selected (group, block) pairs are
// the outer loop and the queries that picked a block are gathered into the
// MFMA's N dimension, so one 128-token K/V block staged in LDS serves every
// (token, head) row that selected it.  The schedule inverts the index lists
// into per-(window, group, block) token lists and cuts each list into work
// items of at most `chunk` tokens (the pages' pre-scheduled tile chunking).
// Each item writes, per (token, head), the un-normalised partial output of
// that block, sum_j exp(s_j - m_b) v_j in bf16, with its max m_b and sum l_b;
// a merge kernel then combines a token's partials with log-sum-exp weights
// (the second stage).  Query tokens are processed in windows so that the partial
// buffer of one window stays small enough to live in the last-level cache
// between the two stages.  No atomics touch floating-point data, so results
// are bitwise reproducible.
//
// Decode gathers, for each (sequence, group), the 16 selected pages of the
// paged cache with 16x16x32 MFMA (the 16 heads of the group on one side),
// splitting the selected keys over workgroups when the batch is small.
//
// The dense kernel (Eq. (1), §2.2) is the Q-outer comparison path.
#include "msa_common.hpp"
#include "msa_internal.hpp"
#include "msa_kvouter.hpp"
#include "msa_profile.hpp"

#include <atomic>
#include <type_traits>

namespace msa {

__global__ void ks_zero_kernel(SchedArgs a) {
  for (int64_t c = blockIdx.x * 256ll + threadIdx.x; c < a.n_cells; c += (int64_t)gridDim.x * 256) {
    a.count[c] = 0;
    a.fill[c] = 0;
  }
}

__global__ void ks_count_kernel(SchedArgs a) {
  const int64_t row = blockIdx.x * 256ll + threadIdx.x;  // (i, r)
  if (row >= (int64_t)a.n_q * a.h_kv) return;
  const int i = (int)(row / a.h_kv), r = (int)(row % a.h_kv);
  const int diag = (a.q_start + i) >> 7;
  int b[kMaxTopK];
  const uint32_t m = sched_used(a.block_idx + row * a.top_k, a.top_k, diag, a.skip_diag, b);
  const int w = i / a.window;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (m & (1u << j)) atomicAdd(&a.count[cell_key(w, r, b[j], a.n_blocks, a.h_kv)], 1);
}

__device__ __forceinline__ void block_excl_scan2(int& x, int& y, int* sh) {
  // sh: 512 ints
  const int t = threadIdx.x;
  sh[t] = x;
  sh[256 + t] = y;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int ax = t >= off ? sh[t - off] : 0;
    const int ay = t >= off ? sh[256 + t - off] : 0;
    __syncthreads();
    sh[t] += ax;
    sh[256 + t] += ay;
    __syncthreads();
  }
  const int ix = sh[t], iy = sh[256 + t];
  __syncthreads();
  x = ix - x;
  y = iy - y;
}

__global__ __launch_bounds__(256) void ks_scan_a_kernel(SchedArgs a) {
  __shared__ int sh[512];
  const int64_t c0 = (int64_t)blockIdx.x * kScanTile + threadIdx.x * kScanPerThread;
  int se = 0, si = 0;
  for (int k = 0; k < kScanPerThread; ++k) {
    const int64_t c = c0 + k;
    if (c < a.n_cells) {
      const int n = a.count[c];
      se += n;
      si += (n + a.chunk - 1) / a.chunk;
    }
  }
  int xe = se, xi = si;
  block_excl_scan2(xe, xi, sh);
  if (threadIdx.x == 255) {
    a.scan[blockIdx.x] = xe + se;
    a.scan[a.n_scan_tiles + blockIdx.x] = xi + si;
  }
}

__global__ __launch_bounds__(256) void ks_scan_b_kernel(SchedArgs a) {
  __shared__ int sh[512];
  const int per = (a.n_scan_tiles + 255) / 256;
  const int t0 = threadIdx.x * per;
  int se = 0, si = 0;
  for (int k = 0; k < per; ++k)
    if (t0 + k < a.n_scan_tiles) {
      se += a.scan[t0 + k];
      si += a.scan[a.n_scan_tiles + t0 + k];
    }
  int xe = se, xi = si;
  block_excl_scan2(xe, xi, sh);
  for (int k = 0; k < per; ++k)
    if (t0 + k < a.n_scan_tiles) {
      const int ve = a.scan[t0 + k], vi = a.scan[a.n_scan_tiles + t0 + k];
      a.scan[2 * a.n_scan_tiles + t0 + k] = xe;
      a.scan[3 * a.n_scan_tiles + t0 + k] = xi;
      xe += ve;
      xi += vi;
    }
  if (threadIdx.x == 255) {
    a.cell_off[a.n_cells] = xe;
    a.item_off[a.n_cells] = xi;
  }
}

__global__ __launch_bounds__(256) void ks_scan_c_kernel(SchedArgs a) {
  __shared__ int sh[512];
  const int64_t c0 = (int64_t)blockIdx.x * kScanTile + threadIdx.x * kScanPerThread;
  int se = 0, si = 0;
  for (int k = 0; k < kScanPerThread; ++k) {
    const int64_t c = c0 + k;
    if (c < a.n_cells) {
      const int n = a.count[c];
      se += n;
      si += (n + a.chunk - 1) / a.chunk;
    }
  }
  int xe = se, xi = si;
  block_excl_scan2(xe, xi, sh);
  xe += a.scan[2 * a.n_scan_tiles + blockIdx.x];
  xi += a.scan[3 * a.n_scan_tiles + blockIdx.x];
  for (int k = 0; k < kScanPerThread; ++k) {
    const int64_t c = c0 + k;
    if (c < a.n_cells) {
      const int n = a.count[c];
      a.cell_off[c] = xe;
      a.item_off[c] = xi;
      xe += n;
      xi += (n + a.chunk - 1) / a.chunk;
    }
  }
}

__global__ void ks_scatter_kernel(SchedArgs a) {
  const int64_t row = blockIdx.x * 256ll + threadIdx.x;
  if (row >= (int64_t)a.n_q * a.h_kv) return;
  const int i = (int)(row / a.h_kv), r = (int)(row % a.h_kv);
  const int diag = (a.q_start + i) >> 7;
  int b[kMaxTopK];
  const uint32_t m = sched_used(a.block_idx + row * a.top_k, a.top_k, diag, a.skip_diag, b);
  const int w = i / a.window;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (m & (1u << j)) {
      const int64_t cell = cell_key(w, r, b[j], a.n_blocks, a.h_kv);
      const int pos = a.cell_off[cell] + atomicAdd(&a.fill[cell], 1);
      a.entries[pos] = (i << 4) | j;
    }
}

// The same two steps with the counters in LDS: one workgroup per (window,
// group), whose rows only ever touch that (window, group)'s cells.  Global
// atomics on hot cells (every token of a query block lists its own block)
// serialise; LDS atomics do not leave the CU.  Used while a window's blocks
// fit in LDS.
constexpr int kSchedLdsBlocks = 16384;

// Workgroup (window w, slice s, group r) takes tokens [t0, t1) of window w.
__device__ __forceinline__ void ks_slice(const SchedArgs& a, int& w, int& t0, int& t1) {
  w = blockIdx.x / a.split;
  const int s = blockIdx.x % a.split, per = (a.window + a.split - 1) / a.split;
  t0 = w * a.window + s * per;
  t1 = min(min(t0 + per, (w + 1) * a.window), a.n_q);
}

// Counts a slice's entries per block of group r into cnt (LDS, zeroed here).
__device__ __forceinline__ void ks_slice_counts(const SchedArgs& a, int r, int t0, int t1, int* cnt) {
  for (int b = threadIdx.x; b < a.n_blocks; b += 256) cnt[b] = 0;
  __syncthreads();
  for (int i = t0 + threadIdx.x; i < t1; i += 256) {
    int b[kMaxTopK];
    const uint32_t m =
        sched_used(a.block_idx + ((size_t)i * a.h_kv + r) * a.top_k, a.top_k, (a.q_start + i) >> 7, a.skip_diag, b);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (m & (1u << j)) atomicAdd(&cnt[b[j]], 1);
  }
  __syncthreads();
}

// With one slice per (window, group) the counts are stored whole; with more,
// each slice adds its nonzero counts (count zeroed beforehand): one global
// atomic per (slice, cell) instead of one per entry.
__global__ __launch_bounds__(256) void ks_count_lds_kernel(SchedArgs a) {
  extern __shared__ int cnt[];  // [n_blocks]
  const int r = blockIdx.y;
  int w, t0, t1;
  ks_slice(a, w, t0, t1);
  ks_slice_counts(a, r, t0, t1, cnt);
  for (int b = threadIdx.x; b < a.n_blocks; b += 256) {
    const int64_t cell = cell_key(w, r, b, a.n_blocks, a.h_kv);
    if (a.split == 1)
      a.count[cell] = cnt[b];
    else if (cnt[b] > 0)
      atomicAdd(&a.count[cell], cnt[b]);
  }
}

// Scatter: a slice reserves a contiguous run of each cell's entries (one
// global atomic on fill per nonzero cell; fill zeroed beforehand when split),
// then places its entries with LDS atomics.  The order of the slices' runs
// within a cell depends on timing; no result depends on that order.
__global__ __launch_bounds__(256) void ks_scatter_lds_kernel(SchedArgs a) {
  extern __shared__ int pos[];  // [n_blocks] next free entry of each cell
  const int r = blockIdx.y;
  int w, t0, t1;
  ks_slice(a, w, t0, t1);
  if (a.split == 1) {
    for (int b = threadIdx.x; b < a.n_blocks; b += 256) pos[b] = a.cell_off[cell_key(w, r, b, a.n_blocks, a.h_kv)];
    __syncthreads();
  } else {
    ks_slice_counts(a, r, t0, t1, pos);
    for (int b = threadIdx.x; b < a.n_blocks; b += 256) {
      const int n = pos[b];
      if (n > 0) {
        const int64_t cell = cell_key(w, r, b, a.n_blocks, a.h_kv);
        pos[b] = a.cell_off[cell] + atomicAdd(&a.fill[cell], n);
      }
    }
    __syncthreads();
  }
  for (int i = t0 + threadIdx.x; i < t1; i += 256) {
    int b[kMaxTopK];
    const uint32_t m =
        sched_used(a.block_idx + ((size_t)i * a.h_kv + r) * a.top_k, a.top_k, (a.q_start + i) >> 7, a.skip_diag, b);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (m & (1u << j)) a.entries[atomicAdd(&pos[b[j]], 1)] = (i << 4) | j;
  }
}

__global__ void ks_items_kernel(SchedArgs a) {
  const int64_t cell = blockIdx.x * 256ll + threadIdx.x;
  if (cell >= a.n_cells) return;
  const int ib = a.item_off[cell], ie = a.item_off[cell + 1];
  const int eb = a.cell_off[cell], ee = a.cell_off[cell + 1];
  int r, b;
  cell_rb(cell, a.n_blocks, a.h_kv, r, b);
  for (int it = ib; it < ie; ++it) {
    const int e0 = eb + (it - ib) * a.chunk;
    a.items[it] = i32x4{b, r, e0, min(e0 + a.chunk, ee)};
  }
}

// Ordered mode: a cell's token list in increasing token order whatever the
// order the threads run in.  Each used (row, slot) sets its token's bit in
// the cell's bitmap; one workgroup per cell then writes the set bits out in
// order at the cell's offset.
__global__ void ks_bits_zero_kernel(SchedArgs a) {
  if (blockIdx.x == 0 && threadIdx.x < 2) a.fill[threadIdx.x] = 0;  // work-queue heads of the consumers
  const int64_t n = a.n_cells * a.words;
  for (int64_t x = blockIdx.x * 256ll + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) a.bitmap[x] = 0u;
}

__global__ void ks_bits_set_kernel(SchedArgs a) {
  const int64_t row = blockIdx.x * 256ll + threadIdx.x;  // (i, r)
  if (row >= (int64_t)a.n_q * a.h_kv) return;
  const int i = (int)(row / a.h_kv), r = (int)(row % a.h_kv);
  const int diag = (a.q_start + i) >> 7;
  int b[kMaxTopK];
  const uint32_t m = row_used(a.block_idx + row * a.top_k, a.top_k, diag, b);
  const int w = i / a.window, il = i - w * a.window;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (m & (1u << j)) {
      const int64_t cell = cell_key(w, r, b[j], a.n_blocks, a.h_kv);
      atomicOr(&a.bitmap[cell * a.words + (il >> 5)], 1u << (il & 31));
    }
}

// The same with the bits of 256 consecutive tokens (8 words per cell) built in
// LDS: workgroup (window, token tile, group) owns those words of every cell
// of its group, so it writes them out whole, without atomics (the tokens of a
// query block all set bits in the same word of their own block's cell).
constexpr int kBitsLdsBlocks = 2048;

__global__ __launch_bounds__(256) void ks_bits_set_lds_kernel(SchedArgs a) {
  extern __shared__ uint32_t lb[];  // [n_blocks][8]
  const int tiles = (a.window + 255) / 256;
  const int w = blockIdx.x / tiles, t = blockIdx.x % tiles, r = blockIdx.y;
  if (blockIdx.x == 0 && r == 0 && threadIdx.x < 2) a.fill[threadIdx.x] = 0;  // work-queue heads of the consumers
  for (int x = threadIdx.x; x < a.n_blocks * 8; x += 256) lb[x] = 0u;
  __syncthreads();
  const int il = t * 256 + threadIdx.x, i = w * a.window + il;
  if (il < a.window && i < a.n_q) {
    int b[kMaxTopK];
    const uint32_t m = row_used(a.block_idx + ((size_t)i * a.h_kv + r) * a.top_k, a.top_k, (a.q_start + i) >> 7, b);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (m & (1u << j)) atomicOr(&lb[b[j] * 8 + (threadIdx.x >> 5)], 1u << (threadIdx.x & 31));
  }
  __syncthreads();
  const int nw = min(8, a.words - 8 * t);
  for (int x = threadIdx.x; x < a.n_blocks * 8; x += 256) {
    const int bb = x >> 3, k = x & 7;
    if (k < nw) a.bitmap[cell_key(w, r, bb, a.n_blocks, a.h_kv) * a.words + 8 * t + k] = lb[x];
  }
}

// Ordered mode's cell sizes: the popcount of each cell's bitmap (no atomics
// on a few hot counters).
__global__ __launch_bounds__(256) void ks_bits_count_kernel(SchedArgs a) {
  __shared__ int red[4];
  const int64_t cell = blockIdx.x;
  const uint32_t* bits = a.bitmap + cell * a.words;
  int n = 0;
  for (int x = threadIdx.x; x < a.words; x += 256) n += __builtin_popcount(bits[x]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) a.count[cell] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void ks_bits_extract_kernel(SchedArgs a) {
  __shared__ int sh[512];
  const int64_t cell = blockIdx.x;
  const int per = (a.words + 255) / 256;
  const int w0 = threadIdx.x * per, w1 = min(w0 + per, a.words);
  const uint32_t* bits = a.bitmap + cell * a.words;
  int n = 0;
  for (int x = w0; x < w1; ++x) n += __builtin_popcount(bits[x]);
  int pos = n, dummy = 0;
  block_excl_scan2(pos, dummy, sh);
  pos += a.cell_off[cell];
  const int w = (int)(cell / ((int64_t)a.h_kv * a.n_blocks));
  for (int x = w0; x < w1; ++x) {
    uint32_t b = bits[x];
    while (b) {
      const int bit = __builtin_ctz(b);
      b &= b - 1u;
      a.entries[pos++] = (w * a.window + x * 32 + bit) << 4;
    }
  }
}

// ====================================================================
// KV-outer sparse attention (one window of query tokens)
// ====================================================================
struct KpArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* k_scale;  // MXFP8 caches only
  const uint8_t* v_scale;
  const int32_t* page_table;
  const int32_t* cell_off;
  const int32_t* item_off;
  const int32_t* entries;
  const i32x4* items;
  void* part_o;       // [span, h_kv, top_k, G, D]  un-normalised sum_j p_j v_j
  float2* part_ml;    // [span, h_kv, top_k, G]     (row max * sm_scale, sum_j p_j)
  int32_t n_kv, q_start, h_q, h_kv, group, g_shift, top_k, n_blocks, window, chunk, w;
  int32_t slot_tok0;  // first token of the span of windows the partial buffer holds
  size_t trash_slot;  // first of two spare slot regions at the end of part_o / part_ml
  float sm_scale;
};




// Query rows of one pass (one 32-row tile per wave) of one item.
template <typename T, int D>
struct KpPass {
  Frag<T> qf[D / 16];
  int pos, slot, head;
  bool ok;
};

// Gathers the query fragments of this lane's row `rho` of item m.  `ent` is
// the (token << 4 | slot) entry of that row.  Rows past the item's end load a
// valid row (the caller clamps `ent`) and are flagged !ok; no branches, so
// the number of outstanding loads is always known at compile time.
template <typename T, int D>
__device__ __forceinline__ void kp_load_pass(KpPass<T, D>& ps, const KpArgs& a, const KpItem& m, int rho, int ent) {
  const T* __restrict__ q = static_cast<const T*>(a.q);
  const int half = (threadIdx.x & 63) >> 5;
  const int G = a.group;
  ps.ok = rho < (m.e_end - m.e_begin) * G;
  const int i = ent >> 4, j = ent & 15;
  ps.head = rho & (G - 1);
  ps.slot = ((i - a.slot_tok0) * a.h_kv + m.r) * a.top_k + j;
  ps.pos = ps.ok ? a.q_start + i : -1;
  const T* qrow = q + ((size_t)i * a.h_q + m.r * G + ps.head) * D + half * 8;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) ps.qf[ks] = load_frag<T>(qrow + ks * 16);
}

template <typename T, int D>
__device__ __forceinline__ int kp_entry(const KpItem& m, int rho, int g_shift, const int* ent_lds) {
  return ent_lds[min(rho >> g_shift, m.e_end - m.e_begin - 1)];
}

// Scores, softmax and P.V for the rows in `ps`, then the partial stores.  The
// math is skipped when no row of the wave is valid; the stores are not (rows
// past the end write a trash row), keeping the memory-op count fixed.
// One 32-row tile of a wave against the block b staged in `lds`: scores
// (keys after the row's position masked), the block-local softmax with max
// `mx` (raw score) and sum `l`, and the un-normalised P.V in t.o.  The query
// fragments and the position are already in t.qf[0] / t.pos[0].
template <typename T, int D>
__device__ __forceinline__ void block_tile_math(float sm_scale, int b, bool ok, const char* lds,
                                                TileRegs<T, D, 1>& t, float& mx, float& l) {
  const float c2 = sm_scale * kLog2e;
  const bool need_mask = ok && (b * kBlock + kBlock - 1 > t.pos[0]);
  tile_scores<T, D, 1>(t, lds, b, __any(need_mask));
  float mm = -__builtin_inff();
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v) mm = fmaxf(mm, t.s[0][kt][v]);
  mm = fmaxf(mm, __shfl_xor(mm, 32, 64));
  mx = mm;
  const float mc = (mm == -__builtin_inff()) ? 0.0f : mm * c2;
  float sum = 0.0f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float pr = fast_exp2(fmaf(t.s[0][kt][v], c2, -mc));
      t.s[0][kt][v] = pr;
      sum += pr;
    }
  l = sum + __shfl_xor(sum, 32, 64);
  tile_pack_p<T, D, 1>(t, 0);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) t.o[0][dt] = f32x16{};
  tile_pv<T, D, 1>(t, lds);
}

template <typename T, int D>
__device__ __forceinline__ void kp_math(const KpArgs& a, int b, const KpPass<T, D>& ps, const char* lds,
                                        TileRegs<T, D, 1>& t, float& mx, float& l) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) t.qf[0][ks] = ps.qf[ks];
  t.pos[0] = ps.pos;
  block_tile_math<T, D>(a.sm_scale, b, ps.ok, lds, t, mx, l);
}

// NT: the partial outputs are stored non-temporally (a template parameter, as
// the compiler merges the two kinds of store when both sit under one branch).
template <typename T, int D, bool NT>
__device__ __forceinline__ void kp_store(const KpArgs& a, const KpPass<T, D>& ps, const TileRegs<T, D, 1>& t,
                                         float mx, float l) {
  const int half = (threadIdx.x & 63) >> 5;
  const int G = a.group;
  const size_t slot = ps.ok ? (size_t)ps.slot : a.trash_slot;
  T* region = static_cast<T*>(a.part_o) + slot * G * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int p = 0; p < 2; ++p)
      store8<T, NT>(region + (size_t)part_chunk(dt, p, half, ps.head, G) * 8, t.o[0][dt], 8 * p);
  const size_t mrow = (half == 0 ? slot : a.trash_slot + 1) * G + ps.head;
  a.part_ml[mrow] = float2{mx * a.sm_scale, l};
}

constexpr int kKpThreads = 512;                    // 8 waves, 32 rows each per pass
constexpr int kKpRowsPerPass = kKpThreads / 2;     // 256
constexpr int kKpItemRows = 2 * kKpRowsPerPass;    // an item holds at most 512 (token, head) rows
constexpr int kKpMaxChunk = kKpItemRows;           // tokens per item when G == 1

template <typename T, int D>
__device__ __forceinline__ KpItem kp_item_s(const KpArgs& a, int it) {
  const i32x4 d = scalar_load(a.items, __builtin_amdgcn_readfirstlane(it));
  return KpItem{d[0], d[1], d[2], d[3]};
}

// Persistent over this XCD's items of the window: the grid is a multiple of 8
// and workgroup g (dispatched to XCD g % 8) takes the XCD's items sub, sub +
// nsub, ...  Each item is two passes of 256 rows.  The next item's K/V and
// token entries are prefetched into registers at the start of an item, the
// next pass's queries while the current pass runs P.V.
template <typename T, int D, typename TC = T, bool STREAM = false>
__global__ __launch_bounds__(kKpThreads) void kp_kernel(KpArgs a) {
  using L = KvLds<T, D>;
  constexpr int NT = kKpThreads;
  constexpr int BUF = L::BYTES + kKpMaxChunk * 4;   // K, V^T, token entries
  constexpr int NB = (2 * BUF <= 160 * 1024) ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char lds[NB][BUF];
  const int x = blockIdx.x & 7, sub = blockIdx.x >> 3, nsub = gridDim.x >> 3;
  const int64_t n_l = (int64_t)a.h_kv * a.n_blocks, per = n_l >> 3;
  const int64_t k0 = (int64_t)a.w * n_l + x * per;
  const int item_begin = scalar_load(a.item_off, k0);
  const int item_end = scalar_load(a.item_off, k0 + per);
  int it = item_begin + sub;
  if (it >= item_end) return;
  const int wave = threadIdx.x >> 6, l32 = threadIdx.x & 31;
  const int rho0 = wave * 32 + l32;                 // this lane's row in pass 0; pass 1 is + 256
  const int tid = threadIdx.x;

  StageRegs<T, D, NT, TC> pre;
  KpItem cur = kp_item_s<T, D>(a, it);
  stage_load<T, D, NT, TC>(pre, block_ptr<TC, D>(a.k, a.v, a.page_table, cur.b, cur.r, a.h_kv, a.n_kv, a.k_scale,
                                                 a.v_scale));
  int pre_ent = a.entries[cur.e_begin + min(tid, cur.e_end - cur.e_begin - 1)];
  stage_store<T, D, NT, TC>(pre, lds[0]);
  reinterpret_cast<int*>(lds[0] + L::BYTES)[tid] = pre_ent;
  __syncthreads();
  KpPass<T, D> ps;
  kp_load_pass<T, D>(ps, a, cur, rho0, kp_entry<T, D>(cur, rho0, a.g_shift, reinterpret_cast<const int*>(lds[0] + L::BYTES)));
  int buf = 0;
  for (;;) {
    const int nx = it + nsub;
    const bool has_next = nx < item_end;
    KpItem nxt = cur;
    int nxt_ent = 0;
    if (has_next) {
      nxt = kp_item_s<T, D>(a, nx);
      stage_load<T, D, NT, TC>(pre, block_ptr<TC, D>(a.k, a.v, a.page_table, nxt.b, nxt.r, a.h_kv, a.n_kv,
                                                     a.k_scale, a.v_scale));
      const int ne = nxt.e_end - nxt.e_begin;
      pre_ent = a.entries[nxt.e_begin + min(tid, ne - 1)];
      nxt_ent = a.entries[nxt.e_begin + min(rho0 >> a.g_shift, ne - 1)];
    }
    const char* L0 = lds[buf];
    const int* ent_lds = reinterpret_cast<const int*>(L0 + L::BYTES);
    TileRegs<T, D, 1> t;
    float mx = 0.f, l = 0.f;
    // an item of at most 256 rows has no second pass (uniform)
    const bool two = (cur.e_end - cur.e_begin) * a.group > kKpRowsPerPass;
    // pass 0
    KpPass<T, D> cp = ps;
    const bool act0 = __any(cp.ok);
    if (act0) kp_math<T, D>(a, cur.b, cp, L0, t, mx, l);
    if (two)
      kp_load_pass<T, D>(ps, a, cur, rho0 + kKpRowsPerPass, kp_entry<T, D>(cur, rho0 + kKpRowsPerPass, a.g_shift, ent_lds));
    else if (has_next)
      kp_load_pass<T, D>(ps, a, nxt, rho0, nxt_ent);
    kp_store<T, D, STREAM>(a, cp, t, mx, l);
    // pass 1
    if (two) {
      cp = ps;
      const bool act1 = __any(cp.ok);
      if (act1) kp_math<T, D>(a, cur.b, cp, L0, t, mx, l);
      if (has_next) kp_load_pass<T, D>(ps, a, nxt, rho0, nxt_ent);
      kp_store<T, D, STREAM>(a, cp, t, mx, l);
    }
    if (!has_next) break;
    if (NB == 1) __syncthreads();
    char* dst = lds[NB == 2 ? (buf ^ 1) : 0];
    stage_store<T, D, NT, TC>(pre, dst);
    reinterpret_cast<int*>(dst + L::BYTES)[tid] = pre_ent;
    __syncthreads();
    it = nx;
    cur = nxt;
    if (NB == 2) buf ^= 1;
  }
}

// Second stage: the diagonal block and the log-sum-exp merge ("MiniMax Sparse
// Attention" digest, §4.4.2: the query's own block as a causal tile, combined
// with the partials of its other selected blocks).  A workgroup of 4 waves
// owns the 128 (token, head) rows of one group whose positions lie in one
// aligned run of 128/G positions, so all its rows share their diagonal block.
//  A) the block's K and V^T are staged in LDS and the causal tile is computed
//     on MFMA (one 32-row tile per wave, as in the KV-outer pass); its
//     un-normalised output goes to LDS in the partial layout (part_chunk),
//     with its (max, sum), next to the (max, sum) of every (row, slot);
//  B) the merge streams the partials like a plain merge: a thread owns one
//     8-value chunk of a (token, head) row at a time, loads that chunk of all
//     the row's partial slots at once (the next chunk's loads issued before
//     the current one is combined) and writes O and lse.
// The schedule left the diagonal blocks out of the KV-outer pass, so no
// partial of them exists.  A row whose list lacks its diagonal block
// (force_local = 0, or a caller's list) gives the tile weight 0.
struct KmArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* k_scale;  // MXFP8 caches only
  const uint8_t* v_scale;
  const int32_t* page_table;
  const int32_t* block_idx;
  const void* part_o;
  const float2* part_ml;
  void* o;
  float* lse;
  int32_t n_q, q_start, n_kv, h_q, h_kv, group, g_shift, top_k, window, w;
  int32_t tile0;        // first run of this window: position / tile_tokens
  int32_t n_runs;       // runs of this window; the grid is n_runs * h_kv
  int32_t tile_tokens;  // 128 / G
  float sm_scale;
};

constexpr int kKmThreads = 256;  // 4 waves x 32 rows
constexpr int kKmRows = 128;

template <typename T, int D, typename TC = T>
__global__ __launch_bounds__(kKmThreads, 2) void km_kernel(KmArgs a) {
  using L = KvLds<T, D>;
  constexpr int DT = D / 32, DC = D / 8;
  constexpr int kPasses = kKmRows * DC / kKmThreads;  // chunks per thread in phase B
  static_assert(kPasses % 2 == 0, "phase B runs passes in pairs");
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  // phase B's use of the same LDS
  T* od_s = reinterpret_cast<T*>(lds);                                              // [rows / G][G * D]
  float2* mld_s = reinterpret_cast<float2*>(lds + (size_t)kKmRows * D * sizeof(T));  // [rows]
  float2* ml_s = mld_s + kKmRows;                                                   // [16 slots][rows]
  uint32_t* parts_s = reinterpret_cast<uint32_t*>(ml_s + kKmRows * kMaxTopK);      // [rows / G]
  static_assert((size_t)kKmRows * D * sizeof(T) + kKmRows * 8 * (1 + kMaxTopK) + kKmRows * 4 <= (size_t)L::BYTES,
                "phase B fits the K/V area");
  // Workgroup L is dispatched to XCD L % 8; each XCD takes a contiguous range of
  // (group, run) ids, so the 128 / tile_tokens runs of one diagonal block read
  // its K/V through one L2.
  int r, run;
  {
    const int n = gridDim.x, L = blockIdx.x, xcd = L & 7, q8 = n >> 3, rem = n & 7;
    const int m = xcd * q8 + min(xcd, rem) + (L >> 3);
    r = m / a.n_runs;
    run = a.tile0 + (m - r * a.n_runs);
  }
  const int G = a.group;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int rho = (tid >> 6) * 32 + l32;
  const int head = rho & (G - 1), tl = rho >> a.g_shift;
  const int p_lo = a.q_start + a.w * a.window;
  const int p_hi = a.q_start + min((a.w + 1) * a.window, a.n_q);  // exclusive
  // token (local index tt in the run) -> window row: rows outside the window
  // compute on a valid token and store nothing
  auto tok = [&](int tt, bool& ok) {
    const int pos = run * a.tile_tokens + tt;
    ok = pos >= p_lo && pos < p_hi;
    return min(max(pos, p_lo), p_hi - 1) - a.q_start;
  };
  bool ok;
  const int i = tok(tl, ok);
  const int diag = (a.q_start + i) >> 7;
  const int bdiag = (run * a.tile_tokens) >> 7;  // the same for every row of the run

  // ---- phase A: the diagonal tile
  StageRegs<T, D, kKmThreads, TC> g;
  stage_load<T, D, kKmThreads, TC>(
      g, block_ptr<TC, D>(a.k, a.v, a.page_table, bdiag, r, a.h_kv, a.n_kv, a.k_scale, a.v_scale));
  int bl[kMaxTopK];
  const uint32_t used = row_used(a.block_idx + ((size_t)i * a.h_kv + r) * a.top_k, a.top_k, diag, bl);
  uint32_t parts = used;
  bool has_diag = false;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (bl[j] == diag && ((used >> j) & 1u)) {
      has_diag = true;
      parts &= ~(1u << j);
    }
  // (max, sum) of every (row, slot), entries tid + 256 e, read now and put in
  // LDS after the tile (the slot index is clamped; unused slots are masked).
  // Slot-major, so that the merge's lanes (consecutive rows, one slot) read
  // consecutive LDS words.
  constexpr int kMlPerThread = kKmRows * kMaxTopK / kKmThreads;
  float2 mlr[kMlPerThread];
#pragma unroll
  for (int e = 0; e < kMlPerThread; ++e) {
    const int x = tid + kKmThreads * e, row = x % kKmRows, j = x / kKmRows;
    bool okr;
    const int ir = tok(row >> a.g_shift, okr);
    const size_t slot = ((size_t)(ir - a.w * a.window) * a.h_kv + r) * a.top_k + min(j, a.top_k - 1);
    mlr[e] = a.part_ml[slot * G + (row & (G - 1))];
  }
  TileRegs<T, D, 1> t;
  {
    const T* qrow = static_cast<const T*>(a.q) + ((size_t)i * a.h_q + r * G + head) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) t.qf[0][ks] = load_frag<T>(qrow + ks * 16);
  }
  t.pos[0] = a.q_start + i;
  stage_store<T, D, kKmThreads, TC>(g, lds);
  __syncthreads();
  float mx_d, l_d;
  block_tile_math<T, D>(a.sm_scale, bdiag, ok, lds, t, mx_d, l_d);
  __syncthreads();  // every wave is done with K and V^T
  {
    T* region = od_s + (size_t)tl * G * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int p = 0; p < 2; ++p) store8<T>(region + (size_t)part_chunk(dt, p, half, head, G) * 8, t.o[0][dt], 8 * p);
    if (half == 0) mld_s[rho] = has_diag ? float2{mx_d * a.sm_scale, l_d} : float2{-__builtin_inff(), 0.0f};
    if (half == 0 && head == 0) parts_s[tl] = parts;
  }
#pragma unroll
  for (int e = 0; e < kMlPerThread; ++e) ml_s[tid + kKmThreads * e] = mlr[e];
  __syncthreads();

  // ---- phase B: merge, one 8-value chunk c of token tt per thread and pass
  const int per_tok = G * DC;
  const T* po = static_cast<const T*>(a.part_o);
  auto issue = [&](Frag<T> (&x)[kMaxTopK], int pass) {
    const int u = pass * kKmThreads + tid, tt = u / per_tok, c = u % per_tok;
    bool okp;
    const int ip = tok(tt, okp);
    const uint32_t pm = parts_s[tt];
    const size_t slot0 = ((size_t)(ip - a.w * a.window) * a.h_kv + r) * a.top_k;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      // every load is issued (an unused slot reads slot 0 again) so that the
      // number in flight is fixed; an unused slot's values are zeroed below
      const size_t sj = slot0 + (((pm >> j) & 1u) ? j : 0);
      x[j] = load_frag<T>(po + sj * G * D + (size_t)c * 8);
    }
  };
  auto finish = [&](const Frag<T> (&x)[kMaxTopK], int pass) {
    const int u = pass * kKmThreads + tid, tt = u / per_tok, c = u % per_tok;
    bool okp;
    const int ip = tok(tt, okp);
    const uint32_t pm = parts_s[tt];
    const int gg = c % G, hf = (c / G) & 1, pp = (c / (2 * G)) & 1, dt = c / (4 * G);
    const int d0 = dt * 32 + 16 * pp + 4 * hf;  // the chunk holds d0..d0+3 and d0+8..d0+11
    const int row = tt * G + gg;
    const float2 md = mld_s[row];
    float2 ml[kMaxTopK];
    float mx = md.x;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      ml[j] = ((pm >> j) & 1u) ? ml_s[j * kKmRows + row] : float2{-__builtin_inff(), 0.0f};
      mx = fmaxf(mx, ml[j].x);
    }
    const float mref = mx == -__builtin_inff() ? 0.0f : mx;
    const float wd = fast_exp2((md.x - mref) * kLog2e);
    float den = wd * md.y;
    const Frag<T> xd = load_frag<T>(od_s + (size_t)tt * G * D + (size_t)c * 8);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = wd * to_f32(xd[e]);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      // a zero weight must not meet stale workspace contents (0 * inf)
      const Frag<T> xj = ((pm >> j) & 1u) ? x[j] : zero_frag<T>();
      const float w = fast_exp2((ml[j].x - mref) * kLog2e);
      den = fmaf(w, ml[j].y, den);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, to_f32(xj[e]), acc[e]);
    }
    if (!okp) return;
    T* out = static_cast<T*>(a.o) + ((size_t)ip * a.h_q + r * G + gg) * D;
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    store4<T>(out + d0, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    store4<T>(out + d0 + 8, acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    if (a.lse && c < G)
      a.lse[(size_t)ip * a.h_q + r * G + gg] = den > 0.0f ? mx + __builtin_amdgcn_logf(den) * kLn2 : -__builtin_inff();
  };
  if constexpr (sizeof(T) == 2) {
    // two buffers: the next chunk's 16 loads are in flight while one is combined
    Frag<T> xa[kMaxTopK], xb[kMaxTopK];
    issue(xa, 0);
#pragma unroll
    for (int pass = 0; pass < kPasses; pass += 2) {
      issue(xb, pass + 1);
      finish(xa, pass);
      MSA_SCHED_FENCE();
      if (pass + 2 < kPasses) issue(xa, pass + 2);
      finish(xb, pass + 1);
      MSA_SCHED_FENCE();
    }
  } else {
    // fp32 fragments are twice as wide: one buffer
    Frag<T> xa[kMaxTopK];
    for (int pass = 0; pass < kPasses; ++pass) {
      issue(xa, pass);
      finish(xa, pass);
    }
  }
}

// ====================================================================
// Dense causal GQA (Q-outer, online softmax) - the comparison kernel
// ====================================================================
struct KgArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t n_q, q_start, n_kv, h_q, h_kv, group, n_tiles, rows_per_tile;
  float sm_scale;
};

template <typename T, int D, int RT, int NT>
__global__ __launch_bounds__(NT) void kg_kernel(KgArgs a) {
  using L = KvLds<T, D>;
  constexpr int NB = (2 * L::BYTES <= 160 * 1024) ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char lds[NB][L::BYTES];
  const int tile = a.n_tiles - 1 - (int)blockIdx.x;  // longest first
  const int r = blockIdx.y;
  const int G = a.group;
  const int tok_per_tile = a.rows_per_tile / G;
  const int tok0 = tile * tok_per_tile;
  const int tok_last = min(tok0 + tok_per_tile, a.n_q) - 1;
  const int min_diag = (a.q_start + tok0) >> 7;
  const int max_diag = (a.q_start + tok_last) >> 7;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const float c2 = a.sm_scale * kLog2e;
  const T* __restrict__ q = static_cast<const T*>(a.q);
  TileRegs<T, D, RT> t;
  int tok[RT], head[RT];
  bool ok[RT];
  float mrun[RT], lrun[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rho = wave * RT * 32 + rt * 32 + l32;
    tok[rt] = tok0 + rho / G;
    head[rt] = rho % G;
    ok[rt] = (rho < a.rows_per_tile) && tok[rt] < a.n_q;
    t.pos[rt] = ok[rt] ? a.q_start + tok[rt] : -1;
    const T* qrow = q + ((size_t)(ok[rt] ? tok[rt] : 0) * a.h_q + r * G + head[rt]) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) t.qf[rt][ks] = ok[rt] ? load_frag<T>(qrow + ks * 16) : zero_frag<T>();
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) t.o[rt][dt] = f32x16{};
    mrun[rt] = -__builtin_inff();
    lrun[rt] = 0.0f;
  }
  StageRegs<T, D, NT> pre;
  stage_load<T, D, NT>(pre, block_ptr<T, D>(a.k, a.v, nullptr, 0, r, a.h_kv, a.n_kv));
  stage_store<T, D, NT>(pre, lds[0]);
  __syncthreads();
  int buf = 0;
  for (int b = 0; b <= max_diag; ++b) {
    const bool has_next = b < max_diag;
    if (has_next) stage_load<T, D, NT>(pre, block_ptr<T, D>(a.k, a.v, nullptr, b + 1, r, a.h_kv, a.n_kv));
    tile_scores<T, D, RT>(t, lds[buf], b, b >= min_diag);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float m = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) m = fmaxf(m, t.s[rt][kt][vv]);
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      const float mnew = fmaxf(mrun[rt], m);
      const float mref = (mnew == -__builtin_inff()) ? 0.0f : mnew * c2;
      const float alpha = fast_exp2(fmaf(mrun[rt], c2, -mref));
      float sum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
          const float p = fast_exp2(fmaf(t.s[rt][kt][vv], c2, -mref));
          t.s[rt][kt][vv] = p;
          sum += p;
        }
      sum += __shfl_xor(sum, 32, 64);
      lrun[rt] = lrun[rt] * alpha + sum;
      mrun[rt] = mnew;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) t.o[rt][dt] *= alpha;
      tile_pack_p<T, D, RT>(t, rt);
    }
    tile_pv<T, D, RT>(t, lds[buf]);
    if (has_next) {
      if (NB == 1) __syncthreads();
      stage_store<T, D, NT>(pre, lds[NB == 2 ? (buf ^ 1) : 0]);
      __syncthreads();
      if (NB == 2) buf ^= 1;
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (!ok[rt]) continue;
    const float inv = 1.0f / lrun[rt];
    T* dst = static_cast<T*>(a.o) + ((size_t)tok[rt] * a.h_q + r * G + head[rt]) * D + 4 * half;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int vv = 0; vv < 4; ++vv)
        store4<T>(dst + dt * 32 + 8 * vv, t.o[rt][dt][4 * vv] * inv, t.o[rt][dt][4 * vv + 1] * inv,
                  t.o[rt][dt][4 * vv + 2] * inv, t.o[rt][dt][4 * vv + 3] * inv);
    if (a.lse && half == 0)
      a.lse[(size_t)tok[rt] * a.h_q + r * G + head[rt]] =
          mrun[rt] * a.sm_scale + __builtin_amdgcn_logf(lrun[rt]) * kLn2;
  }
}

// ====================================================================
// Sparse decode
// ====================================================================
struct KdArgs {
  const void* q;             // [batch, h_q, D]
  const void* k;             // pages [*, h_kv, 128, D]
  const void* v;
  const uint8_t* k_scale;    // MXFP8 caches: [*, h_kv, 128, D / 32]
  const uint8_t* v_scale;
  const int32_t* page_table; // [batch, max_pages]
  const int32_t* seq_lens;
  const int32_t* block_idx;  // [batch, h_kv, top_k]
  void* o;
  float* lse;
  float* part_o;             // [batch, h_kv, split * waves, G, D] (split > 1), un-normalised
  float2* part_ml;           // [batch, h_kv, split * waves, G]: (scaled max, sum)
  int32_t batch, h_q, h_kv, group, top_k, max_pages, split, waves;
  float sm_scale;
};

constexpr int kKdVtStride = 32 * 2 + 8;  // bytes per d row of a 32-key V^T slice (bf16)
constexpr int kKdWaves = 8;       // waves per decode workgroup
constexpr int kKdWavesSplit = 4;  // waves per workgroup when the keys are split over workgroups

// One 32-key unit of a selected page for one wave: K rows as 16x16x32 B
// fragments (keys on the MFMA rows) and V rows as raw 16-byte pieces, to be
// transposed through LDS.
template <int D, typename TC>
struct KdUnit {
  Raw<TC> kf[2][D / 32];
  Raw<TC> vx[D / 32], vy[D / 32];
  // MXFP8: the scale bytes of K rows tt*16 + l16 and of V rows 2*l16, 2*l16 + 1
  // (a lane's dims q4*(D/4) .. +D/4 lie in one 32-element block); 0 otherwise
  uint32_t ksc[2], vsc[2];
};

// Contraction-index / V-chunk maps.  16-bit caches: step ks of lane group q4
// covers dims ks*32 + 8*q4 + e, and V chunk it of q4 is chunk q4 + 4*it.  e4m3
// caches: q4 owns the contiguous run q4*(D/4) .. +D/4 (dims q4*(D/4) + 8*ks + e,
// V chunks (D/32)*q4 + it), so each load moves 16 contiguous bytes per lane.
template <typename TC, int D>
__device__ __forceinline__ int kd_dim(int q4, int ks) {
  return sizeof(TC) == 1 ? q4 * (D / 4) + 8 * ks : ks * 32 + 8 * q4;
}
template <typename TC, int D>
__device__ __forceinline__ int kd_vchunk(int q4, int it) {
  return sizeof(TC) == 1 ? (D / 32) * q4 + it : q4 + 4 * it;
}

// `pages` holds, in lane j, the physical page of slot j (read once per
// workgroup), so a unit's address needs no dependent load.
template <int D, typename TC>
__device__ __forceinline__ void kd_load_unit(KdUnit<D, TC>& x, const KdArgs& a, int pages, int r, int u) {
  const int lane = threadIdx.x & 63, q4 = lane >> 4, l16 = lane & 15;
  const int j = u >> 2, qq = u & 3;
  const int page = __builtin_amdgcn_readlane(pages, j);
  const size_t base = (((size_t)page * a.h_kv + r) * kBlock + qq * 32) * D;
  const TC* kb = static_cast<const TC*>(a.k) + base;
  const TC* vb = static_cast<const TC*>(a.v) + base;
  if constexpr (kIsMx<TC>) {
    const size_t sbase = base / kMxBlock + (q4 * (D / 4)) / kMxBlock;
    x.ksc[0] = a.k_scale[sbase + (size_t)l16 * (D / kMxBlock)];
    x.ksc[1] = a.k_scale[sbase + (size_t)(16 + l16) * (D / kMxBlock)];
    x.vsc[0] = a.v_scale[sbase + (size_t)(2 * l16) * (D / kMxBlock)];
    x.vsc[1] = a.v_scale[sbase + (size_t)(2 * l16 + 1) * (D / kMxBlock)];
  } else {
    x.ksc[0] = x.ksc[1] = x.vsc[0] = x.vsc[1] = 0u;
  }
  if constexpr (sizeof(TC) == 1) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < D / 32; ks += 2) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(kb + (tt * 16 + l16) * D + kd_dim<TC, D>(q4, ks));
        x.kf[tt][ks] = u32x2{w[0], w[1]};
        x.kf[tt][ks + 1] = u32x2{w[2], w[3]};
      }
#pragma unroll
    for (int it = 0; it < D / 32; it += 2) {
      const int c = 8 * kd_vchunk<TC, D>(q4, it);
      const u32x4 wx = *reinterpret_cast<const u32x4*>(vb + (2 * l16) * D + c);
      const u32x4 wy = *reinterpret_cast<const u32x4*>(vb + (2 * l16 + 1) * D + c);
      x.vx[it] = u32x2{wx[0], wx[1]};
      x.vx[it + 1] = u32x2{wx[2], wx[3]};
      x.vy[it] = u32x2{wy[0], wy[1]};
      x.vy[it + 1] = u32x2{wy[2], wy[3]};
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) x.kf[tt][ks] = load_raw<TC>(kb + (tt * 16 + l16) * D + kd_dim<TC, D>(q4, ks));
#pragma unroll
    for (int it = 0; it < D / 32; ++it) {
      const int c = 8 * kd_vchunk<TC, D>(q4, it);
      x.vx[it] = load_raw<TC>(vb + (2 * l16) * D + c);
      x.vy[it] = load_raw<TC>(vb + (2 * l16 + 1) * D + c);
    }
  }
}

// Workgroup (sequence s, group r, split sp) of NW waves.  The selected keys
// are cut into 32-key units (4 per page); wave w of split sp takes units
// sp*NW + w, + NW*split, ...  Each wave keeps an online softmax over its
// units with the next unit's loads in flight while the current one is
// computed.  Without a split the NW waves are then combined in LDS; with one,
// every wave writes its own partial (un-normalised output and its max and
// sum), and kd_merge_kernel combines all of a (sequence, group)'s partials,
// so no wave waits on the others.
template <int D, int NW, typename TC>
__global__ __launch_bounds__(NW * 64) void kd_kernel(KdArgs a) {
  typedef bf16_t T;
  constexpr int kVtBytes = D * kKdVtStride;
  constexpr int kOBytes = 16 * (D + 1) * 4;
  constexpr int kSlab = kVtBytes > kOBytes ? kVtBytes : kOBytes;
  // per wave: the V^T slice while units run, then its output rows
  __shared__ __attribute__((aligned(16))) char slab[NW][kSlab];
  __shared__ float2 mls[NW][16];  // per wave and head: (scaled max, sum)
  __shared__ float cw[NW][16];    // per wave and head: e^(m_w - M) / denominator
  const int sp = blockIdx.x % a.split;
  const int sr = blockIdx.x / a.split;
  const int s = sr / a.h_kv, r = sr % a.h_kv;
  // the wave index is made uniform so that the unit loop below is scalar
  // control flow: loads under per-lane branches make the compiler wait for
  // every load in flight (the prefetched unit included) before the next use
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, q4 = lane >> 4, l16 = lane & 15;
  const int G = a.group;
  const int32_t* br = a.block_idx + ((size_t)s * a.h_kv + r) * a.top_k;
  const T* __restrict__ qp = static_cast<const T*>(a.q) + ((size_t)s * a.h_q + r * G) * D;
  // The block list, the queries and the sequence length are loaded at once
  // (every load unconditional, with clamped indices, so none waits behind a
  // branch), then the page ids of the listed blocks: lane j holds block and
  // physical page of slot j.  The start-up waits on two round trips.
  const int bv_raw = br[min(lane, a.top_k - 1)];
  Frag<T> qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qf[ks] = load_frag<T>(qp + (size_t)min(l16, G - 1) * D + kd_dim<TC, D>(q4, ks));
  const int L = scalar_load(a.seq_lens, s);
  const int bv = lane < a.top_k ? bv_raw : -1;
  const int pall = a.page_table[(size_t)s * a.max_pages + min(max(bv, 0), a.max_pages - 1)];
  const int p = L - 1, diag = p >> 7;
  uint32_t used = 0;
  {
    int prev = -1;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      const int b = __builtin_amdgcn_readlane(bv, j);
      if (j < a.top_k && b > prev && b <= diag) {
        used |= 1u << j;
        prev = b;
      }
    }
  }
  const bool mine = lane < a.top_k && ((used >> lane) & 1u);
  const int bl = mine ? bv : 0;
  const int pages = mine ? pall : 0;
  const float c2 = a.sm_scale * kLog2e;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    if (l16 >= G) qf[ks] = zero_frag<T>();
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{};
  float mrun = -__builtin_inff(), lrun = 0.0f;
  char* vt = slab[wave];
  const int n_units = a.top_k * 4;
  const int step = a.split * NW;
  int u = sp * NW + wave;
  while (u < n_units && !((used >> (u >> 2)) & 1u)) u += step;
  KdUnit<D, TC> cur, nxt;
  if (u < n_units) kd_load_unit<D, TC>(cur, a, pages, r, u);
  while (u < n_units) {
    int un = u + step;
    while (un < n_units && !((used >> (un >> 2)) & 1u)) un += step;
    // unconditional, so the wait before the math below covers the current
    // unit only; past the last unit it reloads the current one (an L2 hit)
    kd_load_unit<D, TC>(nxt, a, pages, r, un < n_units ? un : u);
    MSA_SCHED_FENCE();  // keep the prefetch ahead of the math
    const int b = __builtin_amdgcn_readlane(bl, u >> 2);
    f32x4 sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sc[tt] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) mma16(sc[tt], widen<T, TC>(cur.kf[tt][ks], cur.ksc[tt]), qf[ks]);
    }
    // sc[tt][v]: key (u%4)*32 + tt*16 + 4*q4 + v of block b, head l16
    const int key0 = b * kBlock + (u & 3) * 32;
    float m = -__builtin_inff();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (key0 + tt * 16 + 4 * q4 + v > p) sc[tt][v] = -__builtin_inff();
        m = fmaxf(m, sc[tt][v]);
      }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    // transpose V into LDS: V^T[d][key], key pairs packed per dword
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < D / 32; ++it) {
      const int dc = kd_vchunk<TC, D>(q4, it);
      const u32x4 vx = __builtin_bit_cast(u32x4, widen<T, TC>(cur.vx[it], cur.vsc[0]));
      const u32x4 vy = __builtin_bit_cast(u32x4, widen<T, TC>(cur.vy[it], cur.vsc[1]));
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        const uint32_t lo = (vx[t2] & 0xffffu) | (vy[t2] << 16);
        const uint32_t hi = (vx[t2] >> 16) | (vy[t2] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(vt + (8 * dc + 2 * t2) * kKdVtStride + l16 * 4) = lo;
        *reinterpret_cast<uint32_t*>(vt + (8 * dc + 2 * t2 + 1) * kKdVtStride + l16 * 4) = hi;
      }
    }
    const float mnew = fmaxf(mrun, m);
    const float mref = (mnew == -__builtin_inff()) ? 0.0f : mnew * c2;
    const float alpha = fast_exp2(fmaf(mrun, c2, -mref));
    float pv[8];
    float sum = 0.0f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pv[tt * 4 + v] = fast_exp2(fmaf(sc[tt][v], c2, -mref));
        sum += pv[tt * 4 + v];
      }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    lrun = lrun * alpha + sum;
    mrun = mnew;
    const Frag<T> pf = to_frag<T>(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      o[dt] *= alpha;
      const Frag<T> af = vt_frag<T>(vt, kKdVtStride, dt * 16 + l16, 4 * q4, 16 + 4 * q4);
      mma16(o[dt], af, pf);
    }
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
    u = un;
  }
  // o[dt][v]: d = dt*16 + 4*q4 + v, head l16.
  if (a.split > 1) {
    const size_t pidx = (((size_t)sr * a.split + sp) * NW + wave) * G + l16;
    if (l16 < G) {
      float* po = a.part_o + pidx * D + 4 * q4;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[dt];
      if (q4 == 0) a.part_ml[pidx] = float2{lrun > 0.0f ? mrun * a.sm_scale : -__builtin_inff(), lrun};
    }
    return;
  }
  // Combine the NW waves: each wave's slab now holds its un-normalised output
  // rows and mls its (max, sum) per head.  The weights e^(m_w - M) / den are
  // formed once per (wave, head); then every thread sums 4 consecutive dims of
  // one head over the waves.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* ow = reinterpret_cast<float*>(vt);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int v = 0; v < 4; ++v) ow[l16 * (D + 1) + dt * 16 + 4 * q4 + v] = o[dt][v];
  if (q4 == 0) mls[wave][l16] = float2{lrun > 0.0f ? mrun * a.sm_scale : -__builtin_inff(), lrun};
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float mx = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, mls[w][g].x);
    const float mref = mx == -__builtin_inff() ? 0.0f : mx;
    float e[NW];
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      e[w] = fast_exp2((mls[w][g].x - mref) * kLog2e);  // 0 for a wave without keys
      den = fmaf(e[w], mls[w][g].y, den);
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) cw[w][g] = e[w] * inv;
    if (a.lse)
      a.lse[(size_t)s * a.h_q + r * G + g] = den > 0.0f ? mref + __builtin_amdgcn_logf(den) * kLn2 : -__builtin_inff();
  }
  __syncthreads();
  for (int x = threadIdx.x; x < G * (D / 4); x += NW * 64) {
    const int g = x / (D / 4), d0 = (x % (D / 4)) * 4;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = cw[w][g];
      const float* src = reinterpret_cast<const float*>(slab[w]) + g * (D + 1) + d0;
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = fmaf(c, src[t], acc[t]);
    }
    store4<T>(static_cast<T*>(a.o) + ((size_t)s * a.h_q + r * G + g) * D + d0, acc[0], acc[1], acc[2], acc[3]);
  }
}

// Merge of the per-wave partials of a split decode: one workgroup per
// (sequence, group, head).  With M the largest partial max,
//   o = sum_k e^(m_k - M) o_k / sum_k e^(m_k - M) l_k,  lse = M + ln(sum_k e^(m_k - M) l_k).
// Lane k of wave 0 holds partial k's (max, sum): M and the denominator are
// wave reductions and the weights go to LDS.  Thread (quarter qq, dim d) sums
// partials 16 qq .. 16 qq + 15 of dim d, all loaded before any is used (a
// clamped index keeps the loads unconditional; the weight of a partial past
// the last is 0), and the four quarters are added in LDS.
constexpr int kKdMaxParts = 64;  // split (a power of two, at most 16 for top_k <= 16) * 4 waves
constexpr int kKdMergeQuarter = kKdMaxParts / 4;
template <int D>
__global__ __launch_bounds__(4 * D) void kd_merge_kernel(KdArgs a) {
  __shared__ __attribute__((aligned(16))) float w_s[kKdMaxParts];
  __shared__ float acc_s[4][D];
  __shared__ float2 md_s;  // (M, denominator)
  const int G = a.group;
  const int sr = blockIdx.x / G, g = blockIdx.x % G;
  const int s = sr / a.h_kv, r = sr % a.h_kv;
  const int d = threadIdx.x % D, qq = threadIdx.x / D;
  const int np = a.split * a.waves;
  const size_t base = (size_t)sr * np * G + g;  // + k * G for partial k
  float x[kKdMergeQuarter];
#pragma unroll
  for (int e = 0; e < kKdMergeQuarter; ++e)
    x[e] = a.part_o[(base + (size_t)min(qq * kKdMergeQuarter + e, np - 1) * G) * D + d];
  if (threadIdx.x < 64) {
    const int k = threadIdx.x;
    const float2 ml = k < np ? a.part_ml[base + (size_t)k * G] : float2{-__builtin_inff(), 0.0f};
    float mx = ml.x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float mref = mx == -__builtin_inff() ? 0.0f : mx;
    const float w = fast_exp2((ml.x - mref) * kLog2e);  // 0 for an empty or missing partial
    float den = w * ml.y;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) den += __shfl_xor(den, o, 64);
    w_s[k] = w;
    if (k == 0) md_s = float2{mref, den};
  }
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < kKdMergeQuarter; e += 4) {
    const f32x4 w4 = *reinterpret_cast<const f32x4*>(w_s + qq * kKdMergeQuarter + e);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = fmaf(w4[t], x[e + t], acc);
  }
  acc_s[qq][d] = acc;
  __syncthreads();
  if (qq != 0) return;
  const float mref = md_s.x, den = md_s.y;
  acc = acc_s[0][d] + acc_s[1][d] + acc_s[2][d] + acc_s[3][d];
  bf16_t* out = static_cast<bf16_t*>(a.o) + ((size_t)s * a.h_q + r * G + g) * D + d;
  *out = from_f32<bf16_t>(den > 0.0f ? acc / den : 0.0f);
  if (a.lse && d == 0)
    a.lse[(size_t)s * a.h_q + r * G + g] = den > 0.0f ? mref + __builtin_amdgcn_logf(den) * kLn2 : -__builtin_inff();
}

// ====================================================================
// Host side: plans and launches
// ====================================================================
static size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Largest block count whose schedule counters live in LDS; a test hook can
// lower it (to 0) so that the tests run the global-atomic path too.
static std::atomic<int> g_sched_lds_limit{-1};
void set_schedule_lds_limit(int max_blocks) { g_sched_lds_limit.store(max_blocks < 0 ? -1 : max_blocks); }
static int sched_lds_limit(int dflt) {
  const int v = g_sched_lds_limit.load();
  return v < 0 ? dflt : std::min(v, dflt);
}

// Compute units of the current device (cached per device).
int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// KV-outer workgroups per CU: one 512-thread workgroup with two 64 KB K/V
// buffers fills a CU's LDS.
constexpr int kKpWgPerCu = 1;

void schedule_layout(PrefillPlan& p, int32_t n_q, int32_t q_start, int32_t h_kv, int32_t top_k, int32_t window,
                     int32_t chunk, bool ordered) {
  p.n_blocks = (int32_t)((((int64_t)q_start + n_q - 1) / kBlock + 1 + 7) & ~int64_t(7));
  p.window = window;
  p.n_windows = (int32_t)((n_q + window - 1) / window);
  p.merge_windows = 1;
  p.stream_partials = 0;
  p.chunk = chunk;
  p.n_cells = (int64_t)p.n_windows * h_kv * p.n_blocks;
  const int64_t n_entries = (int64_t)n_q * h_kv * top_k;
  p.max_items = n_entries / p.chunk + p.n_cells + 1;
  const int64_t n_scan_tiles = (p.n_cells + kScanTile - 1) / kScanTile;
  size_t off = 0;
  p.off_count = off; off = align_up(off + p.n_cells * 4);
  p.off_fill = off; off = align_up(off + p.n_cells * 4);
  p.off_cell_off = off; off = align_up(off + (p.n_cells + 1) * 4);
  p.off_item_off = off; off = align_up(off + (p.n_cells + 1) * 4);
  p.off_entries = off; off = align_up(off + n_entries * 4);
  p.off_items = off; off = align_up(off + p.max_items * 16);
  p.off_scan = off; off = align_up(off + 4 * n_scan_tiles * 4);
  p.bitmap_words = ordered ? (window + 31) / 32 : 0;
  p.off_bitmap = off; off = align_up(off + (size_t)p.n_cells * p.bitmap_words * 4);
  p.total = off;
}

// Window sizing of the sparse prefill (measured optima, see prefill_plan):
// partial bytes a window may use at least and at most, the average tokens
// per (group, block) cell the window is grown to; the partial bytes up to
// which a window is merged on its own (the last-level cache holds them), and
// the tokens one merge launch spans past that.
constexpr size_t kPartialBudgetBytes = size_t(128) << 20;
constexpr size_t kPartialCapBytes = size_t(4096) << 20;
constexpr int64_t kCellTokens = 40;
constexpr size_t kMergeAloneBytes = size_t(256) << 20;
constexpr int64_t kMergeSpanTokens = 12288;

PrefillPlan prefill_plan(int dtype, int32_t n_q, int32_t q_start, int32_t n_kv, int32_t h_q,
                         int32_t h_kv, int32_t d_h, int32_t top_k) {
  PrefillPlan p{};
  const size_t esz = dtype == 0 ? 2 : 4;
  const int G = h_q / h_kv;
  (void)n_kv;
  const size_t per_token = (size_t)h_kv * top_k * G * (d_h * esz + 8);
  // Window of query tokens per KV-outer pass.  Its partials should stay in
  // the last-level cache (the budget), but with many blocks to choose from a
  // small window leaves few tokens per (group, block) cell and the items
  // mostly empty, so the window grows until a cell holds about
  // `cell_tokens` tokens on average (bounded by a hard memory cap).
  const size_t budget = kPartialBudgetBytes;
  const size_t cap = kPartialCapBytes;
  const int64_t cell_tokens = kCellTokens;
  const int64_t blocks_seen = ((int64_t)q_start + n_q - 1) / kBlock + 1;
  int64_t w = (int64_t)(budget / per_token);
  const int64_t w_occ = (cell_tokens * blocks_seen + std::max(1, top_k - 1) - 1) / std::max(1, top_k - 1);
  w = std::max<int64_t>(w, std::min<int64_t>(w_occ, (int64_t)(cap / per_token)));
  w = std::max<int64_t>(64, ((w + 63) / 64) * 64);
  w = std::min<int64_t>(w, std::max<int32_t>(n_q, 1));
  p.window = (int32_t)w;
  schedule_layout(p, n_q, q_start, h_kv, top_k, (int32_t)w, 512 / G);  // items of 512 (token, head) rows
  // A window whose partials fit the last-level cache is merged on its own,
  // while they are still cached.  Past that they reach HBM anyway; each merge
  // launch has a fixed cost (its start, where every workgroup stages its
  // diagonal block at once, and its tail), so the partials of several
  // consecutive windows are kept side by side and merged by one launch.
  // Partials that wait for a merge of several windows are stored
  // non-temporally: streaming stores keep them from displacing the gathered
  // queries and staged blocks in L2 (measured at 128K: KV-outer pass -6%,
  // merge -5%).  A single long window (a chunk at long context, about 15
  // tokens per cell, K/V most of the traffic) keeps plain stores, where
  // streaming ones slowed the KV-outer pass by 10%.
  int64_t mw = 1;
  if ((size_t)w * per_token > kMergeAloneBytes) {
    mw = std::max<int64_t>(1, std::min<int64_t>(kMergeSpanTokens / w, (int64_t)(cap / per_token) / w));
    mw = std::min<int64_t>(mw, p.n_windows);
  }
  p.merge_windows = (int32_t)mw;
  p.stream_partials = mw > 1 ? 1 : 0;
  size_t off = p.total;
  const size_t prow = ((size_t)p.window * mw * h_kv * top_k + 2) * G;  // + two trash slots
  p.off_part_o = off; off = align_up(off + prow * d_h * esz);
  p.off_part_lse = off; off = align_up(off + prow * 8);
  p.total = off;
  return p;
}

bool attn_supported(int dtype, int d_h) { return (dtype == 0 || dtype == 1) && (d_h == 64 || d_h == 128); }
bool dense_supported(int dtype, int d_h) { return attn_supported(dtype, d_h); }
bool decode_supported(int dtype, int d_h) { return (dtype == 0 || dtype >= 2) && (d_h == 64 || d_h == 128); }

hipError_t launch_prefill_schedule(const AttnArgs& a, const PrefillPlan& pl, SchedArgs& s, hipStream_t st,
                                   bool skip_diag) {
  char* ws = static_cast<char*>(a.ws);
  s = SchedArgs{};
  s.skip_diag = skip_diag ? 1 : 0;
  s.block_idx = a.block_idx;
  s.n_q = a.n_q;
  s.q_start = a.q_start;
  s.h_kv = a.h_kv;
  s.top_k = a.top_k;
  s.n_blocks = pl.n_blocks;
  s.window = pl.window;
  s.chunk = pl.chunk;
  s.n_cells = pl.n_cells;
  s.count = reinterpret_cast<int32_t*>(ws + pl.off_count);
  s.fill = reinterpret_cast<int32_t*>(ws + pl.off_fill);
  s.cell_off = reinterpret_cast<int32_t*>(ws + pl.off_cell_off);
  s.item_off = reinterpret_cast<int32_t*>(ws + pl.off_item_off);
  s.entries = reinterpret_cast<int32_t*>(ws + pl.off_entries);
  s.items = reinterpret_cast<i32x4*>(ws + pl.off_items);
  s.scan = reinterpret_cast<int32_t*>(ws + pl.off_scan);
  s.n_scan_tiles = (int32_t)((pl.n_cells + kScanTile - 1) / kScanTile);
  s.words = pl.bitmap_words;
  s.bitmap = pl.bitmap_words > 0 ? reinterpret_cast<uint32_t*>(ws + pl.off_bitmap) : nullptr;
  const int64_t rows = (int64_t)a.n_q * a.h_kv;
  const unsigned row_blocks = (unsigned)((rows + 255) / 256);
  // LDS counters while a window's blocks fit (the threshold can be lowered
  // through the environment, which is how the global-atomic path is tested)
  const bool lds_sched = pl.n_blocks <= sched_lds_limit(kSchedLdsBlocks);
  // With few (window, group) pairs (one long window, as in a chunked prefill
  // at long context) each is split into token slices, enough to fill the
  // chip, of at least 128 tokens; otherwise one workgroup per pair (slices
  // would count every entry twice and add global atomics)
  {
    const int64_t wg = (int64_t)pl.n_windows * a.h_kv;
    const int64_t want = wg * 2 < num_cus() ? (2LL * num_cus() + wg - 1) / wg : 1;
    s.split = (int32_t)std::max<int64_t>(1, std::min<int64_t>(want, pl.window / 128));
  }
  const unsigned cell_blocks = (unsigned)((pl.n_cells + 255) / 256);
  if (s.bitmap) {  // ordered: bitmap -> counts -> offsets -> token lists in order
    if (pl.n_blocks <= sched_lds_limit(kBitsLdsBlocks)) {
      const unsigned tiles = (unsigned)((pl.window + 255) / 256);
      hipLaunchKernelGGL(ks_bits_set_lds_kernel, dim3((unsigned)pl.n_windows * tiles, (unsigned)a.h_kv), dim3(256),
                         (size_t)pl.n_blocks * 8 * 4, st, s);
    } else {
      const int64_t nw = pl.n_cells * s.words;
      hipLaunchKernelGGL(ks_bits_zero_kernel, dim3((unsigned)std::min<int64_t>((nw + 255) / 256, 8192)), dim3(256),
                         0, st, s);
      hipLaunchKernelGGL(ks_bits_set_kernel, dim3(row_blocks), dim3(256), 0, st, s);
    }
    hipLaunchKernelGGL(ks_bits_count_kernel, dim3((unsigned)pl.n_cells), dim3(256), 0, st, s);
  } else if (lds_sched) {
    if (s.split > 1)
      hipLaunchKernelGGL(ks_zero_kernel, dim3(std::min<unsigned>(cell_blocks, 4096u)), dim3(256), 0, st, s);
    hipLaunchKernelGGL(ks_count_lds_kernel, dim3((unsigned)(pl.n_windows * s.split), (unsigned)a.h_kv), dim3(256),
                       (size_t)pl.n_blocks * 4, st, s);
  } else {
    hipLaunchKernelGGL(ks_zero_kernel, dim3(std::min<unsigned>(cell_blocks, 4096u)), dim3(256), 0, st, s);
    hipLaunchKernelGGL(ks_count_kernel, dim3(row_blocks), dim3(256), 0, st, s);
  }
  hipLaunchKernelGGL(ks_scan_a_kernel, dim3(s.n_scan_tiles), dim3(256), 0, st, s);
  hipLaunchKernelGGL(ks_scan_b_kernel, dim3(1), dim3(256), 0, st, s);
  hipLaunchKernelGGL(ks_scan_c_kernel, dim3(s.n_scan_tiles), dim3(256), 0, st, s);
  if (s.bitmap)
    hipLaunchKernelGGL(ks_bits_extract_kernel, dim3((unsigned)pl.n_cells), dim3(256), 0, st, s);
  else if (lds_sched)
    hipLaunchKernelGGL(ks_scatter_lds_kernel, dim3((unsigned)(pl.n_windows * s.split), (unsigned)a.h_kv), dim3(256),
                       (size_t)pl.n_blocks * 4, st, s);
  else
    hipLaunchKernelGGL(ks_scatter_kernel, dim3(row_blocks), dim3(256), 0, st, s);
  hipLaunchKernelGGL(ks_items_kernel, dim3(cell_blocks), dim3(256), 0, st, s);
  return hipGetLastError();
}

template <typename T, int D, typename TC = T>
static hipError_t sparse_prefill_typed(const AttnArgs& a, const PrefillPlan& pl, hipStream_t st) {
  char* ws = static_cast<char*>(a.ws);
  SchedArgs s;
  hipError_t e = launch_prefill_schedule(a, pl, s, st, /*skip_diag=*/true);
  if (e != hipSuccess) return e;

  KpArgs kp{};
  kp.q = a.q;
  kp.k = a.k;
  kp.v = a.v;
  kp.k_scale = a.k_scale;
  kp.v_scale = a.v_scale;
  kp.page_table = a.page_table;
  kp.cell_off = s.cell_off;
  kp.item_off = s.item_off;
  kp.entries = s.entries;
  kp.items = s.items;
  kp.part_o = ws + pl.off_part_o;
  kp.part_ml = reinterpret_cast<float2*>(ws + pl.off_part_lse);
  const int span = pl.window * pl.merge_windows;  // tokens whose partials the buffer holds
  kp.trash_slot = (size_t)span * a.h_kv * a.top_k;
  kp.n_kv = a.n_kv;
  kp.q_start = a.q_start;
  kp.h_q = a.h_q;
  kp.h_kv = a.h_kv;
  kp.group = a.group;
  kp.g_shift = __builtin_ctz((unsigned)a.group);
  kp.top_k = a.top_k;
  kp.n_blocks = pl.n_blocks;
  kp.window = pl.window;
  kp.chunk = pl.chunk;
  kp.sm_scale = a.sm_scale;

  KmArgs km{};
  km.q = a.q;
  km.k = a.k;
  km.v = a.v;
  km.k_scale = a.k_scale;
  km.v_scale = a.v_scale;
  km.page_table = a.page_table;
  km.block_idx = a.block_idx;
  km.part_o = kp.part_o;
  km.part_ml = kp.part_ml;
  km.o = a.o;
  km.lse = a.lse;
  km.n_q = a.n_q;
  km.q_start = a.q_start;
  km.n_kv = a.n_kv;
  km.h_q = a.h_q;
  km.h_kv = a.h_kv;
  km.group = a.group;
  km.g_shift = kp.g_shift;
  km.top_k = a.top_k;
  km.window = span;
  km.tile_tokens = kKmRows / a.group;
  km.sm_scale = a.sm_scale;

  const int n_cu = num_cus();
  for (int w = 0; w < pl.n_windows; ++w) {
    const int tok = std::min<int>(pl.window, a.n_q - w * pl.window);
    const int64_t bound = (int64_t)tok * a.h_kv * a.top_k / pl.chunk + (int64_t)a.h_kv * pl.n_blocks + 1;
    kp.w = w;
    kp.slot_tok0 = (w / pl.merge_windows) * span;
    int64_t g = std::min<int64_t>(bound + 8, (int64_t)n_cu * kKpWgPerCu);
    const unsigned grid = (unsigned)std::max<int64_t>(8, (g + 7) & ~int64_t(7));
    const int pk = profile_begin(PK_KP, st);
    if (pl.stream_partials)
      hipLaunchKernelGGL((kp_kernel<T, D, TC, true>), dim3(grid), dim3(kKpThreads), 0, st, kp);
    else
      hipLaunchKernelGGL((kp_kernel<T, D, TC, false>), dim3(grid), dim3(kKpThreads), 0, st, kp);
    profile_end(pk, st);
    // merge once the span's last window (or the call's) is done
    if ((w + 1) % pl.merge_windows != 0 && w + 1 < pl.n_windows) continue;
    km.w = w / pl.merge_windows;
    // aligned runs of tile_tokens positions that meet the span's positions
    const int p0 = a.q_start + km.w * span, p1 = a.q_start + std::min<int>(a.n_q, (km.w + 1) * span);
    km.tile0 = p0 / km.tile_tokens;
    km.n_runs = (p1 - 1) / km.tile_tokens - km.tile0 + 1;
    const int pm = profile_begin(PK_KM, st);
    hipLaunchKernelGGL((km_kernel<T, D, TC>), dim3((unsigned)(km.n_runs * a.h_kv)), dim3(kKmThreads), 0, st, km);
    profile_end(pm, st);
  }
  return hipGetLastError();
}

hipError_t launch_sparse_prefill(int dtype, int d_h, const AttnArgs& a, const PrefillPlan& pl,
                                 hipStream_t st) {
  if (dtype == 2 && d_h == 128) return sparse_prefill_typed<bf16_t, 128, fp8_t>(a, pl, st);
  if (dtype == 2 && d_h == 64) return sparse_prefill_typed<bf16_t, 64, fp8_t>(a, pl, st);
  if (dtype == 3 && d_h == 128) return sparse_prefill_typed<bf16_t, 128, mx8_t>(a, pl, st);
  if (dtype == 3 && d_h == 64) return sparse_prefill_typed<bf16_t, 64, mx8_t>(a, pl, st);
  if (dtype == 0 && d_h == 128) return sparse_prefill_typed<bf16_t, 128>(a, pl, st);
  if (dtype == 0 && d_h == 64) return sparse_prefill_typed<bf16_t, 64>(a, pl, st);
  if (dtype == 1 && d_h == 128) return sparse_prefill_typed<float, 128>(a, pl, st);
  if (dtype == 1 && d_h == 64) return sparse_prefill_typed<float, 64>(a, pl, st);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t dense_typed(const AttnArgs& a, hipStream_t st) {
  KgArgs g{};
  g.q = a.q;
  g.k = a.k;
  g.v = a.v;
  g.o = a.o;
  g.lse = a.lse;
  g.n_q = a.n_q;
  g.q_start = a.q_start;
  g.n_kv = a.n_kv;
  g.h_q = a.h_q;
  g.h_kv = a.h_kv;
  g.group = a.group;
  constexpr int RT = 1, NT = 512;
  g.rows_per_tile = (NT / 64) * RT * 32;
  const int tok_per_tile = g.rows_per_tile / a.group;
  g.n_tiles = (a.n_q + tok_per_tile - 1) / tok_per_tile;
  g.sm_scale = a.sm_scale;
  hipLaunchKernelGGL((kg_kernel<T, D, RT, NT>), dim3(g.n_tiles, a.h_kv), dim3(NT), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_dense_prefill(int dtype, int d_h, const AttnArgs& a, hipStream_t st) {
  if (dtype == 0 && d_h == 128) return dense_typed<bf16_t, 128>(a, st);
  if (dtype == 0 && d_h == 64) return dense_typed<bf16_t, 64>(a, st);
  if (dtype == 1 && d_h == 128) return dense_typed<float, 128>(a, st);
  if (dtype == 1 && d_h == 64) return dense_typed<float, 64>(a, st);
  return hipErrorInvalidValue;
}

DecodePlan decode_plan(int32_t batch, int32_t h_q, int32_t h_kv, int32_t d_h, int32_t top_k) {
  DecodePlan p{};
  const int pairs = batch * h_kv;
  int split = 1, waves = kKdWaves;
  // One workgroup of 8 waves per (sequence, group) while that gives one per
  // CU or more; with fewer pairs the selected keys are split over workgroups
  // of 4 waves (more, smaller workgroups start their loads sooner), aiming at
  // >= 256 workgroups while every wave keeps at least one 32-key unit.  The
  // splits are combined by kd_merge_kernel.
  if (pairs < 256) {
    waves = kKdWavesSplit;
    while (split * waves < top_k * 4 && (int64_t)pairs * split < 256) split <<= 1;
  }
  p.split = split;
  p.waves = waves;
  const int G = h_q / h_kv;
  const size_t parts = (size_t)pairs * split * waves * G;  // one partial per wave and head
  size_t off = 0;
  p.off_part_o = off; off = align_up(off + parts * d_h * 4);
  p.off_part_lse = off; off = align_up(off + parts * 8);
  p.total = split > 1 ? off : 0;
  return p;
}

template <int D, typename TC>
static hipError_t decode_typed(const AttnArgs& a, const DecodePlan& pl, hipStream_t st) {
  KdArgs k{};
  k.q = a.q;
  k.k = a.k;
  k.v = a.v;
  k.k_scale = a.k_scale;
  k.v_scale = a.v_scale;
  k.page_table = a.page_table;
  k.seq_lens = a.seq_lens;
  k.block_idx = a.block_idx;
  k.o = a.o;
  k.lse = a.lse;
  char* ws = static_cast<char*>(a.ws);
  k.part_o = pl.split > 1 ? reinterpret_cast<float*>(ws + pl.off_part_o) : nullptr;
  k.part_ml = pl.split > 1 ? reinterpret_cast<float2*>(ws + pl.off_part_lse) : nullptr;
  k.batch = a.batch;
  k.h_q = a.h_q;
  k.h_kv = a.h_kv;
  k.group = a.group;
  k.top_k = a.top_k;
  k.max_pages = a.max_pages;
  k.split = pl.split;
  k.waves = pl.waves;
  k.sm_scale = a.sm_scale;
  if (pl.split > 1 && pl.split * pl.waves > kKdMaxParts) return hipErrorInvalidValue;
  const int pd = profile_begin(PK_KD, st);
  const dim3 grid((unsigned)(a.batch * a.h_kv * pl.split));
  if (pl.waves == kKdWavesSplit)
    hipLaunchKernelGGL((kd_kernel<D, kKdWavesSplit, TC>), grid, dim3(kKdWavesSplit * 64), 0, st, k);
  else
    hipLaunchKernelGGL((kd_kernel<D, kKdWaves, TC>), grid, dim3(kKdWaves * 64), 0, st, k);
  profile_end(pd, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.split == 1) return e;
  hipLaunchKernelGGL((kd_merge_kernel<D>), dim3(a.batch * a.h_kv * a.group), dim3(4 * D), 0, st, k);
  return hipGetLastError();
}

hipError_t launch_sparse_decode(int dtype, int d_h, const AttnArgs& a, const DecodePlan& pl,
                                hipStream_t st) {
  if (dtype == 0) {
    if (d_h == 128) return decode_typed<128, bf16_t>(a, pl, st);
    if (d_h == 64) return decode_typed<64, bf16_t>(a, pl, st);
  } else if (dtype == 2) {  // bf16 queries, e4m3 cached keys and values
    if (d_h == 128) return decode_typed<128, fp8_t>(a, pl, st);
    if (d_h == 64) return decode_typed<64, fp8_t>(a, pl, st);
  } else if (dtype == 3) {  // bf16 queries, MXFP8 cached keys and values
    if (d_h == 128) return decode_typed<128, mx8_t>(a, pl, st);
    if (d_h == 64) return decode_typed<64, mx8_t>(a, pl, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
