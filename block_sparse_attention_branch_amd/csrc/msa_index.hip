// msa_index.hip - index branch of MiniMax Sparse Attention on gfx950.
//
// Computes, per query and KV group r ("MiniMax Sparse Attention" digest,
// titansim.online, §4.2 Eq. (6) and §4.4.1; tensor shapes per the 163.com
// commentary, "Step 1 Index Attention"):
//   S_j = q_idx^(r) . k_idx_j * idx_scale        (keys j <= p)
//   M_b = max_{j in block b, j <= p} S_j          (block max-pool; as an
//         ablation the mean over the same keys, the block scoring the
//         163.com commentary attributes to MoBA)
//   I   = top-k of M on the raw scores (no exp / softmax: the order is the
//         same), ties to the lower block, diagonal block kept if forced.
//
// Prefill kernel: one workgroup = 256 (query, group) rows x one chunk of KV
// blocks.  Each 128-key index block is staged once in LDS and shared by the 4
// waves; a wave computes S^T = K_idx_block . Q_idx^T for its 64 rows with
// v_mfma_f32_32x32x16_bf16 (keys on the MFMA rows, so the max-pool over the
// block's 128 keys is an in-lane reduction plus one lane-half exchange), and
// feeds the pooled score straight into a per-lane descending top-16 list kept
// in registers.  S and M are never written to memory.  When a tile's block
// range is split over several workgroups, each writes its sorted partial list
// and a merge kernel combines them (the pages' two-stage merge, §4.4.2).
//
// Decode: a paged scan writes M for every page of each sequence (HBM-bound,
// one query per group, 16x16x32 MFMA with the groups as rows), then one
// workgroup per (sequence, group) selects the top-k with a threshold filter
// and rank counting (no sort).
#include "msa_common.hpp"
#include "msa_internal.hpp"
#include "msa_profile.hpp"

#include <cstdlib>
#include <type_traits>

namespace msa {

constexpr int kKiThreads = 256;
constexpr int kKiRowsPerTile = 256;

// --------------------------------------------------------------- planning
KiPlan ki_prefill_plan(int32_t n_q, int32_t h_kv, int32_t q_start, int32_t need_diag) {
  KiPlan p{};
  p.n_rows = n_q * h_kv;
  p.n_tiles = (p.n_rows + kKiRowsPerTile - 1) / kKiRowsPerTile;
  if (p.n_tiles == 0) {
    p.chunk_blocks = 1;
    p.n_chunks = 1;
    p.grid_chunks = 1;
    return p;
  }
  // blocks that need scoring in the last (longest) tile, and in total
  auto hi_of = [&](int64_t t) -> int64_t {
    int64_t last = std::min<int64_t>(t * kKiRowsPerTile + kKiRowsPerTile - 1, p.n_rows - 1);
    return ((q_start + last / h_kv) >> 7) + (need_diag ? 1 : 0);
  };
  const int64_t hi_last = hi_of(p.n_tiles - 1);
  const int64_t hi_first = hi_of(0);
  const int64_t work = (hi_first + hi_last) * p.n_tiles / 2 + 1;
  // Blocks per chunk: long enough to amortise a workgroup's set-up and its
  // partial list, short enough for ~`target` workgroups in all.
  const char* env = getenv("MSA_KI_WORK");
  const int64_t target = (env && atoi(env) > 0) ? atoi(env) : 1024;
  int64_t cb = std::max<int64_t>(8, (hi_last + 63) / 64);
  cb = std::max<int64_t>(cb, (work + target - 1) / target);
  int64_t nch = std::max<int64_t>(1, (hi_last + cb - 1) / cb);
  if (nch >= 8) {
    // one chunk per XCD at a time: the tiles of a chunk share its K_idx
    // range in that XCD's L2
    nch = (nch + 7) & ~int64_t(7);
    cb = (hi_last + nch - 1) / nch;
    nch = (hi_last + cb - 1) / cb;
    p.xcd_major = 1;
    p.grid_chunks = static_cast<int32_t>((nch + 7) & ~int64_t(7));
  } else {
    p.xcd_major = 0;
    p.grid_chunks = static_cast<int32_t>(nch);
  }
  p.chunk_blocks = static_cast<int32_t>(cb);
  p.n_chunks = static_cast<int32_t>(nch);
  return p;
}

// ----------------------------------------------------------- prefill kernel
// POOL: 0 block max-pool (the method), 1 block mean-pool.
template <typename T, int DIDX, typename TC, int POOL>
__global__ __launch_bounds__(kKiThreads, 3) void ki_prefill_kernel(KiPrefillArgs a) {
  constexpr int KS = DIDX / 16;                       // 16-wide contraction steps
  constexpr int ROW_BYTES = DIDX * (int)sizeof(T);
  constexpr int LDS_STRIDE = ROW_BYTES + 16;          // padded row, bytes
  constexpr int CHUNKS_PER_ROW = ROW_BYTES / 16;
  constexpr int LOADS = 128 * CHUNKS_PER_ROW / kKiThreads;
  static_assert(LOADS >= 1 && (128 * CHUNKS_PER_ROW) % kKiThreads == 0, "staging split");
  __shared__ __attribute__((aligned(16))) char lds[2][128 * LDS_STRIDE];

  // Workgroups run chunk-major, so the tiles scoring one K_idx range run
  // together; with xcd_major, chunk c's workgroups all land on XCD c % 8.
  int chunk, tile_i;
  if (a.xcd_major) {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    chunk = x + 8 * (k / a.n_tiles);
    tile_i = k % a.n_tiles;
  } else {
    chunk = blockIdx.x / a.n_tiles;
    tile_i = blockIdx.x % a.n_tiles;
  }
  const int tile = a.n_tiles - 1 - tile_i;  // longest tiles first
  const int row0 = tile * kKiRowsPerTile;
  const int row_last = min(row0 + kKiRowsPerTile - 1, a.n_rows - 1);
  const int min_diag = (a.q_start + row0 / a.h_kv) >> 7;
  const int max_diag = (a.q_start + row_last / a.h_kv) >> 7;
  const int hi = max_diag + (a.need_diag ? 1 : 0);
  const int nch = max(1, (hi + a.chunk_blocks - 1) / a.chunk_blocks);
  if (chunk >= nch) return;
  const int b_begin = chunk * a.chunk_blocks;
  const int b_end = min(b_begin + a.chunk_blocks, hi);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const T* __restrict__ q_idx = static_cast<const T*>(a.q_idx);
  const TC* __restrict__ k_idx = static_cast<const TC*>(a.k_idx);

  const int my_row = row0 + wave * 64 + lane;  // row whose list this lane owns
  const bool my_valid = my_row < a.n_rows;
  const int my_diag = (a.q_start + (my_valid ? my_row : row_last) / a.h_kv) >> 7;

  // S^T columns of this lane: rows wave*64 + rt*32 + l32
  int col_pos[2];
  Frag<T> qf[2][KS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = row0 + wave * 64 + rt * 32 + l32;
    const bool ok = r < a.n_rows;
    col_pos[rt] = ok ? a.q_start + r / a.h_kv : -1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[rt][ks] = ok ? load_frag<T>(q_idx + (size_t)r * DIDX + ks * 16 + half * 8) : zero_frag<T>();
  }

  uint64_t keys[kMaxTopK];
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) keys[s] = 0ull;
  float diag_score = -__builtin_inff();

  // K_idx blocks are staged global -> registers -> LDS two blocks ahead.
  // Thread i of the workgroup copies 16-byte pieces at fixed offsets of a
  // block; only the partial last block of a contiguous cache clamps its rows
  // (those keys lie after every query, so the causal mask drops them).
  // With e4m3 caches each 16-byte (8-element) LDS chunk arrives as 8 bytes
  // and is widened to bf16 when stored.
  typedef typename std::conditional<sizeof(TC) == 1 && sizeof(T) == 2, u32x2, u32x4>::type Chunk;
  constexpr int G_ROW = DIDX * (int)sizeof(TC);                   // cache bytes per key row
  constexpr int G_CHUNK = 16 * (int)sizeof(TC) / (int)sizeof(T);  // cache bytes per LDS chunk
  uint32_t toff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int u = tid + kKiThreads * i;
    toff[i] = (uint32_t)((u / CHUNKS_PER_ROW) * G_ROW + (u % CHUNKS_PER_ROW) * G_CHUNK);
  }
  Chunk pre0[LOADS], pre1[LOADS];
  auto load_block = [&](Chunk (&dst)[LOADS], int b) {
    const int64_t base_tok = a.page_table ? (int64_t)scalar_load(a.page_table, b) * kBlock : (int64_t)b * kBlock;
    const char* base = reinterpret_cast<const char*>(k_idx + base_tok * DIDX);
    if (a.page_table || (int64_t)b * kBlock + kBlock <= a.n_kv) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) dst[i] = *reinterpret_cast<const Chunk*>(base + toff[i]);
    } else {
      const uint32_t last = (uint32_t)(a.n_kv - 1 - b * kBlock);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint32_t row = min(toff[i] / G_ROW, last);
        dst[i] = *reinterpret_cast<const Chunk*>(base + row * G_ROW + toff[i] % G_ROW);
      }
    }
  };
  auto store_block = [&](const Chunk (&src)[LOADS], int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int u = tid + kKiThreads * i;
      const int j = u / CHUNKS_PER_ROW, c = u % CHUNKS_PER_ROW;
      u32x4 w;
      if constexpr (sizeof(Chunk) == 8) {
        w = __builtin_bit_cast(u32x4, fp8x8_to_bf16(src[i]));
      } else {
        w = src[i];
      }
      *reinterpret_cast<u32x4*>(&lds[buf][j * LDS_STRIDE + c * 16]) = w;
    }
  };

  if (b_begin < b_end) {
    load_block(pre0, b_begin);
    store_block(pre0, 0);
  }
  if (b_begin + 1 < b_end) load_block(pre0, b_begin + 1);
  __syncthreads();
  // one block: `cur` holds block b + 1, `nxt` receives block b + 2
  auto block_step = [&](int b, Chunk (&cur)[LOADS], Chunk (&nxt)[LOADS]) {
    const int buf = (b - b_begin) & 1;
    if (b + 2 < b_end) load_block(nxt, b + 2);
    const char* K = lds[buf];
    const bool masked = b >= min_diag;
    constexpr float kDrop = POOL == 0 ? -__builtin_inff() : 0.0f;  // a masked key's contribution
    float m0 = kDrop, m1 = kDrop;
    // not unrolled: an unrolled nest keeps every tile's addresses and mask
    // constants live and halves the occupancy
#pragma unroll 1
    for (int kt = 0; kt < 4; ++kt) {
      f32x16 acc0 = {}, acc1 = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const Frag<T> af = *reinterpret_cast<const Frag<T>*>(
            K + (kt * 32 + l32) * LDS_STRIDE + (ks * 16 + half * 8) * (int)sizeof(T));
        mma32(acc0, af, qf[0][ks]);
        mma32(acc1, af, qf[1][ks]);
      }
      if (masked) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = b * kBlock + kt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          if (key > col_pos[0]) acc0[v] = kDrop;
          if (key > col_pos[1]) acc1[v] = kDrop;
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if constexpr (POOL == 0) {
          m0 = fmaxf(m0, acc0[v]);
          m1 = fmaxf(m1, acc1[v]);
        } else {
          m0 += acc0[v];
          m1 += acc1[v];
        }
      }
    }
    // lanes l and l+32 hold the two key halves of rows l and 32+l: swap so
    // that lane L ends with the whole-block max of wave row L
    const float send = half ? m0 : m1;
    const float recv = __shfl_xor(send, 32, 64);
    float pooled;
    if constexpr (POOL == 0) {
      pooled = fmaxf(half ? m1 : m0, recv) * a.idx_scale;
    } else {  // mean over the keys of block b visible from this lane's row
      const int cnt = min(kBlock, a.q_start + (my_valid ? my_row : row_last) / a.h_kv - b * kBlock + 1);
      pooled = cnt > 0 ? ((half ? m1 : m0) + recv) * a.idx_scale / (float)cnt : -__builtin_inff();
    }
    if (my_valid) {
      const bool cand = a.force_local ? (b < my_diag) : (b <= my_diag);
      if (cand) {
        const uint64_t k = make_key(pooled, b);
        if (k > keys[kMaxTopK - 1]) list_insert(keys, k);
      }
      if (b == my_diag) diag_score = pooled;
    }
    if (b + 1 < b_end) store_block(cur, buf ^ 1);
    __syncthreads();
  };
  // unrolled by two so the register stages swap roles without copies
  for (int b = b_begin; b < b_end; b += 2) {
    block_step(b, pre0, pre1);
    if (b + 1 < b_end) block_step(b + 1, pre1, pre0);
  }

  if (!my_valid) return;
  if (a.n_chunks == 1) {
    const int n_take = a.top_k - (a.force_local ? 1 : 0);
    write_row_list(keys, n_take, a.force_local ? my_diag : -1, diag_score, a.top_k,
                   a.block_idx + (size_t)my_row * a.top_k,
                   a.block_score ? a.block_score + (size_t)my_row * a.top_k : nullptr);
  } else {
    uint64_t* dst = a.part_keys + ((size_t)my_row * a.n_chunks + chunk) * kMaxTopK;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) dst[s] = keys[s];
    if (a.need_diag && my_diag >= b_begin && my_diag < b_end) a.part_diag[my_row] = diag_score;
  }
}

// Second stage of the split: merge the sorted partial lists of each row.
__global__ __launch_bounds__(256) void ki_merge_kernel(KiPrefillArgs a) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= a.n_rows) return;
  const int tile = row / kKiRowsPerTile;
  const int row_last = min(tile * kKiRowsPerTile + kKiRowsPerTile - 1, a.n_rows - 1);
  const int max_diag = (a.q_start + row_last / a.h_kv) >> 7;
  const int hi = max_diag + (a.need_diag ? 1 : 0);
  const int nch = max(1, (hi + a.chunk_blocks - 1) / a.chunk_blocks);
  const int my_diag = (a.q_start + row / a.h_kv) >> 7;
  uint64_t keys[kMaxTopK];
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) keys[s] = 0ull;
  // A chunk's list (128 bytes) is read with 8 independent 16-byte loads, and
  // the next chunk's while the current one is inserted (the load is issued
  // unconditionally, the last chunk again at the end, so that the compiler's
  // wait before the inserts covers the current chunk only).
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
  const u64x2* src = reinterpret_cast<const u64x2*>(a.part_keys + (size_t)row * a.n_chunks * kMaxTopK);
  u64x2 cur[kMaxTopK / 2], nxt[kMaxTopK / 2];
#pragma unroll
  for (int q = 0; q < kMaxTopK / 2; ++q) cur[q] = src[q];
  for (int c = 0; c < nch; ++c) {
    const int cn = min(c + 1, nch - 1);
#pragma unroll
    for (int q = 0; q < kMaxTopK / 2; ++q) nxt[q] = src[cn * (kMaxTopK / 2) + q];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
      const uint64_t k = cur[s >> 1][s & 1];
      if (k <= keys[kMaxTopK - 1]) break;  // lists are descending
      list_insert(keys, k);
    }
#pragma unroll
    for (int q = 0; q < kMaxTopK / 2; ++q) cur[q] = nxt[q];
  }
  const float dscore = (a.need_diag && a.force_local) ? a.part_diag[row] : -__builtin_inff();
  const int n_take = a.top_k - (a.force_local ? 1 : 0);
  write_row_list(keys, n_take, a.force_local ? my_diag : -1, dscore, a.top_k,
                 a.block_idx + (size_t)row * a.top_k,
                 a.block_score ? a.block_score + (size_t)row * a.top_k : nullptr);
}

// ------------------------------------------------------------ decode kernels
// One 128-key page of index keys as 16x16x32 B fragments: kt-th 16-key
// slice, keys on the MFMA columns.
// Contraction-index map: for 16-bit caches lane group q4 holds dims
// ks*32 + 8*q4 + e of step ks; for e4m3 caches it holds the contiguous run
// q4*(DIDX/4) + 8*ks + e, so one 16-byte load covers two steps and a load
// instruction reads whole 64-byte rows.  (The query fragments use the same map.)
template <typename TC, int DIDX>
__device__ __forceinline__ int ki_dim(int q4, int ks) {
  return sizeof(TC) == 1 ? q4 * (DIDX / 4) + 8 * ks : ks * 32 + 8 * q4;
}

template <typename TC, int DIDX>
__device__ __forceinline__ void ki_load_page(Raw<TC> (&f)[8][DIDX / 32], const TC* kp) {
  const int lane = threadIdx.x & 63, q4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    if constexpr (sizeof(TC) == 1 && DIDX >= 64) {
#pragma unroll
      for (int ks = 0; ks < DIDX / 32; ks += 2) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(kp + (kt * 16 + l16) * DIDX + ki_dim<TC, DIDX>(q4, ks));
        f[kt][ks] = u32x2{w[0], w[1]};
        f[kt][ks + 1] = u32x2{w[2], w[3]};
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < DIDX / 32; ++ks)
        f[kt][ks] = load_raw<TC>(kp + (kt * 16 + l16) * DIDX + ki_dim<TC, DIDX>(q4, ks));
    }
  }
}

// T: dtype of q_idx and of the MFMA; TC: dtype of the cached k_idx (T, or
// e4m3 widened to bf16 after loading).
template <typename T, int DIDX, typename TC, int POOL>
__global__ __launch_bounds__(256) void ki_decode_scan_kernel(KiDecodeArgs a) {
  constexpr int KS = DIDX / 32;
  const int s = blockIdx.y;
  const int L = scalar_load(a.seq_lens, s);
  const int p = L - 1;
  const int nb = (L + kBlock - 1) / kBlock;
  const int hi = (a.need_diag || !a.force_local) ? nb : nb - 1;
  const int pg_begin = blockIdx.x * a.pages_per_wg;
  const int pg_end = min(pg_begin + a.pages_per_wg, hi);
  if (pg_begin >= pg_end) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q4 = lane >> 4, l16 = lane & 15;
  const T* __restrict__ q_idx = static_cast<const T*>(a.q_idx);
  const TC* __restrict__ k_idx = static_cast<const TC*>(a.k_idx);
  Frag<T> qa[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qa[ks] = (l16 < a.h_kv) ? load_frag<T>(q_idx + ((size_t)s * a.h_kv + l16) * DIDX + ki_dim<TC, DIDX>(q4, ks))
                            : zero_frag<T>();
  const int32_t* pt = a.page_table + (size_t)s * a.max_pages;
  // Lane j holds the physical page of this wave's j-th page (at most 64: a
  // workgroup covers at most 256 pages), read with one vector load, so no
  // page's loads wait on a page-table read of their own.
  const int my_pg = pg_begin + wave + 4 * lane;
  const int pid = my_pg < pg_end ? pt[my_pg] : 0;
  // For rows of up to 128 bytes the next page's index keys are loaded while
  // the current page is scored (wider rows would not fit two pages).
  constexpr bool kPipe = sizeof(TC) * DIDX <= 128;
  Raw<TC> cur[8][KS], nxt[8][KS];
  int pg = pg_begin + wave;
  int j = 0;
  if (kPipe && pg < pg_end)
    ki_load_page<TC, DIDX>(cur, k_idx + (size_t)__builtin_amdgcn_readlane(pid, 0) * kBlock * DIDX);
  for (; pg < pg_end; pg += 4, ++j) {
    if (!kPipe) ki_load_page<TC, DIDX>(cur, k_idx + (size_t)__builtin_amdgcn_readlane(pid, j) * kBlock * DIDX);
    if (kPipe && pg + 4 < pg_end)
      ki_load_page<TC, DIDX>(nxt, k_idx + (size_t)__builtin_amdgcn_readlane(pid, j + 1) * kBlock * DIDX);
    constexpr float kDrop = POOL == 0 ? -__builtin_inff() : 0.0f;  // a masked key's contribution
    // keys on the MFMA rows, groups on the columns: acc[v] of lane (q4, l16)
    // is key kt*16 + 4*q4 + v against group l16, so the pool over the page's
    // keys is in-lane plus one exchange across the four lane groups
    float m = kDrop;
    const bool masked = (pg == nb - 1);
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      f32x4 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) mma16(acc, widen<T, TC>(cur[kt][ks]), qa[ks]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool vis = !masked || (pg * kBlock + kt * 16 + 4 * q4 + v <= p);
        if constexpr (POOL == 0) {
          m = fmaxf(m, vis ? acc[v] : kDrop);
        } else {
          m += vis ? acc[v] : kDrop;
        }
      }
    }
    if constexpr (POOL == 0) {
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
    } else {
      m += __shfl_xor(m, 16, 64);
      m += __shfl_xor(m, 32, 64);
    }
    // mean-pool: the page's visible keys (all 128 but on the last page)
    const float inv_cnt = POOL == 0 ? 1.0f : 1.0f / (float)(masked ? p - pg * kBlock + 1 : kBlock);
    if (q4 == 0 && l16 < a.h_kv)
      a.scores[((size_t)s * a.h_kv + l16) * a.max_pages + pg] =
          POOL == 0 ? m * a.idx_scale : m * a.idx_scale * inv_cnt;
    if (kPipe) {
#pragma unroll
      for (int kt = 0; kt < 8; ++kt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) cur[kt][ks] = nxt[kt][ks];
    }
  }
}

constexpr int kSelectMaxSurvivors = 1024;  // 16 threads x up to 64 candidates each

// Top-k of one (sequence, group) row of pooled page scores.  Keys are the
// order-preserving bits of the score with the inverted block id below them,
// so they are unique and "larger" means better (ties to the lower block).
//  1) each thread loads its U candidates (pages tid + 256 u) into registers
//     and takes their maximum; the 16th largest of the 256 maxima, T, is a
//     lower bound of the answer: the 16 threads whose maxima are >= T each
//     hold a key >= T, so the 16 best keys are all >= T.  Every wave finds T
//     on its own with a bitwise search over the maxima (64 steps of a ballot
//     count), so no barrier follows;
//  2) every key >= T survives (only those 16 threads hold any); a thread
//     counts its survivors in registers and reserves their places with one
//     LDS atomic;
//  3) each survivor's rank among the survivors places the best 16 in order.
template <int U>
__global__ __launch_bounds__(256) void ki_decode_select_kernel(KiDecodeArgs a) {
  __shared__ uint64_t tm[256];
  __shared__ uint64_t surv[kSelectMaxSurvivors];
  __shared__ uint64_t top[kMaxTopK];
  __shared__ int count;
  const int s = blockIdx.x / a.h_kv, r = blockIdx.x % a.h_kv;
  const int L = scalar_load(a.seq_lens, s);
  const int diag = (L - 1) / kBlock;
  const int ncand = min(a.force_local ? diag : diag + 1, a.max_pages);
  const float* sc = a.scores + ((size_t)s * a.h_kv + r) * a.max_pages;
  const int tid = threadIdx.x, lane = tid & 63;

  // Candidates past the row's end read a clamped (in-bounds) entry and are
  // dropped by the b < ncand test; with no candidates, entry 0 of the row
  // (max_pages >= 1) is read and dropped.
  float v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = sc[max(min(tid + 256 * u, ncand - 1), 0)];
  uint64_t tmax = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int b = tid + 256 * u;
    const uint64_t k = b < ncand ? make_key(v[u], b) : 0ull;
    tmax = k > tmax ? k : tmax;
  }
  tm[tid] = tmax;
  if (tid == 0) count = 0;
  if (tid < kMaxTopK) top[tid] = 0;
  __syncthreads();
  // T: the largest value with at least 16 maxima >= it, i.e. the 16th
  // largest maximum; 0 when fewer than 16 threads hold a candidate (then
  // every candidate survives).
  uint64_t mx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) mx[j] = tm[lane + 64 * j];
  uint64_t thr = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t cand = thr | (1ull << bit);
    int c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) c += __popcll(__ballot(mx[j] >= cand));
    if (c >= kMaxTopK) thr = cand;
  }
  if (tmax >= thr && tmax != 0) {
    int c = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = tid + 256 * u;
      c += (b < ncand && make_key(v[u], b) >= thr) ? 1 : 0;
    }
    int pos = atomicAdd(&count, c);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = tid + 256 * u;
      const uint64_t k = make_key(v[u], b);
      if (b < ncand && k >= thr) {
        if (pos < kSelectMaxSurvivors) surv[pos] = k;
        ++pos;
      }
    }
  }
  __syncthreads();
  const int n = min(count, kSelectMaxSurvivors);
  for (int i = tid; i < n; i += 256) {
    const uint64_t k = surv[i];
    int rk = 0;
    for (int j = 0; j < n; ++j) rk += surv[j] > k ? 1 : 0;
    if (rk < kMaxTopK) top[rk] = k;
  }
  __syncthreads();
  // Assemble the row on wave 0: lane e < 16 holds the e-th best key (used if
  // e < n_take and non-empty), lane 16 the forced diagonal block; a valid
  // entry's rank by block id is its output slot, and the slots past the
  // valid entries get the -1 / -inf padding.
  if (tid < 64) {
    const int n_take = a.top_k - (a.force_local ? 1 : 0);
    int id = 0x7fffffff;
    float scv = 0.0f;
    if (tid < kMaxTopK) {
      const uint64_t k = top[tid];
      if (tid < n_take && k != 0ull) {
        id = key_block(k);
        scv = key_score(k);
      }
    } else if (tid == kMaxTopK && a.force_local) {
      id = diag;
      scv = a.need_diag ? sc[diag] : -__builtin_inff();
    }
    int rk = 0;
#pragma unroll
    for (int j = 0; j <= kMaxTopK; ++j) rk += __shfl(id, j, 64) < id ? 1 : 0;
    const bool valid = id != 0x7fffffff;
    const int n_valid = __popcll(__ballot(valid));
    const size_t row = (size_t)s * a.h_kv + r;
    int32_t* idx_out = a.block_idx + row * a.top_k;
    float* sc_out = a.block_score ? a.block_score + row * a.top_k : nullptr;
    if (valid) {
      idx_out[rk] = id;
      if (sc_out) sc_out[rk] = scv;
    }
    if (tid >= n_valid && tid < a.top_k) {
      idx_out[tid] = -1;
      if (sc_out) sc_out[tid] = -__builtin_inff();
    }
  }
}

// ----------------------------------------------------------------- launch
template <typename T, int DIDX, typename TC = T>
static hipError_t ki_prefill_typed(const KiPrefillArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.grid_chunks * a.n_tiles));
  const int pi = profile_begin(PK_KI_PREFILL, st);
  if (a.pool == 1)
    hipLaunchKernelGGL((ki_prefill_kernel<T, DIDX, TC, 1>), grid, dim3(kKiThreads), 0, st, a);
  else
    hipLaunchKernelGGL((ki_prefill_kernel<T, DIDX, TC, 0>), grid, dim3(kKiThreads), 0, st, a);
  profile_end(pi, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_chunks == 1) return e;
  hipLaunchKernelGGL(ki_merge_kernel, dim3((a.n_rows + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, int DIDX, typename TC = T>
static hipError_t ki_decode_typed(const KiDecodeArgs& a, hipStream_t st) {
  dim3 grid((a.max_pages + a.pages_per_wg - 1) / a.pages_per_wg, a.batch);
  const int ps = profile_begin(PK_KI_DECODE_SCAN, st);
  if (a.pool == 1)
    hipLaunchKernelGGL((ki_decode_scan_kernel<T, DIDX, TC, 1>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((ki_decode_scan_kernel<T, DIDX, TC, 0>), grid, dim3(256), 0, st, a);
  profile_end(ps, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 sg((unsigned)(a.batch * a.h_kv));
  const int per = (a.max_pages + 255) / 256;  // candidates per thread
  if (per <= 4) hipLaunchKernelGGL(ki_decode_select_kernel<4>, sg, dim3(256), 0, st, a);
  else if (per <= 8) hipLaunchKernelGGL(ki_decode_select_kernel<8>, sg, dim3(256), 0, st, a);
  else if (per <= 16) hipLaunchKernelGGL(ki_decode_select_kernel<16>, sg, dim3(256), 0, st, a);
  else if (per <= 32) hipLaunchKernelGGL(ki_decode_select_kernel<32>, sg, dim3(256), 0, st, a);
  else if (per <= 40) hipLaunchKernelGGL(ki_decode_select_kernel<40>, sg, dim3(256), 0, st, a);
  else if (per <= 48) hipLaunchKernelGGL(ki_decode_select_kernel<48>, sg, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(ki_decode_select_kernel<64>, sg, dim3(256), 0, st, a);
  return hipGetLastError();
}

bool ki_supported(int dtype, int d_idx) {
  return (dtype == 0 || dtype == 1) && (d_idx == 32 || d_idx == 64 || d_idx == 128);
}

#define MSA_KI_DISPATCH(FN, ...)                                         \
  do {                                                                  \
    if (dtype == 0) {                                                   \
      if (d_idx == 32) return FN<bf16_t, 32>(__VA_ARGS__);              \
      if (d_idx == 64) return FN<bf16_t, 64>(__VA_ARGS__);              \
      if (d_idx == 128) return FN<bf16_t, 128>(__VA_ARGS__);            \
    } else {                                                            \
      if (d_idx == 32) return FN<float, 32>(__VA_ARGS__);               \
      if (d_idx == 64) return FN<float, 64>(__VA_ARGS__);               \
      if (d_idx == 128) return FN<float, 128>(__VA_ARGS__);             \
    }                                                                   \
    return hipErrorInvalidValue;                                        \
  } while (0)

hipError_t launch_ki_prefill(int dtype, int d_idx, const KiPrefillArgs& a, hipStream_t st) {
  if (dtype == 2) {  // bf16 queries, e4m3 cached index keys
    if (d_idx == 32) return ki_prefill_typed<bf16_t, 32, fp8_t>(a, st);
    if (d_idx == 64) return ki_prefill_typed<bf16_t, 64, fp8_t>(a, st);
    if (d_idx == 128) return ki_prefill_typed<bf16_t, 128, fp8_t>(a, st);
    return hipErrorInvalidValue;
  }
  MSA_KI_DISPATCH(ki_prefill_typed, a, st);
}
hipError_t launch_ki_decode(int dtype, int d_idx, const KiDecodeArgs& a, hipStream_t st) {
  if (dtype == 2) {  // bf16 queries, e4m3 cached index keys
    if (d_idx == 32) return ki_decode_typed<bf16_t, 32, fp8_t>(a, st);
    if (d_idx == 64) return ki_decode_typed<bf16_t, 64, fp8_t>(a, st);
    if (d_idx == 128) return ki_decode_typed<bf16_t, 128, fp8_t>(a, st);
    return hipErrorInvalidValue;
  }
  MSA_KI_DISPATCH(ki_decode_typed, a, st);
}

}  // namespace msa
