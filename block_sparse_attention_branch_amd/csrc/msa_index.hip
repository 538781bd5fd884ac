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
constexpr int64_t kKiTargetWorkgroups = 1024;

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
  // (a sweep of 256-3072 workgroups at 32K, 128K and 1M found 768-1536 equivalent)
  const int64_t target = kKiTargetWorkgroups;
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
// bf16 index keys go from global memory straight into LDS (no register
// staging), which leaves the registers for a fourth wave per SIMD.
template <typename T, typename TC>
constexpr bool kKiDirect = std::is_same<T, bf16_t>::value && std::is_same<TC, bf16_t>::value;

// POOL: 0 block max-pool (the method), 1 block mean-pool.
template <typename T, int DIDX, typename TC, int POOL>
__global__ __launch_bounds__(kKiThreads, (kKiDirect<T, TC> ? 4 : 3)) void ki_prefill_kernel(KiPrefillArgs a) {
  constexpr int KS = DIDX / 16;                       // 16-wide contraction steps
  constexpr int ROW_BYTES = DIDX * (int)sizeof(T);
  constexpr bool kDirect = kKiDirect<T, TC>;
  // staged rows carry a 16-byte pad; direct copies fill whole rows, so there
  // chunk c of row r sits at chunk c ^ swz(r) instead: either way the rows
  // one ds_read_b128 phase reads start on distinct banks
  constexpr int LDS_STRIDE = kDirect ? ROW_BYTES : ROW_BYTES + 16;
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
  // chunk swizzle: the 16 rows that one ds_read_b128 phase reads (16 lanes,
  // 64 four-byte banks) start on 16 distinct bank quads, and so do any 8
  // consecutive rows against 32 banks
  auto swz = [](uint32_t r) -> uint32_t {
    return ROW_BYTES == 64 ? ((r >> 1) & 3u) ^ ((r >> 3) & 1u) : ROW_BYTES == 128 ? (r & 7u) ^ ((r >> 3) & 1u) : r & 15u;
  };
  const T* __restrict__ q_idx = static_cast<const T*>(a.q_idx);
  const TC* __restrict__ k_idx = static_cast<const TC*>(a.k_idx);

  const int my_row = row0 + wave * 64 + lane;  // row whose list this lane owns
  const bool my_valid = my_row < a.n_rows;
  const int my_diag = (a.q_start + (my_valid ? my_row : row_last) / a.h_kv) >> 7;
  // last block this lane's list may take (the forced diagonal is added at
  // the end); -1 for a lane without a row
  const int my_last = !my_valid ? -1 : (a.force_local ? my_diag - 1 : my_diag);
  // the block whose pooled score is the diagonal's (none for a lane without a row)
  const int my_diag_b = my_valid ? my_diag : -1;

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
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) settle(qf[rt][ks]);

  // The lane's list: pooled scores descending (-inf = empty) with their
  // blocks.  Blocks arrive in increasing order, so a later block must beat a
  // score strictly to pass it, which keeps the lower block first on ties
  // without a tie-break field; 32-bit compares and selects suffice.
  float lsc[kMaxTopK];
  int lid[kMaxTopK];
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    lsc[s] = -__builtin_inff();
    lid[s] = 0;
  }
  float diag_score = -__builtin_inff();
  constexpr int kPending = 3;
  float psc[kPending];
  int pbl[kPending];
#pragma unroll
  for (int p = 0; p < kPending; ++p) {
    psc[p] = -__builtin_inff();
    pbl[p] = 0;
  }
  int n_pend = 0;
  // Inserts the pending candidates (in block order) that still beat the
  // list's last entry (inserting one raises that bound for the next).
  // (slot 0 holds the newest pending candidate, slot n_pend - 1 the oldest)
  auto absorb = [&]() {
#pragma unroll
    for (int p = kPending - 1; p >= 0; --p)
      if (p < n_pend && psc[p] > lsc[kMaxTopK - 1]) list_insert_later(lsc, lid, psc[p], pbl[p]);
    n_pend = 0;
  };

  // 8-bit and fp32 index keys are staged global -> registers -> LDS two
  // blocks ahead (bf16 keys are copied directly, below).
  // Thread i of the workgroup copies 16-byte pieces at fixed offsets of a
  // block; only the partial last block of a contiguous cache clamps its rows
  // (those keys lie after every query, so the causal mask drops them).
  // With e4m3 caches each 16-byte (8-element) LDS chunk arrives as 8 bytes
  // and is widened to bf16 when stored; with MXFP8 caches the chunk's scale
  // byte (its 8 elements lie in one 32-element block) comes with it.
  struct MxChunk {
    u32x2 w;
    uint32_t s;
  };
  typedef typename std::conditional<
      kIsMx<TC>, MxChunk, typename std::conditional<sizeof(TC) == 1 && sizeof(T) == 2, u32x2, u32x4>::type>::type
      Chunk;
  constexpr int G_ROW = DIDX * (int)sizeof(TC);                   // cache bytes per key row
  constexpr int G_CHUNK = 16 * (int)sizeof(TC) / (int)sizeof(T);  // cache bytes per LDS chunk
  // thread tid copies, for i < LOADS, the chunk at row srow = tid / CHUNKS_PER_ROW
  // + i * ROWS_PER_PASS, column tid % CHUNKS_PER_ROW (the same offsets for every block)
  static_assert(kKiThreads % CHUNKS_PER_ROW == 0, "staging rows");
  constexpr int ROWS_PER_PASS = kKiThreads / CHUNKS_PER_ROW;
  const uint32_t srow = tid / CHUNKS_PER_ROW;
  const uint32_t col_off = (tid % CHUNKS_PER_ROW) * G_CHUNK;
  // MXFP8: this thread's chunks all sit in scale column (tid % CHUNKS_PER_ROW) / 4
  const uint32_t scol = (tid % CHUNKS_PER_ROW) * 8 / kMxBlock;
  auto load_chunk = [&](Chunk& dst, const char* base, const uint8_t* sbase, uint32_t row) {
    if constexpr (kIsMx<TC>) {
      dst.w = *reinterpret_cast<const u32x2*>(base + row * G_ROW);
      dst.s = sbase[row * (DIDX / kMxBlock) + scol];
    } else {
      dst = *reinterpret_cast<const Chunk*>(base + row * G_ROW);
    }
  };
  auto load_block = [&](Chunk (&dst)[LOADS], int b) {
    const int64_t base_tok = a.page_table ? (int64_t)scalar_load(a.page_table, b) * kBlock : (int64_t)b * kBlock;
    const char* base = reinterpret_cast<const char*>(k_idx + base_tok * DIDX) + col_off;
    const uint8_t* sbase = kIsMx<TC> ? a.k_idx_scale + base_tok * (DIDX / kMxBlock) : nullptr;
    if (a.page_table || (int64_t)b * kBlock + kBlock <= a.n_kv) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) load_chunk(dst[i], base, sbase, srow + i * ROWS_PER_PASS);
    } else {
      const uint32_t last = (uint32_t)(a.n_kv - 1 - b * kBlock);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) load_chunk(dst[i], base, sbase, min(srow + (uint32_t)(i * ROWS_PER_PASS), last));
    }
  };
  auto store_block = [&](const Chunk (&src)[LOADS], int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int u = tid + kKiThreads * i;
      const int j = u / CHUNKS_PER_ROW, c = u % CHUNKS_PER_ROW;
      u32x4 w;
      if constexpr (kIsMx<TC>) {
        w = __builtin_bit_cast(u32x4, fp8x8_to_bf16(src[i].w, e8m0_scale(src[i].s)));
      } else if constexpr (sizeof(Chunk) == 8) {
        w = __builtin_bit_cast(u32x4, fp8x8_to_bf16(src[i]));
      } else {
        w = src[i];
      }
      *reinterpret_cast<u32x4*>(&lds[buf][j * LDS_STRIDE + c * 16]) = w;
    }
  };

  // Scores block b, staged in LDS buffer `buf`, against this wave's rows,
  // pools the scores and offers the pooled score to the lane's list.
  auto score_block = [&](int b, int buf) {
    const char* K = lds[buf];
    const bool masked = b >= min_diag;
    constexpr float kDrop = POOL == 0 ? -__builtin_inff() : 0.0f;  // a masked key's contribution
    float m0 = kDrop, m1 = kDrop;
    // One 32-key tile: its MFMAs, the causal mask (diagonal blocks only) and
    // the pool into (m0, m1).
    auto tile = [&](int kt, bool mask) __attribute__((always_inline)) {
      f32x16 acc0 = {}, acc1 = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int row = kt * 32 + l32;
        const int col = kDirect ? (int)(((uint32_t)(2 * ks + half) ^ swz(row)) * 16) : (ks * 16 + half * 8) * (int)sizeof(T);
        const Frag<T> af = *reinterpret_cast<const Frag<T>*>(K + row * LDS_STRIDE + col);
        mma32(acc0, af, qf[0][ks]);
        mma32(acc1, af, qf[1][ks]);
      }
      if (mask) {
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
    };
    // The diagonal blocks (masked) run a loop; the others unrolled, so their
    // LDS addresses are immediate offsets of the first tile's.
    if (masked) {
#pragma unroll 1
      for (int kt = 0; kt < 4; ++kt) tile(kt, true);
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) tile(kt, false);
    }
    // lanes l and l+32 hold the two key halves of rows l (m0) and 32+l (m1):
    // swapping the upper half of m0 with the lower half of m1 leaves lane L
    // with both halves of wave row L, one in each result
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m0), __float_as_uint(m1), false, false);
    const float h0 = __uint_as_float(sw[0]), h1 = __uint_as_float(sw[1]);
    float pooled;
    if constexpr (POOL == 0) {
      pooled = fmaxf(h0, h1) * a.idx_scale;
    } else {  // mean over the keys of block b visible from this lane's row
      const int cnt = min(kBlock, a.q_start + (my_valid ? my_row : row_last) / a.h_kv - b * kBlock + 1);
      pooled = cnt > 0 ? (h0 + h1) * a.idx_scale / (float)cnt : -__builtin_inff();
    }
    // A candidate that beats the list's last entry is set aside in this
    // lane's pending slots; the list absorbs them when some lane of the wave
    // has filled its slots (and once at the end).  An insertion costs the
    // whole wave when any lane needs one, and with one insertion per block
    // that would be almost every block.
    {
      const bool want = b <= my_last && pooled > lsc[kMaxTopK - 1];
      // a shift: the new candidate enters slot 0, the others move up one
#pragma unroll
      for (int p = kPending - 1; p > 0; --p) {
        psc[p] = want ? psc[p - 1] : psc[p];
        pbl[p] = want ? pbl[p - 1] : pbl[p];
      }
      psc[0] = want ? pooled : psc[0];
      pbl[0] = want ? b : pbl[0];
      n_pend += want ? 1 : 0;
      if (__any(n_pend == kPending)) absorb();
      if (b == my_diag_b) diag_score = pooled;
    }
  };

  if constexpr (kDirect) {
    // Block b + 1 is copied into the other buffer while block b is scored
    // (global_load_lds: lane i of a copy fills 16 bytes at the copy's LDS
    // base + 16 i; the lane fetches the chunk that the swizzle puts there).
    // Each wave waits for its own copies, the barrier for everyone's.
    // the copy's LDS base goes to M0, so it is computed from uniform values;
    // the global address is a uniform base plus a 32-bit lane offset
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto copy_block = [&](int b, int buf) {
      const int64_t base_tok = a.page_table ? (int64_t)scalar_load(a.page_table, b) * kBlock : (int64_t)b * kBlock;
      const char* base = reinterpret_cast<const char*>(k_idx + base_tok * DIDX);
      const bool full = a.page_table || (int64_t)b * kBlock + kBlock <= a.n_kv;
      const uint32_t last = full ? 127u : (uint32_t)(a.n_kv - 1 - b * kBlock);
      char* dst = &lds[buf][wave_u * LOADS * 1024];
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const uint32_t pos = (uint32_t)((wave_u * LOADS + i) * 1024) + (uint32_t)lane * 16;  // byte in the buffer
        const uint32_t r = pos / ROW_BYTES, c = ((pos % ROW_BYTES) / 16) ^ swz(r);
        const uint32_t off = min(r, last) * ROW_BYTES + c * 16;  // r <= 127: a full block needs no clamp
        __builtin_amdgcn_global_load_lds(base + off, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0,
                                         0);
      }
    };
    if (b_begin < b_end) copy_block(b_begin, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int b = b_begin; b < b_end; ++b) {
      const int buf = (b - b_begin) & 1;
      if (b + 1 < b_end) copy_block(b + 1, buf ^ 1);
      score_block(b, buf);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
    Chunk pre0[LOADS], pre1[LOADS];
    if (b_begin < b_end) {
      load_block(pre0, b_begin);
      store_block(pre0, 0);
    }
    if (b_begin + 1 < b_end) load_block(pre0, b_begin + 1);
    __syncthreads();
    // one block: `cur` holds block b + 1, `nxt` receives block b + 2
    auto block_step = [&](int b, Chunk (&cur)[LOADS], Chunk (&nxt)[LOADS]) {
      const int buf = (b - b_begin) & 1;
      // unconditional (past the end it reloads the last block, an L2 hit), so
      // that the wait before storing `cur` below covers `cur` only and the
      // loads of block b + 2 stay in flight through this block's math
      load_block(nxt, min(b + 2, b_end - 1));
      score_block(b, buf);
      if (b + 1 < b_end) store_block(cur, buf ^ 1);
      __syncthreads();
    };
    // unrolled by two so the register stages swap roles without copies
    for (int b = b_begin; b < b_end; b += 2) {
      block_step(b, pre0, pre1);
      if (b + 1 < b_end) block_step(b + 1, pre1, pre0);
    }
  }
  absorb();

  if (!my_valid) return;
  // the list as 64-bit keys (score, then lower block first; 0 = empty)
  uint64_t keys[kMaxTopK];
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) keys[s] = lsc[s] > -__builtin_inff() ? make_key(lsc[s], lid[s]) : 0ull;
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

// MXFP8 caches: sc[kt] receives the scale byte of key kt*16 + l16 for this
// lane's dims (q4*(DIDX/4) .. +DIDX/4, inside one 32-element block); `sp` is
// the page's scale rows.
template <typename TC, int DIDX>
__device__ __forceinline__ void ki_load_page(Raw<TC> (&f)[8][DIDX / 32], uint32_t (&sc)[8], const TC* kp,
                                             const uint8_t* sp) {
  const int lane = threadIdx.x & 63, q4 = lane >> 4, l16 = lane & 15;
  if constexpr (kIsMx<TC>) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
      sc[kt] = sp[(kt * 16 + l16) * (DIDX / kMxBlock) + (q4 * (DIDX / 4)) / kMxBlock];
  } else {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) sc[kt] = 0u;
  }
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
  static_assert(kKiDecodePagesPerWg % 4 == 0 && kKiDecodePagesPerWg <= 256, "4 waves, one page id per lane");
  const int pg_begin = blockIdx.x * kKiDecodePagesPerWg;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q4 = lane >> 4, l16 = lane & 15;
  const T* __restrict__ q_idx = static_cast<const T*>(a.q_idx);
  const TC* __restrict__ k_idx = static_cast<const TC*>(a.k_idx);
  // The query and the page ids are loaded together with the sequence length
  // (neither depends on it), so a workgroup waits for one round trip before
  // its first page load instead of two.  Lane j holds the physical page of
  // this wave's j-th page (at most 64: a workgroup covers at most 256 pages),
  // read with one vector load clamped into the row; entries past the
  // sequence's last page are never used.
  const int32_t* pt = a.page_table + (size_t)s * a.max_pages;
  int pid = pt[min(pg_begin + wave + 4 * lane, a.max_pages - 1)];
  Frag<T> qa[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qa[ks] = load_frag<T>(q_idx + ((size_t)s * a.h_kv + min(l16, a.h_kv - 1)) * DIDX + ki_dim<TC, DIDX>(q4, ks));
  const int L = scalar_load(a.seq_lens, s);
  const int p = L - 1;
  const int nb = (L + kBlock - 1) / kBlock;
  const int hi = (a.need_diag || !a.force_local) ? nb : nb - 1;
  // a workgroup past the sequence's last page scores nothing below (no early
  // exit: a branch on the length would hold the loads above back behind it)
  const int pg_end = min(pg_begin + kKiDecodePagesPerWg, hi);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    if (l16 >= a.h_kv) qa[ks] = zero_frag<T>();
  settle(pid);  // waited for here, so no later wait on it also covers page loads in flight
  // For rows of up to 128 bytes the next page's index keys are loaded while
  // the current page is scored (wider rows would not fit two pages).
  constexpr bool kPipe = sizeof(TC) * DIDX <= 128;
  Raw<TC> cur[8][KS], nxt[8][KS];
  uint32_t csc[8], nsc[8];  // MXFP8 scale bytes of the two pages
  auto load = [&](Raw<TC>(&f)[8][KS], uint32_t(&sc)[8], int page) {
    const size_t tok = (size_t)page * kBlock;
    ki_load_page<TC, DIDX>(f, sc, k_idx + tok * DIDX,
                           kIsMx<TC> ? a.k_idx_scale + tok * (DIDX / kMxBlock) : nullptr);
  };
  // Scores the page held in f (scale bytes sc): returns the pooled score of
  // group l16 (valid in the lanes with q4 == 0 and l16 < h_kv).
  auto score = [&](const Raw<TC>(&f)[8][KS], const uint32_t(&sc)[8], int pg) -> float {
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
      for (int ks = 0; ks < KS; ++ks) mma16(acc, widen<T, TC>(f[kt][ks], sc[kt]), qa[ks]);
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
    return POOL == 0 ? m * a.idx_scale : m * a.idx_scale * inv_cnt;
  };
  // The wave scores pages pg0, pg0 + 4, ... (at most kPw of them).  The loop
  // is unrolled, so the two register sets take turns without copies, and the
  // next page's loads are unconditional (past the wave's last page they load
  // that page again, an L2 hit), so the wait before a page's math covers
  // that page's loads only.  The scores are stored after the loop: a store
  // inside it made the next write to its data register wait for every load
  // in flight (the counter orders loads and stores alike).
  constexpr int kPw = kKiDecodePagesPerWg / 4;
  const int pg0 = pg_begin + __builtin_amdgcn_readfirstlane(wave);
  const int n_mine = (pg_end - pg0 + 3) / 4;  // uniform; 0 or less: no page
  float res[kPw];
  if constexpr (kPipe) {
    if (n_mine > 0) load(cur, csc, __builtin_amdgcn_readlane(pid, 0));
#pragma unroll
    for (int i = 0; i < kPw; ++i) {
      if (i >= n_mine) break;
      const int nx = min(i + 1, n_mine - 1);
      if (i & 1) {
        load(cur, csc, __builtin_amdgcn_readlane(pid, nx));
        MSA_SCHED_FENCE();  // keep the next page's loads ahead of this page's math
        res[i] = score(nxt, nsc, pg0 + 4 * i);
      } else {
        load(nxt, nsc, __builtin_amdgcn_readlane(pid, nx));
        MSA_SCHED_FENCE();
        res[i] = score(cur, csc, pg0 + 4 * i);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPw; ++i) {
      if (i >= n_mine) break;
      load(cur, csc, __builtin_amdgcn_readlane(pid, i));
      res[i] = score(cur, csc, pg0 + 4 * i);
    }
  }
  if (q4 == 0 && l16 < a.h_kv) {
    float* dst = a.scores + ((size_t)s * a.h_kv + l16) * a.max_pages;
#pragma unroll
    for (int i = 0; i < kPw; ++i)
      if (i < n_mine) dst[pg0 + 4 * i] = res[i];
  }
}

// Writes one (sequence, group) row from `top` (its best keys, descending, 0 =
// empty); run by the 64 lanes of one wave.  Lane e < 16 holds the e-th best
// key (used if e < n_take and non-empty), lane 16 the forced diagonal block;
// a valid entry's rank by block id is its output slot, and the slots past the
// valid entries get the -1 / -inf padding.
__device__ __forceinline__ void select_write_row(const KiDecodeArgs& a, int s, int r, int diag, const float* sc,
                                                 const uint64_t* top) {
  const int tid = threadIdx.x & 63;
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
  for (int j = 0; j <= kMaxTopK; ++j) rk += __builtin_amdgcn_readlane(id, j) < id ? 1 : 0;
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

// Top-k of one (sequence, group) row of pooled page scores, one workgroup of
// NT threads per row, thread t holding the candidates t + NT u, u < U.  Keys
// are the order-preserving bits of the score with the inverted block id below
// them, so they are unique and "larger" means better (ties to the lower block).
//  1) each thread takes the maximum of its keys (0: no candidate).  Every lane
//     counts the maxima of its wave above its own (read from LDS as
//     broadcasts); as the nonzero maxima are unique, the lane that counts
//     j - 1 holds the wave's j-th largest maximum t_w(j), j = 1, 2, 4, 8, 16
//     (0 when fewer than j lanes hold a candidate);
//  2) a lower bound T of the 16th best key: for m = 16 / j, m waves each hold
//     j keys >= their t_w(j), so the m-th largest t_w(j) over the waves is
//     one; T is the largest of these bounds.  T >= max_w t_w(16), so in every
//     wave at most 16 lanes hold a maximum >= T, and at most 16 * NW * U keys
//     are >= T: the LDS buffer holds every survivor;
//  3) each survivor's rank among the survivors places the best 16 in order.
template <int NT, int U>
__global__ __launch_bounds__(NT) void ki_decode_select_kernel(KiDecodeArgs a) {
  constexpr int NW = NT / 64;
  constexpr int kCap = kMaxTopK * NW * U;
  constexpr int kLevels = 5;  // j = 16 >> e
  __shared__ uint64_t tm[NT];
  __shared__ uint64_t wthr[kLevels][NW];
  __shared__ uint64_t surv[kCap];
  __shared__ uint64_t top[kMaxTopK];
  __shared__ uint64_t thr[kLevels];
  __shared__ int count;
  const int s = blockIdx.x / a.h_kv, r = blockIdx.x % a.h_kv;
  const float* sc = a.scores + ((size_t)s * a.h_kv + r) * a.max_pages;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The scores are loaded together with the sequence length (clamped into
  // the row, not to its candidates): candidates past the row's end get key 0
  // whatever was read.  All loads are issued before any is used: settle()
  // keeps the compiler from moving each load under its own branch, one round
  // trip at a time.
  float v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = sc[min(tid + NT * u, a.max_pages - 1)];
  const int L = scalar_load(a.seq_lens, s);
  const int diag = (L - 1) / kBlock;
  const int ncand = min(a.force_local ? diag : diag + 1, a.max_pages);
#pragma unroll
  for (int u = 0; u < U; ++u) settle(v[u]);
  uint64_t k[U];
  uint64_t tmax = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int b = tid + NT * u;
    k[u] = b < ncand ? make_key(v[u], b) : 0ull;
    tmax = k[u] > tmax ? k[u] : tmax;
  }
  tm[tid] = tmax;
  if (tid == 0) count = 0;
  if (tid < kMaxTopK) top[tid] = 0;
  __syncthreads();
  {
    const uint64_t* wm = tm + wave * 64;
    int gt = 0;
#pragma unroll 8
    for (int j = 0; j < 64; j += 2) {
      typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
      const u64x2 p = *reinterpret_cast<const u64x2*>(wm + j);
      gt += (p[0] > tmax ? 1 : 0) + (p[1] > tmax ? 1 : 0);
    }
#pragma unroll
    for (int e = 0; e < kLevels; ++e) {
      const uint64_t hit = __ballot(tmax != 0ull && gt == (16 >> e) - 1);
      const uint64_t t = hit ? readlane_u64(tmax, __builtin_ctzll(hit)) : 0ull;  // hit is wave-uniform
      if (lane == 0) wthr[e][wave] = t;
    }
  }
  __syncthreads();
  // wave e takes level e: lane w < NW holds t_w(j), j = 16 >> e, and the m-th
  // largest over the waves (m = 2^e) is the value with m - 1 larger ones
  // (nonzero values are unique keys); levels with m > NW give no bound
  if (wave < kLevels) {
    const int e = wave, m = 1 << e;
    uint64_t t = 0ull;
    if (m <= NW) {
      const uint64_t x = lane < NW ? wthr[e][lane] : 0ull;
      int g = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) g += wthr[e][w] > x ? 1 : 0;
      const uint64_t hit = __ballot(x != 0ull && g == m - 1);
      t = hit ? readlane_u64(x, __builtin_ctzll(hit)) : 0ull;
    }
    if (lane == 0) thr[e] = t;
  }
  __syncthreads();
  uint64_t T = 0ull;
#pragma unroll
  for (int e = 0; e < kLevels; ++e)
    if ((1 << e) <= NW) T = thr[e] > T ? thr[e] : T;
  if (tmax >= T && tmax != 0) {
    int c = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) c += (k[u] != 0ull && k[u] >= T) ? 1 : 0;
    int pos = atomicAdd(&count, c);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k[u] != 0ull && k[u] >= T) surv[pos++] = k[u];
  }
  __syncthreads();
  const int n = count;
  for (int i = tid; i < n; i += NT) {
    const uint64_t ki = surv[i];
    int rk = 0;
    for (int j = 0; j < n; ++j) rk += surv[j] > ki ? 1 : 0;
    if (rk < kMaxTopK) top[rk] = ki;
  }
  __syncthreads();
  if (tid < 64) select_write_row(a, s, r, diag, sc, top);
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
  dim3 grid((a.max_pages + kKiDecodePagesPerWg - 1) / kKiDecodePagesPerWg, a.batch);
  const int ps = profile_begin(PK_KI_DECODE_SCAN, st);
  if (a.pool == 1)
    hipLaunchKernelGGL((ki_decode_scan_kernel<T, DIDX, TC, 1>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((ki_decode_scan_kernel<T, DIDX, TC, 0>), grid, dim3(256), 0, st, a);
  profile_end(ps, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 sg((unsigned)(a.batch * a.h_kv));
  // 256 threads per row up to 2048 pages (8 candidates each), 1024 beyond
  static_assert(kMaxDecodePages <= 16 * 1024, "the select holds at most 16 candidates per thread");
  const int mp = a.max_pages;
  if (mp <= 256 * 4) hipLaunchKernelGGL((ki_decode_select_kernel<256, 4>), sg, dim3(256), 0, st, a);
  else if (mp <= 256 * 8) hipLaunchKernelGGL((ki_decode_select_kernel<256, 8>), sg, dim3(256), 0, st, a);
  else if (mp <= 1024 * 4) hipLaunchKernelGGL((ki_decode_select_kernel<1024, 4>), sg, dim3(1024), 0, st, a);
  else if (mp <= 1024 * 8) hipLaunchKernelGGL((ki_decode_select_kernel<1024, 8>), sg, dim3(1024), 0, st, a);
  else if (mp <= 1024 * 12) hipLaunchKernelGGL((ki_decode_select_kernel<1024, 12>), sg, dim3(1024), 0, st, a);
  else hipLaunchKernelGGL((ki_decode_select_kernel<1024, 16>), sg, dim3(1024), 0, st, a);
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
  if (dtype == 3) {  // bf16 queries, MXFP8 cached index keys
    if (d_idx == 32) return ki_prefill_typed<bf16_t, 32, mx8_t>(a, st);
    if (d_idx == 64) return ki_prefill_typed<bf16_t, 64, mx8_t>(a, st);
    if (d_idx == 128) return ki_prefill_typed<bf16_t, 128, mx8_t>(a, st);
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
  if (dtype == 3) {  // bf16 queries, MXFP8 cached index keys
    if (d_idx == 32) return ki_decode_typed<bf16_t, 32, mx8_t>(a, st);
    if (d_idx == 64) return ki_decode_typed<bf16_t, 64, mx8_t>(a, st);
    if (d_idx == 128) return ki_decode_typed<bf16_t, 128, mx8_t>(a, st);
    return hipErrorInvalidValue;
  }
  MSA_KI_DISPATCH(ki_decode_typed, a, st);
}

}  // namespace msa
