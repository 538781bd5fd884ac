// msa_kvouter.hpp - device building blocks of the KV-outer kernels (main
// branch forward and backward): K/V block staging, the 32x32 MFMA row tiles,
// and the schedule that inverts block lists into per-(window, group, block)
// token lists ("MiniMax Sparse Attention" digest, titansim.online, §4.4.2).
#pragma once

#include "msa_common.hpp"
#include "msa_internal.hpp"

#include <type_traits>

namespace msa {

// ----------------------------------------------------------------- LDS tile
template <typename T, int D>
struct KvLds {
  static constexpr int KS = D * (int)sizeof(T) + 16;                        // bytes per key row
  static constexpr int VS = 128 * (int)sizeof(T) + (sizeof(T) == 2 ? 8 : 16);  // bytes per d row of V^T
  static constexpr int K_BYTES = 128 * KS;
  static constexpr int BYTES = K_BYTES + D * VS;
};

// Two-phase staging for double buffering: global -> registers (issued before
// the current block's math) and registers -> LDS (after it).  NT threads.
// TC is the cache type; with e4m3 caches (T = bf16) each 16-byte bf16 chunk
// arrives as 8 bytes and is widened when stored to LDS; with MXFP8 caches the
// chunk's E8M0 scale byte (its 8 elements lie in one 32-element block) comes
// with it.
template <typename T, int D, int NT, typename TC = T>
struct StageRegs {
  typedef typename std::conditional<sizeof(TC) == 1, u32x2, u32x4>::type Chunk;
  static constexpr int CB = 16 * (int)sizeof(TC) / (int)sizeof(T);          // cache bytes per 16-B LDS chunk
  static constexpr int CPR = D * (int)sizeof(T) / 16;
  static constexpr int KL = 128 * CPR / NT;                                  // K chunks per thread
  static constexpr int VU = (sizeof(T) == 2 ? 64 * (D / 8) : 128 * (D / 4)) / NT;  // V units per thread
  static constexpr int VW = sizeof(T) == 2 ? 2 : 1;                          // loads per V unit
  static_assert(KL >= 1 && VU >= 1, "staging split");
  Chunk k[KL];
  Chunk v[VU][VW];
  uint32_t ksc[KL];      // MXFP8 only: scale byte of K load i
  uint32_t vsc[VU][VW];  // MXFP8 only: scale byte of V load (u, w)
  uint32_t zero_mask;  // bit i: K load i past the end; bit 16 + 2u + w: V load (u, w)
};


// Base addresses of block b of KV group r: row j of K is k + j * stride.
// MXFP8 caches: row j's scale bytes start at ks + j * sstride (one per 32
// elements; the scale arrays have the cache layouts with d / 32 columns).
struct BlockPtr {
  const char* k;
  const char* v;
  int stride;  // bytes between consecutive key rows
  int valid;   // rows that exist (a contiguous cache may end inside the block)
  const uint8_t* ks;
  const uint8_t* vs;
  int sstride;  // scale bytes between consecutive key rows
};

template <typename T, int D>
__device__ __forceinline__ BlockPtr block_ptr(const void* k, const void* v, const int32_t* pt, int b, int r,
                                              int h_kv, int n_kv, const uint8_t* k_scale = nullptr,
                                              const uint8_t* v_scale = nullptr) {
  BlockPtr p;
  size_t row0;  // element offset of row 0, in units of D
  int rstride;  // rows of D elements between consecutive key rows
  if (pt) {
    row0 = ((size_t)scalar_load(pt, b) * h_kv + r) * kBlock;
    rstride = 1;
    p.valid = kBlock;
  } else {
    row0 = ((size_t)b * kBlock) * h_kv + r;
    rstride = h_kv;
    p.valid = min(kBlock, n_kv - b * kBlock);
  }
  p.stride = rstride * D * (int)sizeof(T);
  p.k = static_cast<const char*>(k) + row0 * D * sizeof(T);
  p.v = static_cast<const char*>(v) + row0 * D * sizeof(T);
  if constexpr (kIsMx<T>) {
    p.sstride = rstride * (D / kMxBlock);
    p.ks = k_scale + row0 * (D / kMxBlock);
    p.vs = v_scale + row0 * (D / kMxBlock);
  } else {
    p.sstride = 0;
    p.ks = p.vs = nullptr;
  }
  return p;
}

template <typename T, int D, int NT, typename TC = T>
__device__ __forceinline__ void stage_load(StageRegs<T, D, NT, TC>& g, const BlockPtr& p) {
  // Every load is issued unconditionally (rows past the end of a contiguous
  // cache read the last valid row); the values are zeroed only when stored to
  // LDS, so nothing here waits for the loads to land.
  using S = StageRegs<T, D, NT, TC>;
  typedef typename S::Chunk C;
  static_assert(S::KL <= 16 && S::VU * S::VW <= 16, "zero mask layout");
  const int last = p.valid - 1;
  uint32_t zm = 0;
#pragma unroll
  for (int i = 0; i < S::KL; ++i) {
    const int u = threadIdx.x + NT * i;
    const int j = u / S::CPR, c = u % S::CPR;
    g.k[i] = *reinterpret_cast<const C*>(p.k + (size_t)min(j, last) * p.stride + c * S::CB);
    if constexpr (kIsMx<TC>) g.ksc[i] = p.ks[min(j, last) * p.sstride + (c * 8) / kMxBlock];
    zm |= (j > last ? 1u : 0u) << i;
  }
  if constexpr (sizeof(T) == 2) {
    constexpr int DC = D / 8;
#pragma unroll
    for (int i = 0; i < S::VU; ++i) {
      const int u = threadIdx.x + NT * i;
      const int kp = (u & 15) + 16 * (u / (16 * DC));
      const int dc = (u >> 4) % DC;
      g.v[i][0] = *reinterpret_cast<const C*>(p.v + (size_t)min(2 * kp, last) * p.stride + dc * S::CB);
      g.v[i][1] = *reinterpret_cast<const C*>(p.v + (size_t)min(2 * kp + 1, last) * p.stride + dc * S::CB);
      if constexpr (kIsMx<TC>) {
        g.vsc[i][0] = p.vs[min(2 * kp, last) * p.sstride + (dc * 8) / kMxBlock];
        g.vsc[i][1] = p.vs[min(2 * kp + 1, last) * p.sstride + (dc * 8) / kMxBlock];
      }
      zm |= (2 * kp > last ? 1u : 0u) << (16 + 2 * i);
      zm |= (2 * kp + 1 > last ? 1u : 0u) << (17 + 2 * i);
    }
  } else {
    constexpr int DC = D / 4;
#pragma unroll
    for (int i = 0; i < S::VU; ++i) {
      const int u = threadIdx.x + NT * i;
      const int key = (u & 31) + 32 * (u / (32 * DC));
      const int dc = (u >> 5) % DC;
      g.v[i][0] = *reinterpret_cast<const C*>(p.v + (size_t)min(key, last) * p.stride + dc * S::CB);
      zm |= (key > last ? 1u : 0u) << (16 + 2 * i);
    }
  }
  g.zero_mask = zm;
}

template <typename T, typename TC, typename C>
__device__ __forceinline__ u32x4 stage_widen(const C& c, uint32_t scale_byte) {
  if constexpr (kIsMx<TC>) {
    return __builtin_bit_cast(u32x4, fp8x8_to_bf16(c, e8m0_scale(scale_byte)));
  } else if constexpr (sizeof(C) == 8) {
    return __builtin_bit_cast(u32x4, fp8x8_to_bf16(c));
  } else {
    return c;
  }
}

template <typename T, int D, int NT, typename TC = T>
__device__ __forceinline__ void stage_store(const StageRegs<T, D, NT, TC>& g, char* lds) {
  using S = StageRegs<T, D, NT, TC>;
  using L = KvLds<T, D>;
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < S::KL; ++i) {
    const int u = threadIdx.x + NT * i;
    const int j = u / S::CPR, c = u % S::CPR;
    *reinterpret_cast<u32x4*>(lds + j * L::KS + c * 16) =
        ((g.zero_mask >> i) & 1u) ? z : stage_widen<T, TC>(g.k[i], kIsMx<TC> ? g.ksc[i] : 0u);
  }
  char* vt = lds + L::K_BYTES;
  if constexpr (sizeof(T) == 2) {
    constexpr int DC = D / 8;
#pragma unroll
    for (int i = 0; i < S::VU; ++i) {
      const int u = threadIdx.x + NT * i;
      const int kp = (u & 15) + 16 * (u / (16 * DC));
      const int dc = (u >> 4) % DC;
      const u32x4 x =
          ((g.zero_mask >> (16 + 2 * i)) & 1u) ? z : stage_widen<T, TC>(g.v[i][0], kIsMx<TC> ? g.vsc[i][0] : 0u);
      const u32x4 y =
          ((g.zero_mask >> (17 + 2 * i)) & 1u) ? z : stage_widen<T, TC>(g.v[i][1], kIsMx<TC> ? g.vsc[i][1] : 0u);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t lo = (x[t] & 0xffffu) | (y[t] << 16);
        const uint32_t hi = (x[t] >> 16) | (y[t] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(vt + (8 * dc + 2 * t) * L::VS + kp * 4) = lo;
        *reinterpret_cast<uint32_t*>(vt + (8 * dc + 2 * t + 1) * L::VS + kp * 4) = hi;
      }
    }
  } else {
    constexpr int DC = D / 4;
#pragma unroll
    for (int i = 0; i < S::VU; ++i) {
      const int u = threadIdx.x + NT * i;
      const int key = (u & 31) + 32 * (u / (32 * DC));
      const int dc = (u >> 5) % DC;
      const u32x4 x = ((g.zero_mask >> (16 + 2 * i)) & 1u) ? z : stage_widen<T, TC>(g.v[i][0], 0u);
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(vt + (4 * dc + e) * L::VS + key * 4) = x[e];
    }
  }
}

// A fragment of V^T: row d, elements 0..3 = keys ka..ka+3, 4..7 = keys kb..kb+3.
template <typename T>
__device__ __forceinline__ Frag<T> vt_frag(const char* vt, int vs, int d, int ka, int kb) {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(vt + d * vs + ka * 2);
    const bf16x4 y = *reinterpret_cast<const bf16x4*>(vt + d * vs + kb * 2);
    f = bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  } else {
    const f32x4 x = *reinterpret_cast<const f32x4*>(vt + d * vs + ka * 4);
    const f32x4 y = *reinterpret_cast<const f32x4*>(vt + d * vs + kb * 4);
    f = f32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
  return f;
}

template <typename T>
__device__ __forceinline__ Frag<T> to_frag(float a0, float a1, float a2, float a3, float a4, float a5,
                                           float a6, float a7) {
  Frag<T> f;
  f[0] = from_f32<T>(a0); f[1] = from_f32<T>(a1); f[2] = from_f32<T>(a2); f[3] = from_f32<T>(a3);
  f[4] = from_f32<T>(a4); f[5] = from_f32<T>(a5); f[6] = from_f32<T>(a6); f[7] = from_f32<T>(a7);
  return f;
}

// Store 4 consecutive values (d .. d+3) of one output row.
template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x4*>(dst) = bf16x4{from_f32<T>(a), from_f32<T>(b), from_f32<T>(c), from_f32<T>(d)};
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
  }
}

// Store 8 consecutive values (one 16-byte store for bf16, two for fp32).
// NT: a non-temporal (streaming) store, for data that is not read again
// before it would have left the caches anyway.
template <typename T, bool NT = false>
__device__ __forceinline__ void store8(T* dst, const f32x16& o, int base) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 v{from_f32<T>(o[base]), from_f32<T>(o[base + 1]), from_f32<T>(o[base + 2]), from_f32<T>(o[base + 3]),
                   from_f32<T>(o[base + 4]), from_f32<T>(o[base + 5]), from_f32<T>(o[base + 6]),
                   from_f32<T>(o[base + 7])};
    if constexpr (NT)
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(dst));
    else
      *reinterpret_cast<bf16x8*>(dst) = v;
  } else {
    const f32x4 lo{o[base], o[base + 1], o[base + 2], o[base + 3]};
    const f32x4 hi{o[base + 4], o[base + 5], o[base + 6], o[base + 7]};
    if constexpr (NT) {
      __builtin_nontemporal_store(lo, reinterpret_cast<f32x4*>(dst));
      __builtin_nontemporal_store(hi, reinterpret_cast<f32x4*>(dst + 4));
    } else {
      *reinterpret_cast<f32x4*>(dst) = lo;
      *reinterpret_cast<f32x4*>(dst + 4) = hi;
    }
  }
}

// ------------------------------------------------------------ row tile math
// One wave processes RT tiles of 32 (token, head) rows against the staged
// block.  S^T = K . Q^T puts keys on the MFMA rows: lane l holds 16 keys of
// row (l % 32) per 32-key tile, so softmax reductions are in-lane plus one
// exchange between lanes l and l+32.
template <typename T, int D, int RT>
struct TileRegs {
  Frag<T> qf[RT][D / 16];
  f32x16 s[RT][4];
  Frag<T> pf[RT][4][2];   // P^T fragments (keys kt*32 + 16*h2 + ...)
  f32x16 o[RT][D / 32];
  int pos[RT];
};

template <typename T, int D, int RT>
__device__ __forceinline__ Frag<T> k_frag(const char* lds, int step) {
  using L = KvLds<T, D>;
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int kt = step / (D / 16), ks = step % (D / 16);
  return *reinterpret_cast<const Frag<T>*>(lds + (kt * 32 + l32) * L::KS + (ks * 16 + half * 8) * (int)sizeof(T));
}

// S^T = K . Q^T for the staged block; fragments are read two steps ahead.
template <typename T, int D, int RT>
__device__ __forceinline__ void tile_scores(TileRegs<T, D, RT>& t, const char* lds, int b, bool mask) {
  constexpr int KS = D / 16, NS = 4 * KS;
  const int lane = threadIdx.x & 63, half = lane >> 5;
  Frag<T> f0 = k_frag<T, D, RT>(lds, 0), f1 = k_frag<T, D, RT>(lds, 1);
#pragma unroll
  for (int step = 0; step < NS; ++step) {
    const int kt = step / KS, ks = step % KS;
    Frag<T> f2;
    if (step + 2 < NS) f2 = k_frag<T, D, RT>(lds, step + 2);
    if (ks == 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) t.s[rt][kt] = f32x16{};
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) mma32(t.s[rt][kt], f0, t.qf[rt][ks]);
    f0 = f1;
    f1 = f2;
    MSA_SCHED_FENCE();
  }
  if (mask) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = b * kBlock + kt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          if (key > t.pos[rt]) t.s[rt][kt][v] = -__builtin_inff();
        }
  }
}

// Pack the exponentiated scores of row tile rt into P^T fragments.
template <typename T, int D, int RT>
__device__ __forceinline__ void tile_pack_p(TileRegs<T, D, RT>& t, int rt) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const f32x16& p = t.s[rt][kt];
      const int o = 8 * h2;
      t.pf[rt][kt][h2] = to_frag<T>(p[o], p[o + 1], p[o + 2], p[o + 3], p[o + 4], p[o + 5], p[o + 6], p[o + 7]);
    }
}

// O^T += V^T . P^T; V^T fragments are read two steps ahead.
template <typename T, int D, int RT>
__device__ __forceinline__ Frag<T> v_frag(const char* lds, int step) {
  using L = KvLds<T, D>;
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int kt = step / (2 * (D / 32)), h2 = (step / (D / 32)) & 1, dt = step % (D / 32);
  const int base = kt * 32 + h2 * 16;
  return vt_frag<T>(lds + L::K_BYTES, L::VS, dt * 32 + l32, base + 4 * half, base + 8 + 4 * half);
}

template <typename T, int D, int RT>
__device__ __forceinline__ void tile_pv(TileRegs<T, D, RT>& t, const char* lds) {
  constexpr int DT = D / 32, NS = 4 * 2 * DT;
  Frag<T> f0 = v_frag<T, D, RT>(lds, 0), f1 = v_frag<T, D, RT>(lds, 1);
#pragma unroll
  for (int step = 0; step < NS; ++step) {
    const int kt = step / (2 * DT), h2 = (step / DT) & 1, dt = step % DT;
    Frag<T> f2;
    if (step + 2 < NS) f2 = v_frag<T, D, RT>(lds, step + 2);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) mma32(t.o[rt][dt], f0, t.pf[rt][kt][h2]);
    f0 = f1;
    f1 = f2;
    MSA_SCHED_FENCE();
  }
}

// ====================================================================
// Prefill schedule: invert block lists into per-(window, group, block)
// token lists.  Slot j of row (i, r) is used iff its block is >= 0, causal
// (<= diag) and larger than the previous used block of the row.
// ====================================================================
struct SchedArgs {
  const int32_t* block_idx;
  int32_t n_q, q_start, h_kv, top_k, n_blocks, window, chunk;
  int64_t n_cells;
  int32_t* count;     // [n_cells]
  int32_t* fill;      // [n_cells]
  int32_t* cell_off;  // [n_cells + 1]
  int32_t* item_off;  // [n_cells + 1]
  int32_t* entries;   // [n_q * h_kv * top_k]
  i32x4* items;       // [max_items] {b, r, e_begin, e_end}
  int32_t* scan;      // [4 * n_scan_tiles]
  int32_t n_scan_tiles;
  uint32_t* bitmap;   // ordered mode: [n_cells, words] token bits of each cell; NULL otherwise
                      // (fill[0] and fill[1] are then zeroed as work-queue heads for the consumers)
  int32_t words;      // 32-bit words per cell (window / 32, rounded up)
  int32_t split;      // LDS count/scatter: workgroups per (window, group), each over a slice of the window's tokens
  int32_t skip_diag;  // leave each row's own (diagonal) block out of the cells: the merge computes it
};

// Cells are the (window, group, block) token lists.  Within a window they are
// numbered XCD-major, and the KV-outer workgroups running on XCD x take
// exactly XCD x's cells.  A group's blocks are spread over S = 8 / h_kv XCDs
// (by b mod S), so each XCD gathers the queries of one group only (they stay
// in its L2 while the window's items run) and reads each KV block of its
// cells from one L2 across windows.  nbp = blocks rounded up to 8.
__device__ __forceinline__ int64_t cell_key(int w, int r, int b, int nbp, int h_kv) {
  const int n_l = h_kv * nbp, per = n_l >> 3;
  int x, pos;
  if (h_kv <= 8 && (8 % h_kv) == 0) {
    const int S = 8 / h_kv;
    x = r * S + b % S;
    pos = b / S;
  } else if ((h_kv & 7) == 0) {
    x = r & 7;
    pos = (r >> 3) * nbp + b;
  } else {  // any other head count: interleave all cells over the XCDs
    const int cl = r * nbp + b;
    x = cl & 7;
    pos = cl >> 3;
  }
  return (int64_t)w * n_l + (int64_t)x * per + pos;
}
__device__ __forceinline__ void cell_rb(int64_t k, int nbp, int h_kv, int& r, int& b) {
  const int n_l = h_kv * nbp, per = n_l >> 3;
  const int kl = (int)(k % n_l);
  const int x = kl / per, pos = kl % per;
  if (h_kv <= 8 && (8 % h_kv) == 0) {
    const int S = 8 / h_kv;
    r = x / S;
    b = pos * S + x % S;
  } else if ((h_kv & 7) == 0) {
    r = (pos / nbp) * 8 + x;
    b = pos % nbp;
  } else {
    const int cl = pos * 8 + x;
    r = cl / nbp;
    b = cl % nbp;
  }
}

// The slots of a block list that count: an entry is used when it is above
// every earlier used entry and not past the row's own block (so duplicates,
// out-of-order entries, -1 padding and future blocks are skipped).  The row is
// read into registers with independent loads (clamped index) before the
// serial vetting, so a thread waits for one load latency, not top_k of them.
__device__ __forceinline__ uint32_t row_used(const int32_t* row, int top_k, int diag, int (&b)[kMaxTopK]) {
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) b[j] = row[min(j, top_k - 1)];
  uint32_t m = 0;
  int prev = -1;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < top_k && b[j] > prev && b[j] <= diag) {
      m |= 1u << j;
      prev = b[j];
    }
  return m;
}
// The slots a schedule places in cells: the used ones, without the row's
// diagonal block when the merge kernel computes that block itself.
__device__ __forceinline__ uint32_t sched_used(const int32_t* row, int top_k, int diag, int skip_diag,
                                               int (&b)[kMaxTopK]) {
  uint32_t m = row_used(row, top_k, diag, b);
  if (skip_diag) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (b[j] == diag) m &= ~(1u << j);
  }
  return m;
}
__device__ __forceinline__ uint32_t used_slots(const int32_t* row, int top_k, int diag) {
  int b[kMaxTopK];
  return row_used(row, top_k, diag, b);
}

constexpr int kScanPerThread = 16;
constexpr int kScanTile = 256 * kScanPerThread;

// Partial layout.  The partial of (token, slot) is a region of G * D values
// stored in the order the MFMA accumulators hold them: 8-value chunks indexed
// ((dt * 2 + p) * 2 + half) * G + head hold d = dt*32 + 16p + 4half + {0..3}
// and the same + 8.  A store instruction then writes, for each token of the
// tile, 2 * G chunks back to back (full cache lines) instead of 64 scattered
// 8-byte pieces.
__device__ __forceinline__ int part_chunk(int dt, int p, int half, int head, int G) {
  return ((dt * 2 + p) * 2 + half) * G + head;
}

// One KV-outer work item: (group r, block b) and a run of the tokens that
// selected b.  The K/V block is staged once in LDS and shared by all rows.
struct KpItem {
  int b, r, e_begin, e_end;
};

// Builds the schedule of plan `pl` for the block lists of `a` in the
// workspace: per-cell token lists (`entries`) and work items.
// With `skip_diag` each row's diagonal block is left out (the forward's merge
// kernel computes it); the backward's schedules keep every used slot.
hipError_t launch_prefill_schedule(const AttnArgs& a, const PrefillPlan& pl, SchedArgs& s, hipStream_t st,
                                   bool skip_diag = false);

// Compute units of the current device.
int num_cus();

}  // namespace msa
