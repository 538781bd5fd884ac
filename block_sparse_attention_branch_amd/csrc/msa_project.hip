// msa_project.hip - the index-branch projections and RoPE before the index
// scores (the index-query projection per GQA group and the shared index-key
// projection, with the index key appended to the cache in place).  Built
// without the VGPR-form MFMA option of the index kernels, so the long-call
// kernel's accumulators can live in the accumulation registers.
#include <algorithm>

#include "msa_common.hpp"
#include "msa_internal.hpp"

namespace msa {

// ------------------------------------------- index projections and RoPE
// The steps before the index branch ("MiniMax Sparse Attention" digest,
// §4.2: one index-query projection per GQA group, one shared index-key
// projection; §3.1: RoPE on 64 dims).  C^T = W . x^T on 32x32x16 bf16 MFMA
// with the projected features on the MFMA rows and 32 tokens on the lanes, so
// a RoPE pair (i, i + R/2) sits in one lane; angles in double precision (the
// position times the frequency must stay exact for positions up to 2^20 and
// beyond).  The key projection is appended to the index-key cache in place.
// Short calls (a decode step): a workgroup takes 32 tokens, one projection
// and one slice of d_model (blockIdx.z; the whole of it when the call is not
// split); its 8 waves split the slice (16-wide steps dealt round-robin) and
// their sums are added in a fixed tree through LDS.  Unsplit, wave 0 applies
// RoPE and stores; split, it writes the slice's fp32 sums and kx_reduce_kernel
// adds the slices in order, applies RoPE and stores.  Long calls use
// kx_tile_kernel below.
constexpr int kKxWaves = 8;

// cos and sin of the angle pos * f.  The angle is formed in double and
// reduced modulo 2 pi there (Cody and Waite's method, 2 pi split into three
// parts; the first two have 24 significant bits, so k times either is exact
// for |k| < 2^29, i.e. every int32 position); sine and cosine of the reduced
// angle are taken in fp32.
__device__ __forceinline__ void rope_cos_sin(double pos, double f, float& c, float& s) {
  const double th = pos * f;
  const double k = rint(th * 0.15915494309189535);
  double red = fma(-k, 0x1.921fb4p+2, th);
  red = fma(-k, 0x1.4442d0p-22, red);
  red = fma(-k, 0x1.8469898cc5170p-46, red);
  sincosf((float)red, &s, &c);
}

// Destination row of token t's projection hd (d_idx values): hd < h_kv, the
// query projection in q_out; hd == h_kv, the token's row of the index-key
// cache (contiguous at row positions[t] if in [0, n_kv), paged at row
// positions[t] % 128 of page page_table[seq[t], positions[t] / 128] if that
// page index is below max_pages); nullptr if the row is out of range.
template <int DI>
__device__ __forceinline__ bf16_t* kx_dst(const KxArgs& a, int t, int hd) {
  if (hd < a.h_kv) return static_cast<bf16_t*>(a.q_out) + ((size_t)t * a.h_kv + hd) * DI;
  const int p = a.positions[t];
  if (a.page_table) {
    const int sq = a.seq ? a.seq[t] : 0;
    if (p >= 0 && (p >> 7) < a.max_pages)
      return static_cast<bf16_t*>(a.k_cache) +
             ((size_t)a.page_table[(size_t)sq * a.max_pages + (p >> 7)] * kBlock + (p & (kBlock - 1))) * DI;
  } else if (p >= 0 && p < a.n_kv) {
    return static_cast<bf16_t*>(a.k_cache) + (size_t)p * DI;
  }
  return nullptr;
}

// RoPE and store of one 32-token tile of one projection held as the MFMA
// result C^T: lane (half, l32) has token t, acc[ft][v] = feature
// ft*32 + 8*(v/4) + 4*half + (v%4).  hd < h_kv: query projection hd, written
// to q_out; hd == h_kv: the key projection, appended to the index-key cache.
template <int DI>
__device__ __forceinline__ void kx_rope_store(f32x16 (&acc)[DI / 32], int t, bool ok, int hd, const KxArgs& a) {
  const int half = (threadIdx.x & 63) >> 5;
  const int R = a.rope_dim;
  const double pos = (double)a.positions[t];
  const double lb = log2((double)a.rope_base);
  // Frequencies base^(-2i/R) of this lane's pair indices i = 8j + 4*half + u
  // (u < 4) from two exp2 calls: fq[4j + u] = base^(-2(4 half)/R) * r^(8j+u),
  // r = base^(-2/R) (a few roundings, relative error ~1e-15)
  double fq[16];
  {
    const double r1 = exp2(-2.0 / R * lb), r2 = r1 * r1, r3 = r2 * r1, r8 = (r2 * r2) * (r2 * r2);
    double row = exp2(-2.0 * (4 * half) / R * lb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fq[4 * j] = row;
      fq[4 * j + 1] = row * r1;
      fq[4 * j + 2] = row * r2;
      fq[4 * j + 3] = row * r3;
      row *= r8;
    }
  }
  // turns the pair (acc[fa][va], acc[fb][vb]) by the angle pos * f
  auto turn = [&](int fa, int va, int fb, int vb, double f) __attribute__((always_inline)) {
    float c, s_;
    rope_cos_sin(pos, f, c, s_);
    const float x1 = acc[fa][va], x2 = acc[fb][vb];
    acc[fa][va] = x1 * c - x2 * s_;
    acc[fb][vb] = x2 * c + x1 * s_;
  };
  // acc[ft][v] is feature ft*32 + 8*(v/4) + 4*half + (v%4): pair index
  // 8*(v/4) + 4*half + (v%4) (plus 32 for ft = 1 at R = 128)
  if (R == 32) {
#pragma unroll
    for (int v = 0; v < 8; ++v) turn(0, v, 0, v + 8, fq[v]);
  }
  if constexpr (DI >= 64) {
    if (R == 64) {
#pragma unroll
      for (int v = 0; v < 16; ++v) turn(0, v, 1, v, fq[v]);
    }
  }
  if constexpr (DI >= 128) {
    if (R == 128) {
      // pair indices 32 + ...: one more factor r^32 = base^(-64/R)
      const double r32 = exp2(-64.0 / R * lb);
#pragma unroll
      for (int v = 0; v < 16; ++v) turn(0, v, 2, v, fq[v]);
#pragma unroll
      for (int v = 0; v < 16; ++v) turn(1, v, 3, v, fq[v] * r32);
    }
  }
  bf16_t* dst = kx_dst<DI>(a, t, hd);
  if (ok && dst) {
#pragma unroll
    for (int ft = 0; ft < DI / 32; ++ft)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<bf16x4*>(dst + ft * 32 + 8 * c + 4 * half) =
            bf16x4{from_f32<bf16_t>(acc[ft][4 * c]), from_f32<bf16_t>(acc[ft][4 * c + 1]),
                   from_f32<bf16_t>(acc[ft][4 * c + 2]), from_f32<bf16_t>(acc[ft][4 * c + 3])};
  }
}

template <int DI>
__global__ __launch_bounds__(kKxWaves * 64) void kx_project_kernel(KxArgs a) {
  constexpr int FT = DI / 32;
  __shared__ f32x4 red[kKxWaves / 2][FT * 4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int hd = blockIdx.y;  // 0 .. h_kv - 1: query projections; h_kv: the key projection
  const int t_raw = blockIdx.x * 32 + l32;
  const bool ok = t_raw < a.n_tok;
  const int t = min(t_raw, a.n_tok - 1);
  const bf16_t* w = static_cast<const bf16_t*>(hd < a.h_kv ? a.w_q : a.w_k) +
                    (hd < a.h_kv ? (size_t)hd * DI * a.d_model : 0);
  const bf16_t* xr = static_cast<const bf16_t*>(a.x) + (size_t)t * a.d_model + half * 8;
  const int k_lo = blockIdx.z * a.k_per_split, k_hi = min(a.d_model, k_lo + a.k_per_split);
  f32x16 acc[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) acc[ft] = f32x16{};
#pragma unroll 4
  for (int k0 = k_lo + wave * 16; k0 < k_hi; k0 += kKxWaves * 16) {
    const bf16x8 xb = load_frag<bf16_t>(xr + k0);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
      mma32(acc[ft], load_frag<bf16_t>(w + (size_t)(ft * 32 + l32) * a.d_model + k0 + half * 8), xb);
  }
  // tree: the upper half of the live waves hands its sums to the lower half
#pragma unroll
  for (int live = kKxWaves; live > 1; live >>= 1) {
    const int h = live >> 1;
    if (wave >= h && wave < live) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          red[wave - h][ft * 4 + c][lane] =
              f32x4{acc[ft][4 * c], acc[ft][4 * c + 1], acc[ft][4 * c + 2], acc[ft][4 * c + 3]};
    }
    __syncthreads();
    if (wave < h) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 o = red[wave][ft * 4 + c][lane];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[ft][4 * c + q] += o[q];
        }
    }
    __syncthreads();
  }
  if (wave != 0) return;
  if (a.split > 1) {
    // acc[ft][4c .. 4c+3] are features ft*32 + 8c + 4*half + 0..3
    if (ok) {
      float* dst = a.part + (((size_t)blockIdx.z * a.n_tok + t) * (a.h_kv + 1) + hd) * DI;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<f32x4*>(dst + ft * 32 + 8 * c + 4 * half) =
              f32x4{acc[ft][4 * c], acc[ft][4 * c + 1], acc[ft][4 * c + 2], acc[ft][4 * c + 3]};
    }
    return;
  }
  kx_rope_store<DI>(acc, t, ok, hd, a);
}

// Sum of the split slices (in slice order) for one (token, projection): item
// j < R/2 is the RoPE pair (j, j + R/2), turned by the angle of pair j; items
// from R/2 on are the dims past rope_dim, stored as they are.  One thread per
// item, so every partial is read once.
template <int DI>
__global__ __launch_bounds__(256) void kx_reduce_kernel(KxArgs a) {
  const int nproj = a.h_kv + 1;
  const int R = a.rope_dim, H = R / 2, NI = DI - H;  // items per (token, projection)
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.n_tok * nproj * NI) return;
  const int j = (int)(idx % NI);
  const int hd = (int)((idx / NI) % nproj);
  const int t = (int)(idx / ((int64_t)NI * nproj));
  const bool pair = j < H;
  const int f1 = pair ? j : j + H, f2 = pair ? j + H : f1;
  const size_t stride = (size_t)a.n_tok * nproj * DI;
  const float* src = a.part + ((size_t)t * nproj + hd) * DI;
  // slices in groups of 8 independent loads (clamped past the last slice,
  // which then adds zero), summed in slice order
  float x = 0.0f, y = 0.0f;
  for (int z0 = 0; z0 < a.split; z0 += 8) {
    float vx[8], vy[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t o = (size_t)min(z0 + u, a.split - 1) * stride;
      vx[u] = src[o + f1];
      vy[u] = src[o + f2];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      x += z0 + u < a.split ? vx[u] : 0.0f;
      y += z0 + u < a.split ? vy[u] : 0.0f;
    }
  }
  bf16_t* dst = kx_dst<DI>(a, t, hd);
  if (!dst) return;
  if (pair) {
    float c, s;
    rope_cos_sin((double)a.positions[t], exp2(-2.0 * j / R * log2((double)a.rope_base)), c, s);
    dst[f1] = from_f32<bf16_t>(x * c - y * s);
    dst[f2] = from_f32<bf16_t>(y * c + x * s);
  } else {
    dst[f1] = from_f32<bf16_t>(x);
  }
}

// Long calls: a workgroup of 8 waves takes 32*TT tokens (128 at d_idx 32 and
// 64, 32 at d_idx 128) and P <= 5 projections.  Waves 0 .. P-1 compute, one
// projection each; the other waves only stage x.  Per 64-wide chunk of
// d_model the tokens' x rows go through a ring of three LDS buffers (rows
// padded to 144 bytes, so the 32 rows one MFMA operand reads spread over all
// banks), loaded by the staging waves three chunks ahead (the bytes in flight
// per CU must cover HBM latency); the compute waves load their projection's W
// rows straight into MFMA operands, a chunk ahead, and hold the accumulators.
// Splitting the roles keeps the x prefetch out of the compute waves'
// registers.  Both roles pass one barrier per chunk; the chunk count is
// rounded up to a multiple of three, chunks past d_model loading as zeros.
// x is read from HBM once and W from L2 once per workgroup.  The result has
// the layout of the short kernel's (features on the MFMA rows, tokens on the
// lanes) and goes through the same RoPE and store.
constexpr int kKxChunk = 64;
constexpr int kKxSteps = kKxChunk / 16;    // MFMA k-steps per chunk
constexpr int kKxRowPieces = kKxChunk / 8;  // 16-byte pieces per row and chunk
constexpr int kKxRowBytes = kKxChunk * 2 + 16;
constexpr int kKxTileMinTokens = 256;
constexpr int kKxTileWaves = 8;
constexpr int kKxMaxCompute = 5;  // compute waves per workgroup (>= 3 stage)
// 32-token tiles per workgroup: accumulators 16 * TT * d_idx / 32 registers
// per lane, W operands 16 * d_idx / 32
template <int DI>
constexpr int kx_tile_tt() { return DI >= 128 ? 1 : 4; }
// x pieces (16 bytes) per staging thread and chunk, with at least 3 staging waves
template <int DI>
constexpr int kx_tile_npt() { return (kx_tile_tt<DI>() * 32 * kKxRowPieces + 64 * (kKxTileWaves - kKxMaxCompute) - 1) / (64 * (kKxTileWaves - kKxMaxCompute)); }

template <int DI>
__global__ __launch_bounds__(kKxTileWaves * 64) void kx_tile_kernel(KxArgs a, int proj_per_wg) {
  constexpr int FT = DI / 32, TT = kx_tile_tt<DI>(), ROWS = TT * 32, NPT = kx_tile_npt<DI>();
  constexpr int PIECES = ROWS * kKxRowPieces;  // 16-byte pieces of x per chunk
  __shared__ __align__(16) unsigned char xs[3][ROWS * kKxRowBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int tok0 = blockIdx.x * ROWS;
  const int D = a.d_model;
  const int nch3 = ((D + kKxChunk - 1) / kKxChunk + 2) / 3 * 3;

  if (wave >= proj_per_wg) {
    // ---- staging waves: piece p = row * kKxRowPieces + col, 16 bytes at
    // k = c * kKxChunk + 8 col
    const int sid = threadIdx.x - proj_per_wg * 64, nst = (kKxTileWaves - proj_per_wg) * 64;
    const bf16_t* x = static_cast<const bf16_t*>(a.x);
    // d_model is a multiple of 16, so an 8-wide piece is wholly inside or
    // past the end; pieces past the end read an in-bounds piece and are
    // stored as zeros (the choice is made at the store, so no load is waited
    // for early).  Threads past the last piece load it again and store nothing.
    auto x_load = [&](bf16x8(&r)[NPT], int c) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        const int p = min(sid + j * nst, PIECES - 1);
        const int tok = min(tok0 + p / kKxRowPieces, a.n_tok - 1);
        r[j] = load_frag<bf16_t>(x + (size_t)tok * D + min(c * kKxChunk + 8 * (p % kKxRowPieces), D - 8));
      }
    };
    auto x_store = [&](const bf16x8(&r)[NPT], int buf, int c) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        const int p = sid + j * nst;
        const bool in = c * kKxChunk + 8 * (p % kKxRowPieces) < D;
        if (p < PIECES)
          *reinterpret_cast<bf16x8*>(&xs[buf][(p / kKxRowPieces) * kKxRowBytes + (p % kKxRowPieces) * 16]) = in ? r[j] : zero_frag<bf16_t>();
      }
    };
    bf16x8 r0[NPT], r1[NPT], r2[NPT];
    x_load(r0, 0);
    x_load(r1, 1);
    x_load(r2, 2);
    x_store(r0, 0, 0);
    __syncthreads();
    // iteration c: the set that held chunk c (already in its buffer) takes
    // chunk c + 3; chunk c + 1 goes to buffer (c + 1) % 3, last read by the
    // compute waves in iteration c - 2
    for (int c = 0; c < nch3; c += 3) {
      x_load(r0, c + 3);
      x_store(r1, 1, c + 1);
      __syncthreads();
      x_load(r1, c + 4);
      x_store(r2, 2, c + 2);
      __syncthreads();
      x_load(r2, c + 5);
      x_store(r0, 0, c + 3);
      __syncthreads();
    }
    return;
  }

  // ---- compute waves
  const int hd_raw = blockIdx.y * proj_per_wg + wave;
  // compute waves past the last projection (last group only) redo the key
  // projection and store nothing
  const int hd = min(hd_raw, a.h_kv);
  const bf16_t* w = static_cast<const bf16_t*>(hd < a.h_kv ? a.w_q : a.w_k) +
                    (hd < a.h_kv ? (size_t)hd * DI * D : 0);
  // W operand of feature tile ft, 16-wide step st: row ft*32 + l32,
  // k = 64 c + 16 st + 8 half (the x operand below uses the same k); past
  // d_model an in-bounds piece is loaded and replaced by zeros where it is
  // used, a chunk later
  auto w_frag = [&](int ft, int st, int c) __attribute__((always_inline)) {
    return load_frag<bf16_t>(w + (size_t)(ft * 32 + l32) * D + min(c * kKxChunk + 16 * st + 8 * half, D - 8));
  };
  f32x16 acc[TT][FT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) acc[tt][ft] = f32x16{};
  bf16x8 wa[FT][kKxSteps];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int st = 0; st < kKxSteps; ++st) wa[ft][st] = w_frag(ft, st, 0);
  __syncthreads();
  auto chunk = [&](int c, int buf) __attribute__((always_inline)) {
    const int cn = c + 1;
    const unsigned char* xb = xs[buf] + l32 * kKxRowBytes + 16 * half;
    // x operand of tile tt, step st: row tt*32 + l32, k = 16 st + 8 half;
    // each step's operands are read from LDS one step ahead of their MFMAs
    bf16x8 bx[TT], bn[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) bx[tt] = *reinterpret_cast<const bf16x8*>(xb + tt * 32 * kKxRowBytes);
#pragma unroll
    for (int st = 0; st < kKxSteps; ++st) {
      if (st < kKxSteps - 1) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          bn[tt] = *reinterpret_cast<const bf16x8*>(xb + tt * 32 * kKxRowBytes + 32 * (st + 1));
      }
      const bool in = c * kKxChunk + 16 * st + 8 * half < D;
      bf16x8 wv[FT];
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) wv[ft] = in ? wa[ft][st] : zero_frag<bf16_t>();
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) mma32(acc[tt][ft], wv[ft], bx[tt]);
      // this step's W operands are free: load the next chunk's in their place
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) wa[ft][st] = w_frag(ft, st, cn);
      MSA_SCHED_FENCE();
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) bx[tt] = bn[tt];
    }
    __syncthreads();
  };
  for (int c = 0; c < nch3; c += 3) {
    chunk(c, 0);
    chunk(c + 1, 1);
    chunk(c + 2, 2);
  }
  if (hd_raw > a.h_kv) return;
  // one call per tile with a constant index (a loop over tiles this large is
  // not unrolled, and a variable index would put acc in private memory)
  auto store = [&](f32x16(&t)[FT], int tt) __attribute__((always_inline)) {
    const int t_raw = tok0 + tt * 32 + l32;
    kx_rope_store<DI>(t, min(t_raw, a.n_tok - 1), t_raw < a.n_tok, hd, a);
  };
  store(acc[0], 0);
  if constexpr (TT > 1) store(acc[1], 1);
  if constexpr (TT > 2) {
    store(acc[2], 2);
    store(acc[3], 3);
  }
}

template <int DI>
static void kx_tile_launch(const KxArgs& a, hipStream_t st) {
  constexpr int ROWS = kx_tile_tt<DI>() * 32;
  const int nproj = a.h_kv + 1;
  const int groups = (nproj + kKxMaxCompute - 1) / kKxMaxCompute;
  const int P = (nproj + groups - 1) / groups;  // compute waves, 1 .. 5
  const dim3 grid((unsigned)((a.n_tok + ROWS - 1) / ROWS), (unsigned)groups), block(kKxTileWaves * 64);
  hipLaunchKernelGGL((kx_tile_kernel<DI>), grid, block, 0, st, a, P);
}

hipError_t launch_index_project(int d_idx, const KxArgs& a, hipStream_t st) {
  if (a.n_tok == 0) return hipSuccess;
  if (d_idx != 32 && d_idx != 64 && d_idx != 128) return hipErrorInvalidValue;
  if (a.n_tok >= kKxTileMinTokens) {
    if (d_idx == 32) kx_tile_launch<32>(a, st);
    else if (d_idx == 64) kx_tile_launch<64>(a, st);
    else kx_tile_launch<128>(a, st);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a.n_tok + 31) / 32), (unsigned)(a.h_kv + 1), (unsigned)std::max(1, a.split));
  const dim3 block(kKxWaves * 64);
  if (d_idx == 32) hipLaunchKernelGGL(kx_project_kernel<32>, grid, block, 0, st, a);
  else if (d_idx == 64) hipLaunchKernelGGL(kx_project_kernel<64>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(kx_project_kernel<128>, grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.split <= 1) return e;
  const int64_t n = (int64_t)a.n_tok * (a.h_kv + 1) * (d_idx - a.rope_dim / 2);
  const dim3 rg((unsigned)((n + 255) / 256));
  if (d_idx == 32) hipLaunchKernelGGL(kx_reduce_kernel<32>, rg, dim3(256), 0, st, a);
  else if (d_idx == 64) hipLaunchKernelGGL(kx_reduce_kernel<64>, rg, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(kx_reduce_kernel<128>, rg, dim3(256), 0, st, a);
  return hipGetLastError();
}

KxPlan kx_plan(int32_t n_tok, int32_t d_model, int32_t h_kv, int32_t d_idx) {
  KxPlan p{1, d_model, 0};
  if (n_tok <= 0 || n_tok >= kKxTileMinTokens || d_model <= 0) return p;
  // aim for >= 256 workgroups; every slice keeps >= 2 steps of 16 per wave
  const int64_t wg = (int64_t)((n_tok + 31) / 32) * (h_kv + 1);
  const int64_t want = (256 + wg - 1) / wg;
  const int64_t most = std::max<int64_t>(1, d_model / (kKxWaves * 32));
  const int64_t split = std::min(want, most);
  if (split <= 1) return p;
  const int32_t kps = (int32_t)(((d_model + split - 1) / split + 15) / 16 * 16);
  p.k_per_split = kps;
  p.split = (d_model + kps - 1) / kps;
  p.total = (size_t)p.split * n_tok * (h_kv + 1) * d_idx * sizeof(float);
  return p;
}

}  // namespace msa
