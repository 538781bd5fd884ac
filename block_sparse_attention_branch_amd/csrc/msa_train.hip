// msa_train.hip - training path of the main branch on gfx950.
//
// Gradients of Eq. (8) of the "MiniMax Sparse Attention" digest
// (titansim.online, §4.3) over the selected blocks, for the training of §4.5.
// Per (token, head) row with P = softmax over the visible keys of the
// group's selected blocks, dP = dO.V^T and D = rowsum(dO * O):
//   dS = P * (dP - D),  dQ = scale * dS.K,  dK = scale * dS^T.Q,  dV = P^T.dO.
// P is recomputed from the forward's lse.  Both passes are KV-outer like the
// forward (§4.4.2) and run on the forward's schedule kernels:
//  * dQ pass (windows of query tokens): an item is one (group, block) and up
//    to 512 of the rows that selected it; S^T = K.Q^T, dP^T = V.dO^T and
//    dQ^T = K^T.dS^T on v_mfma_f32_32x32x16_bf16 with keys on the MFMA rows.
//    Each (token, head, slot) writes a bf16 partial dQ and a merge kernel
//    sums a row's partials (the two-stage merge without rescaling).
//  * dK/dV pass (one window over all queries): an item keeps its block's
//    dK^T and dV^T in registers (four waves of 32 keys) while it sweeps its
//    rows 32 at a time: S = Q.K^T, dP = dO.V^T, dV^T += dO^T.P,
//    dK^T += Q^T.dS.  A (group, block) cell split over several items writes
//    fp32 partials that a reduce kernel sums; unselected blocks get zeros.
// No floating-point atomics: results are bitwise reproducible.
#include "msa_common.hpp"
#include "msa_internal.hpp"
#include "msa_kvouter.hpp"
#include "msa_profile.hpp"

namespace msa {

struct KbArgs {
  const void* q;            // [n_q, h_q, D]
  const void* k;            // [n_kv, h_kv, D]
  const void* v;
  const void* o;            // [n_q, h_q, D]
  const float* lse;         // [n_q, h_q]
  const void* d_o;          // [n_q, h_q, D]
  void* dq;                 // [n_q, h_q, D]
  void* dk;                 // [n_kv, h_kv, D]
  void* dv;
  float* dsum;              // [n_q, h_q]  rowsum(dO * O)
  const int32_t* block_idx; // [n_q, h_kv, top_k]
  const int32_t* item_off;
  const int32_t* entries;
  const i32x4* items;
  int32_t* queue;           // dK/dV pass: next item to take (zeroed by the schedule)
  bf16_t* part_dq;          // dQ pass: [window * h_kv * top_k + 2 trash, G, D]
  float* part_dkv;          // dK/dV pass: [max_items, 2, 128, D]
  int32_t n_q, q_start, n_kv, h_q, h_kv, group, g_shift, top_k, n_blocks, window, w;
  size_t trash_slot;
  float sm_scale;
  // KL-alignment term (pmain == NULL: not requested)
  float* pmain;             // [n_q, h_kv, top_k, 128] group-mean main-branch probabilities per selected key
  const void* q_idx;        // [n_q, h_kv, d_idx]
  const void* k_idx;        // [n_kv, d_idx]
  float idx_scale, kl_scale;
  float* part_kl;           // index pass: [window * h_kv * top_k + 1 trash, 4 + 2 d_idx]
  float* lse_idx;           // [n_q, h_kv]
  float* kl;                // [n_q, h_kv], nullable
  void* dq_idx;             // [n_q, h_kv, d_idx]
  void* dk_idx;             // [n_kv, d_idx]
  float* part_dki;          // dk_idx pass: [max_items, 128, d_idx]
};

// ------------------------------------------------------------- D = rowsum
template <int D>
__global__ __launch_bounds__(256) void kb_dsum_kernel(KbArgs a) {
  constexpr int LPR = D / 8;  // lanes per row, 8 values each
  const int64_t t = blockIdx.x * 256ll + threadIdx.x;
  const int64_t row = t / LPR;
  const int c = (int)(t % LPR);
  const bool ok = row < (int64_t)a.n_q * a.h_q;
  float s = 0.0f;
  if (ok) {
    const bf16x8 x = load_frag<bf16_t>(static_cast<const bf16_t*>(a.o) + row * D + c * 8);
    const bf16x8 y = load_frag<bf16_t>(static_cast<const bf16_t*>(a.d_o) + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(to_f32(x[e]), to_f32(y[e]), s);
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off, 64);
  if (ok && c == 0) a.dsum[row] = s;
}

// ----------------------------------------------------- K/V block staging
// The dQ pass needs K with keys on rows (for S^T = K.Q^T), V with keys on
// rows (dP^T = V.dO^T) and K^T with d on rows (dQ^T = K^T.dS^T).  K is
// loaded as pairs of adjacent keys so both layouts come from one load.
template <int D>
struct KbqLds {
  static constexpr int KS = D * 2 + 16;   // bytes per key row
  static constexpr int TS = 128 * 2 + 8;  // bytes per d row of K^T
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 128 * KS;
  static constexpr int KT_OFF = 2 * 128 * KS;
  static constexpr int ENT_OFF = KT_OFF + D * TS;
  static constexpr int BYTES = ENT_OFF + 512 * 4;  // token entries of an item (at most 512)
};

template <int D, int NT>
struct KbStage {
  static constexpr int DC = D / 8;
  static constexpr int KU = 64 * DC / NT;   // (key pair, chunk) units of K per thread
  static constexpr int VL = 128 * DC / NT;  // key-row chunks of V per thread
  static_assert(KU >= 1 && VL >= 1, "staging split");
  u32x4 k[KU][2];
  u32x4 v[VL];
  uint32_t zk, zv;  // bit set: that row lies past n_kv (stored as zeros)
};

template <int D, int NT>
__device__ __forceinline__ void kb_stage_load(KbStage<D, NT>& g, const KbArgs& a, int b, int r) {
  using S = KbStage<D, NT>;
  const int stride = a.h_kv * D * 2;
  const char* kb = static_cast<const char*>(a.k) + (((size_t)b * kBlock) * a.h_kv + r) * D * 2;
  const char* vb = static_cast<const char*>(a.v) + (((size_t)b * kBlock) * a.h_kv + r) * D * 2;
  const int last = min(kBlock, a.n_kv - b * kBlock) - 1;
  uint32_t zk = 0, zv = 0;
#pragma unroll
  for (int i = 0; i < S::KU; ++i) {
    const int u = threadIdx.x + NT * i;
    const int dc = u % S::DC, kp = u / S::DC;
    g.k[i][0] = *reinterpret_cast<const u32x4*>(kb + (size_t)min(2 * kp, last) * stride + dc * 16);
    g.k[i][1] = *reinterpret_cast<const u32x4*>(kb + (size_t)min(2 * kp + 1, last) * stride + dc * 16);
    zk |= (2 * kp > last ? 1u : 0u) << (2 * i);
    zk |= (2 * kp + 1 > last ? 1u : 0u) << (2 * i + 1);
  }
#pragma unroll
  for (int i = 0; i < S::VL; ++i) {
    const int u = threadIdx.x + NT * i;
    const int dc = u % S::DC, j = u / S::DC;
    g.v[i] = *reinterpret_cast<const u32x4*>(vb + (size_t)min(j, last) * stride + dc * 16);
    zv |= (j > last ? 1u : 0u) << i;
  }
  g.zk = zk;
  g.zv = zv;
}

template <int D, int NT>
__device__ __forceinline__ void kb_stage_store(const KbStage<D, NT>& g, char* lds) {
  using S = KbStage<D, NT>;
  using L = KbqLds<D>;
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < S::KU; ++i) {
    const int u = threadIdx.x + NT * i;
    const int dc = u % S::DC, kp = u / S::DC;
    const u32x4 x = ((g.zk >> (2 * i)) & 1u) ? z : g.k[i][0];
    const u32x4 y = ((g.zk >> (2 * i + 1)) & 1u) ? z : g.k[i][1];
    *reinterpret_cast<u32x4*>(lds + L::K_OFF + (2 * kp) * L::KS + dc * 16) = x;
    *reinterpret_cast<u32x4*>(lds + L::K_OFF + (2 * kp + 1) * L::KS + dc * 16) = y;
#pragma unroll
    for (int t = 0; t < 4; ++t) {  // K^T: d rows, each 32-bit word = keys (2kp, 2kp + 1)
      const uint32_t lo = (x[t] & 0xffffu) | (y[t] << 16);
      const uint32_t hi = (x[t] >> 16) | (y[t] & 0xffff0000u);
      *reinterpret_cast<uint32_t*>(lds + L::KT_OFF + (8 * dc + 2 * t) * L::TS + kp * 4) = lo;
      *reinterpret_cast<uint32_t*>(lds + L::KT_OFF + (8 * dc + 2 * t + 1) * L::TS + kp * 4) = hi;
    }
  }
#pragma unroll
  for (int i = 0; i < S::VL; ++i) {
    const int u = threadIdx.x + NT * i;
    const int dc = u % S::DC, j = u / S::DC;
    *reinterpret_cast<u32x4*>(lds + L::V_OFF + j * L::KS + dc * 16) = ((g.zv >> i) & 1u) ? z : g.v[i];
  }
}

// Sum over aligned runs of n lanes (n = 1, 2, 4, 8 or 16) with DPP moves on
// the VALU: quad permutations for 2 and 4, then the half-row and row
// mirrors, which pair the remaining quads and half-rows of a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_group_sum(float x, int n) {
  if (n >= 2) x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  if (n >= 4) x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  if (n >= 8) x += dpp_f32<0x141>(x);  // row_half_mirror
  if (n >= 16) x += dpp_f32<0x140>(x); // row_mirror
  return x;
}

// ---------------------------------------------------------------- dQ pass
constexpr int kKbqThreads = 512;      // 8 waves, 32 rows each per pass
constexpr int kKbqRowsPerPass = 256;

template <int D>
struct KbqPass {
  bf16x8 qf[D / 16];
  bf16x8 df[D / 16];
  float lse2, dsum;
  int pos, slot, head;
  int64_t slot_g;  // (token, group, slot) over the whole call; rows past the item: a trash slot
  bool ok;
};

// Row `rho` of item m (entries in LDS); rows past the item's end load a valid
// row and are flagged !ok.
template <int D>
__device__ __forceinline__ void kbq_load_pass(KbqPass<D>& ps, const KbArgs& a, const KpItem& m, int rho,
                                              const int* ent_lds) {
  const int half = (threadIdx.x & 63) >> 5;
  const int G = a.group;
  const int n_tok = m.e_end - m.e_begin;
  ps.ok = rho < n_tok * G;
  const int ent = ent_lds[min(rho >> a.g_shift, n_tok - 1)];
  const int i = ent >> 4, j = ent & 15;
  ps.head = rho & (G - 1);
  ps.slot = ((i - a.w * a.window) * a.h_kv + m.r) * a.top_k + j;
  ps.slot_g = ps.ok ? ((int64_t)i * a.h_kv + m.r) * a.top_k + j : (int64_t)a.n_q * a.h_kv * a.top_k;
  ps.pos = ps.ok ? a.q_start + i : -1;
  const size_t row = (size_t)i * a.h_q + m.r * G + ps.head;
  const bf16_t* qrow = static_cast<const bf16_t*>(a.q) + row * D + half * 8;
  const bf16_t* drow = static_cast<const bf16_t*>(a.d_o) + row * D + half * 8;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    ps.qf[ks] = load_frag<bf16_t>(qrow + ks * 16);
    ps.df[ks] = load_frag<bf16_t>(drow + ks * 16);
  }
  ps.lse2 = a.lse[row] * kLog2e;
  ps.dsum = a.dsum[row];
}

// dQ^T of the wave's 32 rows against the staged block, one 32-key tile at a
// time to bound the live accumulators.
template <int D, bool KL>
__device__ __forceinline__ void kbq_math(const KbArgs& a, int b, const KbqPass<D>& ps, const char* lds,
                                         f32x16 (&dq)[D / 32]) {
  using L = KbqLds<D>;
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const float c2 = a.sm_scale * kLog2e;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dq[dt] = f32x16{};
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int off = (kt * 32 + l32) * L::KS + (ks * 16 + half * 8) * 2;
      mma32(s, *reinterpret_cast<const bf16x8*>(lds + L::K_OFF + off), ps.qf[ks]);
      mma32(dp, *reinterpret_cast<const bf16x8*>(lds + L::V_OFF + off), ps.df[ks]);
    }
    float dsv[16], pm[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = b * kBlock + kt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      const float pv = fast_exp2(key > ps.pos ? -__builtin_inff() : fmaf(s[v], c2, -ps.lse2));
      dsv[v] = pv * (dp[v] - ps.dsum);
      pm[v] = pv;
    }
    if constexpr (KL) {
      // group mean of P over the token's heads (lanes token * G + head of
      // this half, an aligned run of G <= 16 lanes), written by all of them
      // (same values, same addresses)
#pragma unroll
      for (int v = 0; v < 16; ++v) pm[v] = lane_group_sum(pm[v], a.group);
      const float inv_g = 1.0f / (float)a.group;
      float* dst = a.pmain + ((size_t)ps.slot_g * kBlock + kt * 32 + 4 * half);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<f32x4*>(dst + 8 * c) =
            f32x4{pm[4 * c] * inv_g, pm[4 * c + 1] * inv_g, pm[4 * c + 2] * inv_g, pm[4 * c + 3] * inv_g};
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int o = 8 * h2, base = kt * 32 + h2 * 16;
      const bf16x8 dsf = to_frag<bf16_t>(dsv[o], dsv[o + 1], dsv[o + 2], dsv[o + 3], dsv[o + 4], dsv[o + 5],
                                         dsv[o + 6], dsv[o + 7]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        mma32(dq[dt], vt_frag<bf16_t>(lds + L::KT_OFF, L::TS, dt * 32 + l32, base + 4 * half, base + 8 + 4 * half),
              dsf);
    }
    MSA_SCHED_FENCE();
  }
}

// bf16 partial of (token, slot) (like the forward's partial O): [G][D] in
// natural order; rows past the item write the trash slot so the store count
// never depends on the data.
template <int D>
__device__ __forceinline__ void kbq_store(const KbArgs& a, const KbqPass<D>& ps, const f32x16 (&dq)[D / 32]) {
  const int half = (threadIdx.x & 63) >> 5;
  const size_t slot = ps.ok ? (size_t)ps.slot : a.trash_slot;
  bf16_t* dst = a.part_dq + (slot * a.group + ps.head) * D;
  const float sc = a.sm_scale;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      store4<bf16_t>(dst + dt * 32 + 8 * c + 4 * half, dq[dt][4 * c] * sc, dq[dt][4 * c + 1] * sc,
                     dq[dt][4 * c + 2] * sc, dq[dt][4 * c + 3] * sc);
}

// Persistent over this XCD's items of window w (the forward's item order):
// workgroup g runs on XCD g % 8 and takes items sub, sub + nsub, ...  The next
// item's K/V are loaded into registers while the current item computes.
template <int D, bool KL>
__global__ __launch_bounds__(kKbqThreads) void kbq_kernel(KbArgs a) {
  using L = KbqLds<D>;
  constexpr int NT = kKbqThreads;
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  const int x = blockIdx.x & 7, sub = blockIdx.x >> 3, nsub = gridDim.x >> 3;
  const int64_t n_l = (int64_t)a.h_kv * a.n_blocks, per = n_l >> 3;
  const int64_t k0 = (int64_t)a.w * n_l + x * per;
  const int item_begin = scalar_load(a.item_off, k0);
  const int item_end = scalar_load(a.item_off, k0 + per);
  int it = item_begin + sub;
  if (it >= item_end) return;
  const int tid = threadIdx.x, wave = tid >> 6, l32 = tid & 31;
  int* ent_lds = reinterpret_cast<int*>(lds + L::ENT_OFF);

  KbStage<D, NT> pre;
  i32x4 d = scalar_load(a.items, __builtin_amdgcn_readfirstlane(it));
  KpItem cur{d[0], d[1], d[2], d[3]};
  kb_stage_load<D, NT>(pre, a, cur.b, cur.r);
  int pre_ent = a.entries[cur.e_begin + min(tid, cur.e_end - cur.e_begin - 1)];
  for (;;) {
    kb_stage_store<D, NT>(pre, lds);
    ent_lds[tid] = pre_ent;
    __syncthreads();
    const int nx = it + nsub;
    const bool has_next = nx < item_end;
    KpItem nxt = cur;
    if (has_next) {
      d = scalar_load(a.items, __builtin_amdgcn_readfirstlane(nx));
      nxt = KpItem{d[0], d[1], d[2], d[3]};
      kb_stage_load<D, NT>(pre, a, nxt.b, nxt.r);
      pre_ent = a.entries[nxt.e_begin + min(tid, nxt.e_end - nxt.e_begin - 1)];
    }
    const int rows = (cur.e_end - cur.e_begin) * a.group;
    for (int p0 = 0; p0 < rows; p0 += kKbqRowsPerPass) {
      KbqPass<D> ps;
      kbq_load_pass<D>(ps, a, cur, p0 + wave * 32 + l32, ent_lds);
      if (__any(ps.ok)) {
        f32x16 dq[D / 32];
        kbq_math<D, KL>(a, cur.b, ps, lds, dq);
        kbq_store<D>(a, ps, dq);
      }
    }
    if (!has_next) break;
    __syncthreads();  // every wave is done with this item's LDS
    it = nx;
    cur = nxt;
  }
}

// Second stage of dQ: the sum of a row's per-slot partials.
template <int D>
__global__ __launch_bounds__(256) void kbq_merge_kernel(KbArgs a) {
  constexpr int DC = D / 8;
  const int64_t t = blockIdx.x * 256ll + threadIdx.x;
  const int64_t rl = t / DC;  // il * h_q + h
  const int c = (int)(t % DC);
  const int il = (int)(rl / a.h_q), h = (int)(rl % a.h_q);
  const int i = a.w * a.window + il;
  if (il >= a.window || i >= a.n_q) return;
  const int G = a.group, r = h / G, g = h % G;
  const int diag = (a.q_start + i) >> 7;
  const uint32_t used = used_slots(a.block_idx + ((size_t)i * a.h_kv + r) * a.top_k, a.top_k, diag);
  const size_t slot0 = ((size_t)il * a.h_kv + r) * a.top_k;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.top_k; ++j) {
    if (!((used >> j) & 1u)) continue;
    const bf16x8 x = load_frag<bf16_t>(a.part_dq + ((slot0 + j) * G + g) * D + c * 8);
    s0 += f32x4{to_f32(x[0]), to_f32(x[1]), to_f32(x[2]), to_f32(x[3])};
    s1 += f32x4{to_f32(x[4]), to_f32(x[5]), to_f32(x[6]), to_f32(x[7])};
  }
  bf16_t* dst = static_cast<bf16_t*>(a.dq) + ((size_t)i * a.h_q + h) * D + c * 8;
  *reinterpret_cast<bf16x8*>(dst) = bf16x8{from_f32<bf16_t>(s0[0]), from_f32<bf16_t>(s0[1]), from_f32<bf16_t>(s0[2]),
                                           from_f32<bf16_t>(s0[3]), from_f32<bf16_t>(s1[0]), from_f32<bf16_t>(s1[1]),
                                           from_f32<bf16_t>(s1[2]), from_f32<bf16_t>(s1[3])};
}

// ------------------------------------------------------------ dK/dV pass
constexpr int kKbkvThreads = 256;  // 4 waves, 32 keys each

template <int D>
struct KbkvLds {
  static constexpr int KS = D * 2 + 16;   // bytes per key row / query row
  static constexpr int TS = 32 * 2 + 8;   // bytes per d row of a 32-row Q^T / dO^T tile
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = 128 * KS;
  // one row tile: Q rows, dO rows, Q^T, dO^T, then lse2, dsum, pos per row
  static constexpr int Q_R = 0;
  static constexpr int D_R = 32 * KS;
  static constexpr int Q_T = 2 * 32 * KS;
  static constexpr int D_T = Q_T + D * TS;
  static constexpr int SC = D_T + D * TS;
  static constexpr int TILE = SC + 3 * 32 * 4;
  static constexpr int T_OFF = 2 * 128 * KS;
  static constexpr int ENT_OFF = T_OFF + 2 * TILE;
  static constexpr int ENT_CAP = 2048;  // token entries of an item
  static constexpr int BYTES = ENT_OFF + ENT_CAP * 4;
};

// Row tile staging: unit u = (row pair rp, 16-byte chunk dc) of Q and dO.
template <int D>
struct KbkvTileRegs {
  u32x4 q0, q1, d0, d1;
  float lse2, dsum;
  int pos;
};

// Every thread issues the same loads whatever its index (the last units and
// the per-row scalars are duplicated across threads and only some threads
// store them), so no load sits under a divergent branch: the compiler then
// never has to drain the loads of the passes in flight to resolve one.
// Pass `ps` of an item with `n_pass` passes; passes past the end re-read the
// last one's rows but flag every row invalid (pos -1), so they add nothing.
template <int D>
__device__ __forceinline__ void kbkv_tile_load(KbkvTileRegs<D>& g, const KbArgs& a, const KpItem& m, int ps,
                                               int n_pass, const int* ent_lds) {
  constexpr int DC = D / 8;
  const int tid = threadIdx.x;
  const int G = a.group, n_tok = m.e_end - m.e_begin, rows = n_tok * G;
  const int row0 = min(ps, n_pass - 1) * 32;
  const int u = tid % (16 * DC);
  const int dc = u % DC, rp = u / DC;
  const int ra = row0 + 2 * rp, rb = ra + 1;
  const int ea = ent_lds[min(ra >> a.g_shift, n_tok - 1)], eb = ent_lds[min(rb >> a.g_shift, n_tok - 1)];
  const size_t xa = ((size_t)(ea >> 4) * a.h_q + m.r * G + (ra & (G - 1))) * D + dc * 8;
  const size_t xb = ((size_t)(eb >> 4) * a.h_q + m.r * G + (rb & (G - 1))) * D + dc * 8;
  g.q0 = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(a.q) + xa);
  g.q1 = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(a.q) + xb);
  g.d0 = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(a.d_o) + xa);
  g.d1 = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(a.d_o) + xb);
  const int rr = row0 + (tid & 31);
  const bool ok = ps * 32 + (tid & 31) < rows;
  const int e = ent_lds[min(rr >> a.g_shift, n_tok - 1)];
  const size_t x = (size_t)(e >> 4) * a.h_q + m.r * G + (rr & (G - 1));
  const float l = a.lse[x], ds = a.dsum[x];
  g.lse2 = ok ? l * kLog2e : 0.0f;
  g.dsum = ok ? ds : 0.0f;
  g.pos = ok ? a.q_start + (e >> 4) : -1;
}

template <int D>
__device__ __forceinline__ void kbkv_tile_store(const KbkvTileRegs<D>& g, char* tile) {
  using L = KbkvLds<D>;
  constexpr int DC = D / 8;
  const int tid = threadIdx.x;
  if (tid < 16 * DC) {
    const int dc = tid % DC, rp = tid / DC;
    *reinterpret_cast<u32x4*>(tile + L::Q_R + (2 * rp) * L::KS + dc * 16) = g.q0;
    *reinterpret_cast<u32x4*>(tile + L::Q_R + (2 * rp + 1) * L::KS + dc * 16) = g.q1;
    *reinterpret_cast<u32x4*>(tile + L::D_R + (2 * rp) * L::KS + dc * 16) = g.d0;
    *reinterpret_cast<u32x4*>(tile + L::D_R + (2 * rp + 1) * L::KS + dc * 16) = g.d1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {  // d rows; each 32-bit word = rows (2rp, 2rp + 1)
      *reinterpret_cast<uint32_t*>(tile + L::Q_T + (8 * dc + 2 * t) * L::TS + rp * 4) =
          (g.q0[t] & 0xffffu) | (g.q1[t] << 16);
      *reinterpret_cast<uint32_t*>(tile + L::Q_T + (8 * dc + 2 * t + 1) * L::TS + rp * 4) =
          (g.q0[t] >> 16) | (g.q1[t] & 0xffff0000u);
      *reinterpret_cast<uint32_t*>(tile + L::D_T + (8 * dc + 2 * t) * L::TS + rp * 4) =
          (g.d0[t] & 0xffffu) | (g.d1[t] << 16);
      *reinterpret_cast<uint32_t*>(tile + L::D_T + (8 * dc + 2 * t + 1) * L::TS + rp * 4) =
          (g.d0[t] >> 16) | (g.d1[t] & 0xffff0000u);
    }
  }
  if (tid < 32) {
    float* sc = reinterpret_cast<float*>(tile + L::SC);
    sc[tid] = g.lse2;
    sc[32 + tid] = g.dsum;
    reinterpret_cast<int*>(sc + 64)[tid] = g.pos;
  }
}

// Items of all (group, block) cells taken from a work queue by a persistent
// grid (items run in cell order, which puts the most-selected early blocks
// first).  Each wave owns keys 32*wave .. 32*wave + 31 of the item's block.
template <int D>
__global__ __launch_bounds__(kKbkvThreads) void kbkv_kernel(KbArgs a) {
  using L = KbkvLds<D>;
  constexpr int NT = kKbkvThreads;
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int n_items = scalar_load(a.item_off, (int64_t)a.h_kv * a.n_blocks);
  int* ent_lds = reinterpret_cast<int*>(lds + L::ENT_OFF);
  const float c2 = a.sm_scale * kLog2e;
  __shared__ int next_item;
  for (;;) {
    if (tid == 0) next_item = atomicAdd(a.queue, 1);
    __syncthreads();
    const int it = next_item;
    if (it >= n_items) break;
    const i32x4 d = scalar_load(a.items, __builtin_amdgcn_readfirstlane(it));
    const KpItem m{d[0], d[1], d[2], d[3]};
    const int n_tok = m.e_end - m.e_begin;
    const int rows = n_tok * a.group;
    __syncthreads();  // the previous item's readers are done
    // K and V rows of the block (zeros past n_kv)
    {
      constexpr int DC = D / 8;
      const int stride = a.h_kv * D * 2;
      const size_t base = (((size_t)m.b * kBlock) * a.h_kv + m.r) * D * 2;
      const int last = min(kBlock, a.n_kv - m.b * kBlock) - 1;
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 128 * DC / NT; ++i) {
        const int u = tid + NT * i;
        const int dc = u % DC, j = u / DC;
        const size_t off = base + (size_t)min(j, last) * stride + dc * 16;
        const u32x4 kx = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.k) + off);
        const u32x4 vx = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v) + off);
        *reinterpret_cast<u32x4*>(lds + L::K_OFF + j * L::KS + dc * 16) = j > last ? z : kx;
        *reinterpret_cast<u32x4*>(lds + L::V_OFF + j * L::KS + dc * 16) = j > last ? z : vx;
      }
      for (int e = tid; e < n_tok; e += NT) ent_lds[e] = a.entries[m.e_begin + e];
    }
    __syncthreads();
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      dk[dt] = f32x16{};
      dv[dt] = f32x16{};
    }
    const int key_abs = m.b * kBlock + wave * 32 + l32;
    const int n_pass = (rows + 31) / 32;
    // this wave's 32 keys of K and V stay in registers for the whole item
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int koff = (wave * 32 + l32) * L::KS + (ks * 16 + half * 8) * 2;
      kf[ks] = *reinterpret_cast<const bf16x8*>(lds + L::K_OFF + koff);
      vf[ks] = *reinterpret_cast<const bf16x8*>(lds + L::V_OFF + koff);
    }
    // Row tiles are gathered three passes ahead through a ring of register
    // sets (x: the next pass's tile, y: the one after, z: free) and stored to
    // the LDS buffer the pass after next reads.
    KbkvTileRegs<D> ga, gb, gc;
    // (loads are unconditional: past the last pass they re-read it, so the
    // number of loads in flight never depends on the data)
    kbkv_tile_load<D>(ga, a, m, 0, n_pass, ent_lds);
    kbkv_tile_load<D>(gb, a, m, 1, n_pass, ent_lds);
    kbkv_tile_load<D>(gc, a, m, 2, n_pass, ent_lds);
    kbkv_tile_store<D>(ga, lds + L::T_OFF);
    __syncthreads();
    auto pass = [&](int ps, KbkvTileRegs<D>& gx, KbkvTileRegs<D>& gz) {
      const char* tile = lds + L::T_OFF + (ps & 1) * L::TILE;
      kbkv_tile_load<D>(gz, a, m, ps + 3, n_pass, ent_lds);
      // S = Q.K^T and dP = dO.V^T for the tile's 32 rows x this wave's 32 keys
      f32x16 sa = {}, dpa = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int roff = l32 * L::KS + (ks * 16 + half * 8) * 2;
        mma32(sa, *reinterpret_cast<const bf16x8*>(tile + L::Q_R + roff), kf[ks]);
        mma32(dpa, *reinterpret_cast<const bf16x8*>(tile + L::D_R + roff), vf[ks]);
      }
      // per-row lse, D and position of this lane's 16 rows (4 runs of 4)
      const float* sc = reinterpret_cast<const float*>(tile + L::SC);
      float pv[16], dsv[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r0 = 8 * c + 4 * half;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(sc + r0);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sc + 32 + r0);
        const i32x4 p4 = *reinterpret_cast<const i32x4*>(sc + 64 + r0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v = 4 * c + q;
          const float pr = fast_exp2(key_abs > p4[q] ? -__builtin_inff() : fmaf(sa[v], c2, -l4[q]));
          pv[v] = pr;
          dsv[v] = pr * (dpa[v] - d4[q]);
        }
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int o = 8 * h2;
        const bf16x8 pf = to_frag<bf16_t>(pv[o], pv[o + 1], pv[o + 2], pv[o + 3], pv[o + 4], pv[o + 5], pv[o + 6],
                                          pv[o + 7]);
        const bf16x8 dsf = to_frag<bf16_t>(dsv[o], dsv[o + 1], dsv[o + 2], dsv[o + 3], dsv[o + 4], dsv[o + 5],
                                           dsv[o + 6], dsv[o + 7]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int dd = dt * 32 + l32;
          mma32(dv[dt], vt_frag<bf16_t>(tile + L::D_T, L::TS, dd, 16 * h2 + 4 * half, 16 * h2 + 8 + 4 * half), pf);
          mma32(dk[dt], vt_frag<bf16_t>(tile + L::Q_T, L::TS, dd, 16 * h2 + 4 * half, 16 * h2 + 8 + 4 * half), dsf);
        }
      }
      kbkv_tile_store<D>(gx, lds + L::T_OFF + ((ps + 1) & 1) * L::TILE);
      __syncthreads();
    };
    // ring rotation: pass ps stores the set holding pass ps + 1 and refills
    // the free set with pass ps + 3.  The body always runs three passes (up
    // to two of them past the end, adding zeros) so no branch splits the
    // loads in flight.
    for (int ps = 0; ps < n_pass; ps += 3) {
      pass(ps, gb, ga);
      pass(ps + 1, gc, gb);
      pass(ps + 2, ga, gc);
    }
    // dK = scale * (dS^T.Q), dV = P^T.dO for key `key_abs`: lane holds d =
    // dt*32 + 8c + 4*half + {0..3}
    const int64_t cell = cell_key(0, m.r, m.b, a.n_blocks, a.h_kv);
    const int ib = scalar_load(a.item_off, cell), ie = scalar_load(a.item_off, cell + 1);
    if (ie - ib == 1) {
      if (key_abs < a.n_kv) {
        bf16_t* pk = static_cast<bf16_t*>(a.dk) + ((size_t)key_abs * a.h_kv + m.r) * D;
        bf16_t* pv2 = static_cast<bf16_t*>(a.dv) + ((size_t)key_abs * a.h_kv + m.r) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int d0 = dt * 32 + 8 * c + 4 * half;
            store4<bf16_t>(pk + d0, dk[dt][4 * c] * a.sm_scale, dk[dt][4 * c + 1] * a.sm_scale,
                           dk[dt][4 * c + 2] * a.sm_scale, dk[dt][4 * c + 3] * a.sm_scale);
            store4<bf16_t>(pv2 + d0, dv[dt][4 * c], dv[dt][4 * c + 1], dv[dt][4 * c + 2], dv[dt][4 * c + 3]);
          }
      }
    } else {
      float* pk = a.part_dkv + (((size_t)it * 2 + 0) * kBlock + wave * 32 + l32) * D;
      float* pv2 = a.part_dkv + (((size_t)it * 2 + 1) * kBlock + wave * 32 + l32) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int d0 = dt * 32 + 8 * c + 4 * half;
          *reinterpret_cast<f32x4*>(pk + d0) = f32x4{dk[dt][4 * c] * a.sm_scale, dk[dt][4 * c + 1] * a.sm_scale,
                                                     dk[dt][4 * c + 2] * a.sm_scale, dk[dt][4 * c + 3] * a.sm_scale};
          *reinterpret_cast<f32x4*>(pv2 + d0) = f32x4{dv[dt][4 * c], dv[dt][4 * c + 1], dv[dt][4 * c + 2],
                                                      dv[dt][4 * c + 3]};
        }
    }
  }
}

// dK/dV of every (block, group): the sum of a split cell's item partials, or
// zeros for blocks no query selected.  Single-item cells were written by the
// pass itself.
template <int D>
__global__ __launch_bounds__(256) void kbkv_reduce_kernel(KbArgs a) {
  const int b = blockIdx.x, r = blockIdx.y;
  int ib = 0, ie = 0;
  if (b < a.n_blocks) {
    const int64_t cell = cell_key(0, r, b, a.n_blocks, a.h_kv);
    ib = a.item_off[cell];
    ie = a.item_off[cell + 1];
  }
  if (ie - ib == 1) return;
  for (int e = threadIdx.x; e < kBlock * D / 4; e += 256) {
    const int key = e / (D / 4), d0 = 4 * (e % (D / 4));
    const int key_abs = b * kBlock + key;
    if (key_abs >= a.n_kv) continue;
    f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    for (int it = ib; it < ie; ++it) {
      sk += *reinterpret_cast<const f32x4*>(a.part_dkv + (((size_t)it * 2 + 0) * kBlock + key) * D + d0);
      sv += *reinterpret_cast<const f32x4*>(a.part_dkv + (((size_t)it * 2 + 1) * kBlock + key) * D + d0);
    }
    const size_t o = ((size_t)key_abs * a.h_kv + r) * D + d0;
    store4<bf16_t>(static_cast<bf16_t*>(a.dk) + o, sk[0], sk[1], sk[2], sk[3]);
    store4<bf16_t>(static_cast<bf16_t*>(a.dv) + o, sv[0], sv[1], sv[2], sv[3]);
  }
}

// ------------------------------------------------------ KL-alignment term
// For each query and group over the visible keys T of its selected blocks:
//   target p_main(j)  (group mean of the main-branch softmax, written in fp32
//                      by the dQ pass), prediction p_idx(j) = softmax_T(S_idx),
//   S_idx(j) = q_idx . k_idx_j * idx_scale,
//   KL = sum_j p_main (ln p_main - S_idx + lse_idx),
//   dS_idx(j) = kl_scale (p_idx(j) - p_main(j)),
//   dq_idx = idx_scale sum_j dS_idx(j) k_idx_j,  dk_idx_j = idx_scale sum dS_idx q_idx.
// Every per-key quantity is formed in fp32 before it is summed (p_idx and
// p_main nearly coincide when the branches agree, so the gradient and the
// KL are small differences and must not be taken between large sums).
// Index passes (KV-outer over the dQ pass's windows, one wave per item, 32
// tokens per MFMA tile): phase 0 writes each (token, slot)'s block max and
// sum of exp(S_idx - max), merged into lse_idx; phase 1 writes the block's
// KL terms and U = sum_j (p_idx - p_main) k_idx_j, merged into KL and dq_idx.
// A third pass (ordered single-window schedule, keys on lanes) accumulates
// dk_idx per block; a reduce sums a block's items over all groups (k_idx is
// shared by the groups).
constexpr int kKlWaves = 4;

template <int DI>
struct KlLds {
  static constexpr int TS = 128 * 2 + 8;  // bytes per d row of K_idx^T
  static constexpr int WAVE = DI * TS;
};

template <int DI>
__device__ __forceinline__ float* kl_part(const KbArgs& a, size_t slot) {
  return a.part_kl + slot * (8 + DI);
}

template <int DI, int PHASE>
__global__ __launch_bounds__(kKlWaves * 64) void kl_index_kernel(KbArgs a) {
  using L = KlLds<DI>;
  __shared__ __attribute__((aligned(16))) char lds[PHASE == 1 ? kKlWaves : 1][PHASE == 1 ? L::WAVE : 16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  char* kt_lds = lds[PHASE == 1 ? wave : 0];
  const int64_t n_l = (int64_t)a.h_kv * a.n_blocks;
  const int item_begin = scalar_load(a.item_off, (int64_t)a.w * n_l);
  const int item_end = scalar_load(a.item_off, (int64_t)(a.w + 1) * n_l);
  const bf16_t* kidx = static_cast<const bf16_t*>(a.k_idx);
  const bf16_t* qidx = static_cast<const bf16_t*>(a.q_idx);
  for (int it = item_begin + blockIdx.x * kKlWaves + wave; it < item_end; it += gridDim.x * kKlWaves) {
    const i32x4 d = scalar_load(a.items, __builtin_amdgcn_readfirstlane(it));
    const int b = d[0], r = d[1], e0 = d[2], n_tok = d[3] - d[2];
    const int last = min(kBlock, a.n_kv - b * kBlock) - 1;
    if constexpr (PHASE == 1) {
      // K_idx^T of block b into this wave's LDS: pairs of keys interleaved
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < DI / 8; ++i) {
        const int u = lane + 64 * i;
        const int dc = u % (DI / 8), kp = u / (DI / 8);
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(kidx + ((size_t)b * kBlock + min(2 * kp, last)) * DI + dc * 8);
        const u32x4 y0 =
            *reinterpret_cast<const u32x4*>(kidx + ((size_t)b * kBlock + min(2 * kp + 1, last)) * DI + dc * 8);
        const u32x4 x = 2 * kp > last ? z : x0;
        const u32x4 y = 2 * kp + 1 > last ? z : y0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          *reinterpret_cast<uint32_t*>(kt_lds + (8 * dc + 2 * t) * L::TS + kp * 4) = (x[t] & 0xffffu) | (y[t] << 16);
          *reinterpret_cast<uint32_t*>(kt_lds + (8 * dc + 2 * t + 1) * L::TS + kp * 4) =
              (x[t] >> 16) | (y[t] & 0xffff0000u);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    for (int t0 = 0; t0 < n_tok; t0 += 32) {
      const bool ok = t0 + l32 < n_tok;
      const int ent = a.entries[e0 + min(t0 + l32, n_tok - 1)];
      const int i = ent >> 4, j = ent & 15;
      const int pos = ok ? a.q_start + i : -1;
      const size_t slot = ok ? ((size_t)(i - a.w * a.window) * a.h_kv + r) * a.top_k + j : a.trash_slot;
      bf16x8 qf[DI / 16];
#pragma unroll
      for (int ks = 0; ks < DI / 16; ++ks)
        qf[ks] = load_frag<bf16_t>(qidx + ((size_t)i * a.h_kv + r) * DI + ks * 16 + half * 8);
      // S_idx^T = K_idx . q_idx^T (keys on the MFMA rows, tokens on lanes);
      // this lane holds keys kt*32 + 8c + 4*half + q of its token
      f32x16 sc[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        sc[kt] = f32x16{};
        const bf16_t* krow = kidx + ((size_t)b * kBlock + min(kt * 32 + l32, last)) * DI + half * 8;
#pragma unroll
        for (int ks = 0; ks < DI / 16; ++ks) mma32(sc[kt], load_frag<bf16_t>(krow + ks * 16), qf[ks]);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = b * kBlock + kt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          sc[kt][v] = key > pos ? -__builtin_inff() : sc[kt][v] * a.idx_scale;
        }
      }
      float* dst = kl_part<DI>(a, slot);
      if constexpr (PHASE == 0) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kt][v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mc = mx == -__builtin_inff() ? 0.0f : mx;
        float sl = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) sl += fast_exp2((sc[kt][v] - mc) * kLog2e);
        sl += __shfl_xor(sl, 32, 64);
        *reinterpret_cast<f32x2*>(dst) = f32x2{mx, sl};
      } else {
        const float lse = a.lse_idx[(size_t)i * a.h_kv + r];
        const float* pmrow = a.pmain + (((size_t)i * a.h_kv + r) * a.top_k + j) * kBlock + 4 * half;
        float klt = 0.f;
        bf16x8 df[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          float dv[16];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const f32x4 p4 = *reinterpret_cast<const f32x4*>(pmrow + kt * 32 + 8 * c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int v = 4 * c + q;
              const float lp = sc[kt][v] - lse;  // ln p_idx (-inf where masked)
              const float pi = fast_exp2(lp * kLog2e);
              const float pm = ok ? p4[q] : 0.0f;
              dv[v] = pi - pm;
              klt += pm > 0.0f ? pm * (__logf(pm) - lp) : 0.0f;
            }
          }
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int o = 8 * h2;
            df[kt][h2] = to_frag<bf16_t>(dv[o], dv[o + 1], dv[o + 2], dv[o + 3], dv[o + 4], dv[o + 5], dv[o + 6],
                                         dv[o + 7]);
          }
        }
        klt += __shfl_xor(klt, 32, 64);
        // U^T = K_idx^T . (p_idx - p_main)^T (d_idx on the MFMA rows)
        f32x16 u[DI / 32];
#pragma unroll
        for (int dt = 0; dt < DI / 32; ++dt) u[dt] = f32x16{};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int base = kt * 32 + h2 * 16;
#pragma unroll
            for (int dt = 0; dt < DI / 32; ++dt)
              mma32(u[dt], vt_frag<bf16_t>(kt_lds, L::TS, dt * 32 + l32, base + 4 * half, base + 8 + 4 * half),
                    df[kt][h2]);
          }
        dst[0] = klt;
#pragma unroll
        for (int dt = 0; dt < DI / 32; ++dt)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int d0 = dt * 32 + 8 * c + 4 * half;
            *reinterpret_cast<f32x4*>(dst + 8 + d0) =
                f32x4{u[dt][4 * c], u[dt][4 * c + 1], u[dt][4 * c + 2], u[dt][4 * c + 3]};
          }
      }
    }
    __builtin_amdgcn_wave_barrier();  // this wave's LDS is rewritten for its next item
  }
}

// Row merges of window w.  Phase 0: lse_idx of every (token, group).
// Phase 1: KL and dq_idx.
template <int DI, int PHASE>
__global__ __launch_bounds__(256) void kl_merge_kernel(KbArgs a) {
  constexpr int DC = PHASE == 0 ? 1 : DI / 8;
  const int64_t t = blockIdx.x * 256ll + threadIdx.x;
  const int64_t rl = t / DC;  // il * h_kv + r
  const int c = (int)(t % DC);
  const int il = (int)(rl / a.h_kv), r = (int)(rl % a.h_kv);
  const int i = a.w * a.window + il;
  if (il >= a.window || i >= a.n_q) return;
  const int diag = (a.q_start + i) >> 7;
  const uint32_t used = used_slots(a.block_idx + ((size_t)i * a.h_kv + r) * a.top_k, a.top_k, diag);
  const size_t slot0 = ((size_t)il * a.h_kv + r) * a.top_k;
  if constexpr (PHASE == 0) {
    float mm = -__builtin_inff();
    for (int j = 0; j < a.top_k; ++j)
      if ((used >> j) & 1u) mm = fmaxf(mm, kl_part<DI>(a, slot0 + j)[0]);
    float ll = 0.f;
    for (int j = 0; j < a.top_k; ++j)
      if ((used >> j) & 1u) {
        const float* p = kl_part<DI>(a, slot0 + j);
        ll += p[1] * __expf(p[0] - mm);
      }
    a.lse_idx[(size_t)i * a.h_kv + r] = used ? mm + __logf(ll) : 0.0f;
  } else {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float klv = 0.f;
    for (int j = 0; j < a.top_k; ++j)
      if ((used >> j) & 1u) {
        const float* p = kl_part<DI>(a, slot0 + j);
        klv += p[0];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += p[8 + c * 8 + e];
      }
    const float g = a.idx_scale * a.kl_scale;
    bf16_t* dst = static_cast<bf16_t*>(a.dq_idx) + ((size_t)i * a.h_kv + r) * DI + c * 8;
    *reinterpret_cast<bf16x8*>(dst) =
        bf16x8{from_f32<bf16_t>(g * acc[0]), from_f32<bf16_t>(g * acc[1]), from_f32<bf16_t>(g * acc[2]),
               from_f32<bf16_t>(g * acc[3]), from_f32<bf16_t>(g * acc[4]), from_f32<bf16_t>(g * acc[5]),
               from_f32<bf16_t>(g * acc[6]), from_f32<bf16_t>(g * acc[7])};
    if (c == 0 && a.kl) a.kl[(size_t)i * a.h_kv + r] = klv;
  }
}

// dk_idx pass: items of the ordered single-window schedule from a work queue;
// wave w owns keys 32w .. 32w + 31 of the block, tokens go in tiles of 32.
template <int DI>
struct KlDkLds {
  static constexpr int QS = DI * 2 + 16;   // bytes per token row of q_idx
  static constexpr int TS = 32 * 2 + 8;    // bytes per d row of a 32-token q_idx^T tile
  static constexpr int Q_R = 0;
  static constexpr int Q_T = 32 * QS;
  static constexpr int SC = Q_T + DI * TS;     // lse_idx, pos, pmain row (int64 as 2 ints) per token
  static constexpr int BYTES = SC + 32 * 16;
  static constexpr int ENT_OFF = BYTES;
  static constexpr int TOTAL = ENT_OFF + 2048 * 4;
};

template <int DI>
__global__ __launch_bounds__(256) void kl_dk_kernel(KbArgs a) {
  using L = KlDkLds<DI>;
  __shared__ __attribute__((aligned(16))) char lds[L::TOTAL];
  __shared__ int next_item;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int n_items = scalar_load(a.item_off, (int64_t)a.h_kv * a.n_blocks);
  int* ent_lds = reinterpret_cast<int*>(lds + L::ENT_OFF);
  const bf16_t* kidx = static_cast<const bf16_t*>(a.k_idx);
  const bf16_t* qidx = static_cast<const bf16_t*>(a.q_idx);
  for (;;) {
    if (tid == 0) next_item = atomicAdd(a.queue + 1, 1);
    __syncthreads();
    const int it = next_item;
    if (it >= n_items) break;
    const i32x4 d = scalar_load(a.items, __builtin_amdgcn_readfirstlane(it));
    const int b = d[0], r = d[1], e0 = d[2], n_tok = d[3] - d[2];
    for (int e = tid; e < n_tok; e += 256) ent_lds[e] = a.entries[e0 + e] >> 4;
    const int last = min(kBlock, a.n_kv - b * kBlock) - 1;
    const int key_l = wave * 32 + l32;
    const int key_abs = b * kBlock + key_l;
    bf16x8 kf[DI / 16];
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks)
      kf[ks] = load_frag<bf16_t>(kidx + ((size_t)b * kBlock + min(key_l, last)) * DI + ks * 16 + half * 8);
    f32x16 dk[DI / 32];
#pragma unroll
    for (int dt = 0; dt < DI / 32; ++dt) dk[dt] = f32x16{};
    __syncthreads();
    for (int t0 = 0; t0 < n_tok; t0 += 32) {
      // stage the tile: q_idx rows and q_idx^T, and per token lse_idx, pos, pmain row
      {
        constexpr int DC = DI / 8;
        for (int u = tid; u < 16 * DC; u += 256) {
          const int dc = u % DC, rp = u / DC;
          const int ia = ent_lds[min(t0 + 2 * rp, n_tok - 1)], ib = ent_lds[min(t0 + 2 * rp + 1, n_tok - 1)];
          const u32x4 x = *reinterpret_cast<const u32x4*>(qidx + ((size_t)ia * a.h_kv + r) * DI + dc * 8);
          const u32x4 y = *reinterpret_cast<const u32x4*>(qidx + ((size_t)ib * a.h_kv + r) * DI + dc * 8);
          *reinterpret_cast<u32x4*>(lds + L::Q_R + (2 * rp) * L::QS + dc * 16) = x;
          *reinterpret_cast<u32x4*>(lds + L::Q_R + (2 * rp + 1) * L::QS + dc * 16) = y;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            *reinterpret_cast<uint32_t*>(lds + L::Q_T + (8 * dc + 2 * t) * L::TS + rp * 4) = (x[t] & 0xffffu) | (y[t] << 16);
            *reinterpret_cast<uint32_t*>(lds + L::Q_T + (8 * dc + 2 * t + 1) * L::TS + rp * 4) =
                (x[t] >> 16) | (y[t] & 0xffff0000u);
          }
        }
        if (tid < 32) {
          const bool ok = t0 + tid < n_tok;
          const int i = ent_lds[min(t0 + tid, n_tok - 1)];
          const int32_t* br = a.block_idx + ((size_t)i * a.h_kv + r) * a.top_k;
          int j = 0;
          for (int s = 0; s < a.top_k; ++s) j = br[s] == b ? s : j;
          int* sc = reinterpret_cast<int*>(lds + L::SC) + 4 * tid;
          reinterpret_cast<float*>(sc)[0] = a.lse_idx[(size_t)i * a.h_kv + r];
          sc[1] = ok ? a.q_start + i : -1;
          const int64_t row = ((int64_t)i * a.h_kv + r) * a.top_k + j;
          sc[2] = (int)(row & 0xffffffff);
          sc[3] = (int)(row >> 32);
        }
      }
      __syncthreads();
      // S_idx = q_idx . K_idx^T (tokens on the MFMA rows, this wave's keys on lanes)
      f32x16 s = {};
#pragma unroll
      for (int ks = 0; ks < DI / 16; ++ks)
        mma32(s, *reinterpret_cast<const bf16x8*>(lds + L::Q_R + l32 * L::QS + (ks * 16 + half * 8) * 2), kf[ks]);
      float dsv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * half + (v & 3);
        const int* sc = reinterpret_cast<const int*>(lds + L::SC) + 4 * row;
        const float lse = reinterpret_cast<const float*>(sc)[0];
        const int pos = sc[1];
        const int64_t prow = (int64_t)(uint32_t)sc[2] | ((int64_t)sc[3] << 32);
        const bool vis = key_abs <= pos;
        const float pi = fast_exp2(vis ? (s[v] * a.idx_scale - lse) * kLog2e : -__builtin_inff());
        const float pm = a.pmain[prow * kBlock + key_l];
        dsv[v] = vis ? a.kl_scale * (pi - pm) : 0.0f;
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int o = 8 * h2;
        const bf16x8 f = to_frag<bf16_t>(dsv[o], dsv[o + 1], dsv[o + 2], dsv[o + 3], dsv[o + 4], dsv[o + 5],
                                         dsv[o + 6], dsv[o + 7]);
#pragma unroll
        for (int dt = 0; dt < DI / 32; ++dt)
          mma32(dk[dt], vt_frag<bf16_t>(lds + L::Q_T, L::TS, dt * 32 + l32, 16 * h2 + 4 * half, 16 * h2 + 8 + 4 * half),
                f);
      }
      __syncthreads();
    }
    float* dst = a.part_dki + ((size_t)it * kBlock + key_l) * DI;
#pragma unroll
    for (int dt = 0; dt < DI / 32; ++dt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = dt * 32 + 8 * c + 4 * half;
        *reinterpret_cast<f32x4*>(dst + d0) = f32x4{dk[dt][4 * c] * a.idx_scale, dk[dt][4 * c + 1] * a.idx_scale,
                                                    dk[dt][4 * c + 2] * a.idx_scale, dk[dt][4 * c + 3] * a.idx_scale};
      }
  }
}

// dk_idx of block b: the sum of the items of every group's cell (b, r).
template <int DI>
__global__ __launch_bounds__(256) void kl_dk_reduce_kernel(KbArgs a) {
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < kBlock * DI / 4; e += 256) {
    const int key = e / (DI / 4), d0 = 4 * (e % (DI / 4));
    const int key_abs = b * kBlock + key;
    if (key_abs >= a.n_kv) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (b < a.n_blocks)
      for (int r = 0; r < a.h_kv; ++r) {
        const int64_t cell = cell_key(0, r, b, a.n_blocks, a.h_kv);
        const int ib = a.item_off[cell], ie = a.item_off[cell + 1];
        for (int it = ib; it < ie; ++it)
          acc += *reinterpret_cast<const f32x4*>(a.part_dki + ((size_t)it * kBlock + key) * DI + d0);
      }
    store4<bf16_t>(static_cast<bf16_t*>(a.dk_idx) + (size_t)key_abs * DI + d0, acc[0], acc[1], acc[2], acc[3]);
  }
}

// ------------------------------------------------------------------- host
bool backward_supported(int dtype, int d_h) { return dtype == 0 && (d_h == 64 || d_h == 128); }

BackwardPlan backward_plan(int32_t n_q, int32_t q_start, int32_t n_kv, int32_t h_q, int32_t h_kv, int32_t d_h,
                           int32_t top_k, int32_t d_idx, bool with_kl) {
  BackwardPlan p{};
  const int G = h_q / h_kv;
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  // dQ pass: the forward's windows (its partials are fp32 here)
  p.q = prefill_plan(1, n_q, q_start, n_kv, h_q, h_kv, d_h, top_k);
  p.q.total = p.q.off_part_o;  // schedule arrays only
  // dK/dV pass: one window; items of up to KbkvLds::ENT_CAP tokens
  schedule_layout(p.kv, n_q, q_start, h_kv, top_k, std::max<int32_t>(n_q, 1), KbkvLds<128>::ENT_CAP,
                  /*ordered=*/true);
  size_t off = 0;
  p.off_q = off; off = align(off + p.q.total);
  p.off_kv = off; off = align(off + p.kv.total);
  p.off_dsum = off; off = align(off + (size_t)n_q * h_q * 4);
  p.off_part_dq = off; off = align(off + ((size_t)p.q.window * h_kv * top_k + 2) * G * d_h * 2);
  p.off_part_dkv = off; off = align(off + (size_t)p.kv.max_items * 2 * kBlock * d_h * 4);
  if (with_kl) {
    p.off_pmain = off; off = align(off + ((size_t)n_q * h_kv * top_k + 1) * kBlock * 4);
    p.off_part_kl = off; off = align(off + ((size_t)p.q.window * h_kv * top_k + 1) * (8 + d_idx) * 4);
    p.off_lse_idx = off; off = align(off + (size_t)n_q * h_kv * 4);
    p.off_part_dki = off; off = align(off + (size_t)p.kv.max_items * kBlock * d_idx * 4);
  }
  p.total = off;
  return p;
}

template <int DI>
static void launch_kl_index_typed(const KbArgs& k, unsigned grid, int64_t rows, hipStream_t st) {
  hipLaunchKernelGGL((kl_index_kernel<DI, 0>), dim3(grid), dim3(kKlWaves * 64), 0, st, k);
  hipLaunchKernelGGL((kl_merge_kernel<DI, 0>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, k);
  hipLaunchKernelGGL((kl_index_kernel<DI, 1>), dim3(grid), dim3(kKlWaves * 64), 0, st, k);
  hipLaunchKernelGGL((kl_merge_kernel<DI, 1>), dim3((unsigned)((rows * (DI / 8) + 255) / 256)), dim3(256), 0, st, k);
}

static void launch_kl_index(int d_idx, const KbArgs& k, unsigned grid, int64_t rows, hipStream_t st) {
  if (d_idx == 32) launch_kl_index_typed<32>(k, grid, rows, st);
  else if (d_idx == 64) launch_kl_index_typed<64>(k, grid, rows, st);
  else launch_kl_index_typed<128>(k, grid, rows, st);
}

static void launch_kl_dk(int d_idx, const KbArgs& k, unsigned grid, unsigned nb_kv, hipStream_t st) {
  if (d_idx == 32) {
    hipLaunchKernelGGL(kl_dk_kernel<32>, dim3(grid), dim3(256), 0, st, k);
    hipLaunchKernelGGL(kl_dk_reduce_kernel<32>, dim3(nb_kv), dim3(256), 0, st, k);
  } else if (d_idx == 64) {
    hipLaunchKernelGGL(kl_dk_kernel<64>, dim3(grid), dim3(256), 0, st, k);
    hipLaunchKernelGGL(kl_dk_reduce_kernel<64>, dim3(nb_kv), dim3(256), 0, st, k);
  } else {
    hipLaunchKernelGGL(kl_dk_kernel<128>, dim3(grid), dim3(256), 0, st, k);
    hipLaunchKernelGGL(kl_dk_reduce_kernel<128>, dim3(nb_kv), dim3(256), 0, st, k);
  }
}

static void launch_kl_dk_reduce(int d_idx, const KbArgs& k, unsigned nb_kv, hipStream_t st) {
  if (d_idx == 32) hipLaunchKernelGGL(kl_dk_reduce_kernel<32>, dim3(nb_kv), dim3(256), 0, st, k);
  else if (d_idx == 64) hipLaunchKernelGGL(kl_dk_reduce_kernel<64>, dim3(nb_kv), dim3(256), 0, st, k);
  else hipLaunchKernelGGL(kl_dk_reduce_kernel<128>, dim3(nb_kv), dim3(256), 0, st, k);
}

template <int D>
static hipError_t backward_typed(const BackwardArgs& ba, const BackwardPlan& pl, hipStream_t st) {
  const AttnArgs& a = ba.attn;
  char* ws = static_cast<char*>(a.ws);
  KbArgs k{};
  k.q = a.q;
  k.k = a.k;
  k.v = a.v;
  k.o = a.o;
  k.lse = a.lse;
  k.d_o = ba.d_o;
  k.dq = ba.dq;
  k.dk = ba.dk;
  k.dv = ba.dv;
  k.dsum = reinterpret_cast<float*>(ws + pl.off_dsum);
  k.block_idx = a.block_idx;
  k.part_dq = reinterpret_cast<bf16_t*>(ws + pl.off_part_dq);
  k.part_dkv = reinterpret_cast<float*>(ws + pl.off_part_dkv);
  if (ba.kl) {
    k.pmain = reinterpret_cast<float*>(ws + pl.off_pmain);
    k.part_kl = reinterpret_cast<float*>(ws + pl.off_part_kl);
    k.lse_idx = reinterpret_cast<float*>(ws + pl.off_lse_idx);
    k.part_dki = reinterpret_cast<float*>(ws + pl.off_part_dki);
    k.q_idx = ba.q_idx;
    k.k_idx = ba.k_idx;
    k.kl = ba.kl_out;
    k.dq_idx = ba.dq_idx;
    k.dk_idx = ba.dk_idx;
    k.idx_scale = ba.idx_scale;
    k.kl_scale = ba.kl_scale;
  }
  k.n_q = a.n_q;
  k.q_start = a.q_start;
  k.n_kv = a.n_kv;
  k.h_q = a.h_q;
  k.h_kv = a.h_kv;
  k.group = a.group;
  k.g_shift = __builtin_ctz((unsigned)a.group);
  k.top_k = a.top_k;
  k.sm_scale = a.sm_scale;

  const unsigned nb_kv = (unsigned)((a.n_kv + kBlock - 1) / kBlock);
  if (a.n_q == 0) {  // no query attends: dK = dV = 0 (and dk_idx = 0)
    k.n_blocks = 0;
    if (nb_kv > 0) {
      hipLaunchKernelGGL(kbkv_reduce_kernel<D>, dim3(nb_kv, (unsigned)a.h_kv), dim3(256), 0, st, k);
      if (ba.kl) launch_kl_dk_reduce(ba.d_idx, k, nb_kv, st);
    }
    return hipGetLastError();
  }
  const int64_t rows = (int64_t)a.n_q * a.h_q;
  hipLaunchKernelGGL(kb_dsum_kernel<D>, dim3((unsigned)((rows * (D / 8) + 255) / 256)), dim3(256), 0, st, k);

  // dQ: windows of the forward's schedule
  AttnArgs aq = a;
  aq.ws = ws + pl.off_q;
  SchedArgs sq;
  hipError_t e = launch_prefill_schedule(aq, pl.q, sq, st);
  if (e != hipSuccess) return e;
  k.item_off = sq.item_off;
  k.entries = sq.entries;
  k.items = sq.items;
  k.n_blocks = pl.q.n_blocks;
  k.window = pl.q.window;
  k.trash_slot = (size_t)pl.q.window * a.h_kv * a.top_k;
  const int n_cu = num_cus();
  for (int w = 0; w < pl.q.n_windows; ++w) {
    const int tok = std::min<int>(pl.q.window, a.n_q - w * pl.q.window);
    const int64_t bound = (int64_t)tok * a.h_kv * a.top_k / pl.q.chunk + (int64_t)a.h_kv * pl.q.n_blocks + 1;
    const int64_t g = std::min<int64_t>(bound + 8, (int64_t)n_cu);
    const unsigned grid = (unsigned)std::max<int64_t>(8, (g + 7) & ~int64_t(7));
    k.w = w;
    const int pk = profile_begin(PK_KBQ, st);
    if (k.pmain)
      hipLaunchKernelGGL((kbq_kernel<D, true>), dim3(grid), dim3(kKbqThreads), 0, st, k);
    else
      hipLaunchKernelGGL((kbq_kernel<D, false>), dim3(grid), dim3(kKbqThreads), 0, st, k);
    profile_end(pk, st);
    const int64_t mrows = (int64_t)tok * a.h_q;
    hipLaunchKernelGGL(kbq_merge_kernel<D>, dim3((unsigned)((mrows * (D / 8) + 255) / 256)), dim3(256), 0, st, k);
    if (ba.kl) {
      k.trash_slot = (size_t)pl.q.window * a.h_kv * a.top_k;
      launch_kl_index(ba.d_idx, k, (unsigned)(2 * n_cu), (int64_t)tok * a.h_kv, st);
    }
  }

  // dK/dV: one window over all queries
  AttnArgs akv = a;
  akv.ws = ws + pl.off_kv;
  SchedArgs skv;
  e = launch_prefill_schedule(akv, pl.kv, skv, st);
  if (e != hipSuccess) return e;
  k.item_off = skv.item_off;
  k.entries = skv.entries;
  k.items = skv.items;
  k.queue = skv.fill;
  k.n_blocks = pl.kv.n_blocks;
  k.window = pl.kv.window;
  k.w = 0;
  const int pk = profile_begin(PK_KBKV, st);
  hipLaunchKernelGGL(kbkv_kernel<D>, dim3((unsigned)n_cu), dim3(kKbkvThreads), 0, st, k);
  profile_end(pk, st);
  if (nb_kv > 0)
    hipLaunchKernelGGL(kbkv_reduce_kernel<D>, dim3(nb_kv, (unsigned)a.h_kv), dim3(256), 0, st, k);
  if (ba.kl && nb_kv > 0) launch_kl_dk(ba.d_idx, k, (unsigned)(2 * n_cu), nb_kv, st);
  return hipGetLastError();
}

hipError_t launch_sparse_prefill_backward(int d_h, const BackwardArgs& a, const BackwardPlan& pl, hipStream_t st) {
  if (d_h == 128) return backward_typed<128>(a, pl, st);
  if (d_h == 64) return backward_typed<64>(a, pl, st);
  return hipErrorInvalidValue;
}

}  // namespace msa
