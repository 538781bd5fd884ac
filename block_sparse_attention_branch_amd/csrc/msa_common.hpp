// msa_common.hpp - device-side building blocks shared by the libmsa kernels
// (gfx950 / CDNA4, wave64).
//
// Fragment convention used everywhere: an MFMA operand fragment is 8 values
// per lane.  For the 32x32 shapes lane l supplies row/col (l % 32) and the
// contraction indices 8*(l/32) + e, e = 0..7; for the 16x16 shapes lane l
// supplies row/col (l % 16) and contraction indices 8*(l/16) + e.  A bf16
// fragment feeds one v_mfma_f32_{32x32x16,16x16x32}_bf16; an fp32 fragment
// feeds eight v_mfma_f32_{32x32x2,16x16x4}_f32, instruction e contracting
// element e of every lane.  Because A and B use the same per-lane index map,
// any fixed permutation of the contraction index is harmless.
//
// Accumulator layouts (gfx9 MFMA):
//   32x32: acc[v] of lane l holds C[8*(v/4) + 4*(l/32) + (v%4)][l % 32]
//   16x16: acc[v] of lane l holds C[4*(l/16) + v][l % 16]
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

namespace msa {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;     // tokens per KV block / page
constexpr int kMaxTopK = 16;    // capacity of the per-row top-k lists
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- fragments
template <typename T> struct FragT;
template <> struct FragT<bf16_t> { typedef bf16x8 type; };
template <> struct FragT<float> { typedef f32x8 type; };
template <typename T> using Frag = typename FragT<T>::type;

template <typename T>
__device__ __forceinline__ Frag<T> load_frag(const T* p) {
  return *reinterpret_cast<const Frag<T>*>(p);
}
template <typename T>
__device__ __forceinline__ Frag<T> zero_frag() {
  Frag<T> z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = T(0.0f);
  return z;
}

__device__ __forceinline__ void mma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
}

// -------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f32(bf16_t x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return static_cast<bf16_t>(x); }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 8-bit cache entries: OCP e4m3 ("fn": bias 7, no infinities), 1 byte each,
// used as stored (no scale).  Every e4m3 value is exactly a bf16 value, so
// widening to bf16 loses nothing.
typedef uint8_t fp8_t;

// Eight e4m3 codes (byte e of the pair of dwords = element e) to bf16.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w[0], false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w[0], true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w[1], false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(w[1], true);
  return bf16x8{static_cast<bf16_t>(a[0]), static_cast<bf16_t>(a[1]), static_cast<bf16_t>(b[0]),
                static_cast<bf16_t>(b[1]), static_cast<bf16_t>(c[0]), static_cast<bf16_t>(c[1]),
                static_cast<bf16_t>(d[0]), static_cast<bf16_t>(d[1])};
}

// MXFP8 caches (the OCP microscaling format): E4M3 codes as above, plus one
// E8M0 scale byte per 32 consecutive elements of a row, value 2^(s - 127)
// (0xFF is NaN).  An E4M3 value times a power of two has at most 4
// significant bits, so the scaled value is still exact in bf16 whenever it
// lies in bf16's range.  mx8_t tags these caches; its codes are laid out and
// loaded exactly like fp8_t's, and every scale array has the layout of its
// cache with the last dimension divided by 32.
struct mx8_t {
  uint8_t code;
};
template <typename TC>
inline constexpr bool kIsMx = std::is_same<TC, mx8_t>::value;
constexpr int kMxBlock = 32;

__device__ __forceinline__ float e8m0_scale(uint32_t s) {
  return s == 0xFFu ? __builtin_nanf("") : (s == 0u ? 0x1p-127f : __builtin_bit_cast(float, s << 23));
}

// Eight e4m3 codes times one scale, to bf16 (exact, see above).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w, float sc) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w[0], false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w[0], true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w[1], false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(w[1], true);
  return bf16x8{static_cast<bf16_t>(a[0] * sc), static_cast<bf16_t>(a[1] * sc), static_cast<bf16_t>(b[0] * sc),
                static_cast<bf16_t>(b[1] * sc), static_cast<bf16_t>(c[0] * sc), static_cast<bf16_t>(c[1] * sc),
                static_cast<bf16_t>(d[0] * sc), static_cast<bf16_t>(d[1] * sc)};
}

// A cache fragment as loaded: 8 elements of the cache type, kept raw until
// the math needs them (so converting never waits on loads in flight).
template <typename TC> struct RawT;
template <> struct RawT<bf16_t> { typedef bf16x8 type; };
template <> struct RawT<float> { typedef f32x8 type; };
template <> struct RawT<fp8_t> { typedef u32x2 type; };
template <> struct RawT<mx8_t> { typedef u32x2 type; };
template <typename TC> using Raw = typename RawT<TC>::type;

template <typename TC>
__device__ __forceinline__ Raw<TC> load_raw(const TC* p) {
  return *reinterpret_cast<const Raw<TC>*>(p);
}
// Raw fragment -> compute fragment (T = bf16 for fp8 caches).
template <typename T, typename TC>
__device__ __forceinline__ Frag<T> widen(const Raw<TC>& r) {
  if constexpr (sizeof(TC) == 1) {
    return fp8x8_to_bf16(r);
  } else {
    return r;
  }
}
// Raw fragment and the E8M0 byte of its 32-element block -> compute fragment
// (the scale is ignored for caches without one).
template <typename T, typename TC>
__device__ __forceinline__ Frag<T> widen(const Raw<TC>& r, uint32_t scale_byte) {
  if constexpr (kIsMx<TC>) {
    return fp8x8_to_bf16(r, e8m0_scale(scale_byte));
  } else {
    return widen<T, TC>(r);
  }
}

// ------------------------------------------------------------ top-k keys
// A candidate block is packed into one 64-bit key whose unsigned order is the
// selection order: pooled score descending, then block index ascending.
// Key 0 means "empty slot" and loses to every real candidate.
__device__ __forceinline__ uint32_t order_f32(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unorder_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t make_key(float score, int32_t block) {
  return (static_cast<uint64_t>(order_f32(score)) << 32) |
         static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(block));
}
__device__ __forceinline__ int32_t key_block(uint64_t k) {
  return static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(k));
}
__device__ __forceinline__ float key_score(uint64_t k) {
  return unorder_f32(static_cast<uint32_t>(k >> 32));
}

// Insert v into the descending list `keys` (capacity L, unique keys).
// The caller checks v > keys[L-1]; the last entry falls off.  Slot s becomes
// max(keys[s], min(keys[s-1], v)): entries above v stay, v lands where the
// first smaller entry was, and the smaller ones shift down by one.  Every
// slot is computed from the old list, so there is no serial chain.
template <int L>
__device__ __forceinline__ void list_insert(uint64_t (&keys)[L], uint64_t v) {
  uint64_t prev = ~0ull;
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const uint64_t cur = keys[s];
    const uint64_t m = prev < v ? prev : v;
    keys[s] = cur > m ? cur : m;
    prev = cur;
  }
}

// Insert (v, b) into a list of scores sorted descending with their blocks
// (capacity L), where b comes after every listed block: an equal score stays
// ahead of v.  The caller checks v > sc[L-1]; the last entry falls off.  The
// new score of slot s is max(sc[s], min(sc[s-1], v)), the median of the
// three since sc[s] <= sc[s-1]; its block is the old one while sc[s] >= v,
// b where v lands, and the block of slot s-1 below that.  Every slot is
// computed from the old list, so there is no serial chain.
template <int L>
__device__ __forceinline__ void list_insert_later(float (&sc)[L], int (&id)[L], float v, int b) {
  // bottom up, so that each slot is overwritten after the slot below has
  // read it: the update stays in place
#pragma unroll
  for (int s = L - 1; s >= 0; --s) {
    const float up = s > 0 ? sc[s - 1] : __builtin_inff();
    const bool up_ge = s > 0 ? sc[s - 1] >= v : true;
    const int up_id = s > 0 ? id[s - 1] : b;
    id[s] = sc[s] >= v ? id[s] : (up_ge ? b : up_id);
    sc[s] = __builtin_amdgcn_fmed3f(sc[s], up, v);
  }
}

// Write one row's final index list: the `n_take` best keys of `keys`
// (descending, 0 = empty), plus `forced` (>= 0) if given, as ascending block
// ids padded with -1 to top_k; the pooled score of each id goes to `score_out`
// (nullable), forced_score for the forced block, -inf for padding.
template <int L>
__device__ __forceinline__ void write_row_list(const uint64_t (&keys)[L], int n_take, int forced,
                                               float forced_score, int top_k, int32_t* idx_out,
                                               float* score_out) {
  int32_t id[L + 1];
  float sc[L + 1];
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const bool ok = (s < n_take) && (keys[s] != 0ull);
    id[s] = ok ? key_block(keys[s]) : 0x7fffffff;
    sc[s] = ok ? key_score(keys[s]) : 0.0f;
  }
  id[L] = forced >= 0 ? forced : 0x7fffffff;
  sc[L] = forced_score;
  for (int t = 0; t < top_k; ++t) {
    idx_out[t] = -1;
    if (score_out) score_out[t] = -__builtin_inff();
  }
#pragma unroll
  for (int s = 0; s <= L; ++s) {
    int rank = 0;
#pragma unroll
    for (int t = 0; t <= L; ++t) rank += (id[t] < id[s]) ? 1 : 0;
    if (id[s] != 0x7fffffff && rank < top_k) {
      idx_out[rank] = id[s];
      if (score_out) score_out[rank] = sc[s];
    }
  }
}

// Uniform reads through the constant address space become scalar loads (they
// count against lgkmcnt, so they never wait for outstanding vector stores).
template <typename U>
__device__ __forceinline__ U scalar_load(const U* p, int64_t i) {
  typedef const __attribute__((address_space(4))) U* CP;
  return ((CP)p)[i];
}

// Keeps the scheduler from hoisting every unrolled LDS fragment load (or
// every MFMA of a loop nest) to the top, which costs registers and forces
// spills or accumulator-register traffic.
#ifndef MSA_NO_SCHED_FENCE
#define MSA_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
#else
#define MSA_SCHED_FENCE() do {} while (0)
#endif

// Waits here, once, for the load that produced `x`: an empty asm statement
// that reads it makes the compiler put the wait in front of it.  Without it
// the wait lands before x's first use inside a loop, and that wait then also
// drains, in every iteration, the prefetches issued earlier in the iteration.
template <typename V>
__device__ __forceinline__ void settle(const V& x) {
  static_assert(sizeof(V) % 4 == 0, "whole dwords");
  struct Words {
    uint32_t w[sizeof(V) / 4];
  };
  const Words d = __builtin_bit_cast(Words, x);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(V) / 4); ++i) asm volatile("" ::"v"(d.w[i]));
}

// --------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_xor_f32(float x, int mask) { return __shfl_xor(x, mask, 64); }

// x of lane `lane`, which must be the same in every lane (v_readlane; a
// shuffle would go through LDS).
__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace msa
