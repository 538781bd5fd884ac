// msa_api.hip - the C ABI of libmsa (declared in include/msa.h): argument
// validation, workspace layout and kernel dispatch.  Every check runs on the
// host before anything is launched; on failure the call returns a status,
// launches nothing and leaves the outputs untouched.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "msa.h"

#include <cstdlib>
#include "msa_internal.hpp"
#include "msa_profile.hpp"

namespace {

thread_local std::string g_last_error;

msa_status fail(msa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

msa_status ok() {
  g_last_error.clear();
  return MSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float idx_scale_of(const msa_shape& s) { return s.idx_scale > 0.f ? s.idx_scale : 1.0f / sqrtf((float)s.d_idx); }
float sm_scale_of(const msa_shape& s) { return s.sm_scale > 0.f ? s.sm_scale : 1.0f / sqrtf((float)s.d_h); }

// Checks common to every call.  `need_idx` / `need_attn` select the fields used.
msa_status check_shape(const msa_shape* s, bool need_idx, bool need_attn) {
  if (!s) return fail(MSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->h_q <= 0 || s->h_kv <= 0) return fail(MSA_ERR_INVALID_ARG, "h_q=%d h_kv=%d must be > 0", s->h_q, s->h_kv);
  if (s->h_q % s->h_kv != 0) return fail(MSA_ERR_INVALID_ARG, "h_q=%d is not a multiple of h_kv=%d", s->h_q, s->h_kv);
  const int G = s->h_q / s->h_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(MSA_ERR_UNSUPPORTED, "heads per group h_q/h_kv=%d not in {1,2,4,8,16}", G);
  if (s->block_size != MSA_BLOCK_SIZE) return fail(MSA_ERR_UNSUPPORTED, "block_size=%d, only 128 is built", s->block_size);
  if (s->dtype != MSA_BF16 && s->dtype != MSA_FP32) return fail(MSA_ERR_INVALID_ARG, "dtype=%d is not a msa_dtype", s->dtype);
  if (s->top_k < 1 || s->top_k > MSA_MAX_TOP_K) return fail(MSA_ERR_UNSUPPORTED, "top_k=%d not in [1,16]", s->top_k);
  if (s->force_local != 0 && s->force_local != 1) return fail(MSA_ERR_INVALID_ARG, "force_local=%d must be 0 or 1", s->force_local);
  if (!(s->sm_scale >= 0.f) || !(s->idx_scale >= 0.f))
    return fail(MSA_ERR_INVALID_ARG, "sm_scale=%g idx_scale=%g must be >= 0 (0 = default)", s->sm_scale, s->idx_scale);
  if (need_idx && s->pool != MSA_POOL_MAX && s->pool != MSA_POOL_MEAN)
    return fail(MSA_ERR_INVALID_ARG, "pool=%d is not a msa_pool", s->pool);
  if (need_idx && !msa::ki_supported(s->dtype, s->d_idx))
    return fail(MSA_ERR_UNSUPPORTED, "d_idx=%d not in {32,64,128}", s->d_idx);
  if (need_attn && !msa::attn_supported(s->dtype, s->d_h))
    return fail(MSA_ERR_UNSUPPORTED, "d_h=%d not in {64,128}", s->d_h);
  return MSA_OK;
}

bool mx_cache(const msa_shape& s) { return s.cache_dtype == MSA_MXFP8_E4M3; }
bool fp8_cache(const msa_shape& s) { return s.cache_dtype == MSA_FP8_E4M3 || mx_cache(s); }

// 8-bit caches (e4m3, MXFP8): bf16 compute only; every call but the dense
// comparison, the backward and the projections.
msa_status check_cache_dtype(const msa_shape& s, bool allowed) {
  if (!fp8_cache(s)) return MSA_OK;
  if (s.dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "8-bit (e4m3, MXFP8) caches need dtype MSA_BF16");
  if (!allowed)
    return fail(MSA_ERR_UNSUPPORTED,
                "8-bit (e4m3, MXFP8) caches are not built for the dense comparison, the backward or the projections");
  return MSA_OK;
}

// MXFP8 caches: the scale arrays the call reads must be given.
msa_status check_scales(const msa_shape& s, const msa_kv* kv, bool need_idx, bool need_kv) {
  if (!mx_cache(s)) return MSA_OK;
  if (need_idx && !kv->k_idx_scale) return fail(MSA_ERR_INVALID_ARG, "MXFP8 caches: kv->k_idx_scale is NULL");
  if (need_kv && (!kv->k_scale || !kv->v_scale))
    return fail(MSA_ERR_INVALID_ARG, "MXFP8 caches: kv->k_scale/v_scale is NULL");
  if ((need_idx && !aligned16(kv->k_idx_scale)) || (need_kv && (!aligned16(kv->k_scale) || !aligned16(kv->v_scale))))
    return fail(MSA_ERR_INVALID_ARG, "MXFP8 caches: scale arrays must be 16-byte aligned");
  return MSA_OK;
}

// Kernel dispatch code: 0 bf16, 1 fp32, 2 bf16 with e4m3 caches, 3 bf16 with
// MXFP8 caches.
int kernel_dtype(const msa_shape& s) { return mx_cache(s) ? 3 : (fp8_cache(s) ? 2 : s.dtype); }

msa_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MSA_OK;
  if (!ws) return fail(MSA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(MSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(MSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return MSA_OK;
}

msa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t ki_prefill_ws(const msa_shape& s, int32_t n_q, int32_t q_start, int need_diag) {
  const msa::KiPlan p = msa::ki_prefill_plan(n_q, s.h_kv, q_start, need_diag);
  if (p.n_chunks <= 1) return 0;
  const size_t keys = (size_t)p.n_rows * p.n_chunks * 16 * 8;
  return ((keys + 255) & ~size_t(255)) + (((size_t)p.n_rows * 4 + 255) & ~size_t(255));
}

// Decode mode of msa_index_topk after its checks: the paged scan writes the
// pooled score of every page to `scores` [batch, h_kv, max_pages], then the
// select reads them back.
msa_status launch_index_decode(const msa_shape& s, int32_t batch, const void* q_idx, const msa_kv* kv,
                               int32_t* block_idx, float* block_score, float* scores, hipStream_t stream,
                               const char* what) {
  msa::KiDecodeArgs a{};
  a.q_idx = q_idx;
  a.k_idx = kv->k_idx;
  a.k_idx_scale = mx_cache(s) ? kv->k_idx_scale : nullptr;
  a.page_table = kv->page_table;
  a.seq_lens = kv->seq_lens;
  a.batch = batch;
  a.h_kv = s.h_kv;
  a.max_pages = kv->max_pages;
  a.pages_per_wg = msa::kKiDecodePagesPerWg;
  a.idx_scale = idx_scale_of(s);
  a.force_local = s.force_local;
  a.pool = s.pool;
  a.top_k = s.top_k;
  // the diagonal block is scored when its pooled score is reported or when it
  // competes as an ordinary candidate
  a.need_diag = (block_score != nullptr || !s.force_local) ? 1 : 0;
  a.scores = scores;
  a.block_idx = block_idx;
  a.block_score = block_score;
  return hip_status(msa::launch_ki_decode(kernel_dtype(s), s.d_idx, a, stream), what);
}

}  // namespace

// --------------------------------------------------- allocation-free variant
// msa_index_topk_decode_static keeps the pooled page scores of the decode
// index call in this array instead of a caller workspace: every GPU the
// library runs on holds its own copy (16 MiB) until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device.
static constexpr size_t kScratchFloats = size_t(1) << 22;
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with the device current).
msa_status scratch_address(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MSA_ERR_UNSUPPORTED, "device %d: only devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

msa_status msa_index_topk_decode_static(const msa_shape* shape, int32_t batch, const void* q_idx, const msa_kv* kv,
                                        int32_t* block_idx, float* block_score, void* hip_stream) {
  msa_status st = check_shape(shape, true, false);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if (!kv) return fail(MSA_ERR_INVALID_ARG, "kv is NULL");
  if (batch < 0) return fail(MSA_ERR_INVALID_ARG, "batch=%d", batch);
  if (!kv->k_idx) return fail(MSA_ERR_INVALID_ARG, "kv->k_idx is NULL");
  if (!aligned16(q_idx) || !aligned16(kv->k_idx)) return fail(MSA_ERR_INVALID_ARG, "q_idx/k_idx must be 16-byte aligned");
  if ((st = check_cache_dtype(s, true)) != MSA_OK) return st;
  if ((st = check_scales(s, kv, true, false)) != MSA_OK) return st;
  if (!kv->seq_lens || !kv->page_table) return fail(MSA_ERR_INVALID_ARG, "decode mode needs seq_lens and a page_table");
  if (kv->max_pages < 1 || kv->max_pages > msa::kMaxDecodePages)
    return fail(MSA_ERR_UNSUPPORTED, "max_pages=%d not in [1,%d]", kv->max_pages, msa::kMaxDecodePages);
  const size_t need = (size_t)batch * s.h_kv * kv->max_pages;
  if (need > kScratchFloats)
    return fail(MSA_ERR_UNSUPPORTED,
                "batch * h_kv * max_pages = %zu exceeds the %zu page scores of the built-in scratch; "
                "use msa_index_topk with a workspace", need, kScratchFloats);
  if (batch == 0) return ok();
  if (!q_idx || !block_idx) return fail(MSA_ERR_INVALID_ARG, "q_idx/block_idx is NULL");
  float* scores = nullptr;
  if ((st = scratch_address(&scores)) != MSA_OK) return st;
  return launch_index_decode(s, batch, q_idx, kv, block_idx, block_score, scores, static_cast<hipStream_t>(hip_stream),
                             "msa_index_topk_decode_static");
}


int32_t msa_abi_version(void) { return MSA_ABI_VERSION; }

msa_status msa_profile_enable(int32_t on) {
  msa::profile_set(on != 0);
  return ok();
}

msa_status msa_probe_mfma(int32_t n_wg, int32_t iters, float* out, void* hip_stream) {
  if (n_wg < 1 || iters < 1) return fail(MSA_ERR_INVALID_ARG, "n_wg=%d iters=%d must be >= 1", n_wg, iters);
  if (!out) return fail(MSA_ERR_INVALID_ARG, "out is NULL");
  return hip_status(msa::launch_mfma_probe(n_wg, iters, out, static_cast<hipStream_t>(hip_stream)), "msa_probe_mfma");
}

msa_status msa_test_schedule_lds_limit(int32_t max_blocks) {
  msa::set_schedule_lds_limit(max_blocks);
  return ok();
}

msa_status msa_profile_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(MSA_ERR_INVALID_ARG, "total_ms and launches must not be NULL");
  const int k = msa::profile_kernel_id(kernel);
  if (k < 0) return fail(MSA_ERR_INVALID_ARG, "unknown kernel name '%s'", kernel ? kernel : "(null)");
  long long n = 0;
  const hipError_t e = msa::profile_collect(static_cast<msa::ProfKernel>(k), total_ms, &n);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "profile_collect: %s", hipGetErrorString(e));
  *launches = n;
  return ok();
}

const char* msa_status_string(msa_status st) {
  switch (st) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

const char* msa_last_error(void) { return g_last_error.c_str(); }

size_t msa_workspace_size(int32_t op, const msa_shape* shape, int32_t batch, int32_t n_q, int32_t q_start,
                          int32_t n_kv, int32_t max_pages) {
  if (op < 0 || op > 7) {
    fail(MSA_ERR_INVALID_ARG, "op=%d not in 0..7", op);
    return 0;
  }
  if (op == 7) {  // msa_index_project: n_q = n_tok, n_kv = d_model
    if (check_shape(shape, true, false) != MSA_OK) return 0;
    if (n_q < 0 || n_kv < 0) {
      fail(MSA_ERR_INVALID_ARG, "negative size");
      return 0;
    }
    ok();
    return msa::kx_plan(n_q, n_kv, shape->h_kv, shape->d_idx).total;
  }
  if (check_shape(shape, op == 0 || op == 4 || op == 6, (op >= 1 && op <= 3) || op >= 5) != MSA_OK) return 0;
  if (check_cache_dtype(*shape, op != 3 && op < 5) != MSA_OK) return 0;
  if (batch < 0 || n_q < 0 || q_start < 0 || n_kv < 0 || max_pages < 0) {
    fail(MSA_ERR_INVALID_ARG, "negative size");
    return 0;
  }
  const msa_shape& s = *shape;
  (void)n_kv;
  ok();
  switch (op) {
    case 0:
      return std::max(ki_prefill_ws(s, n_q, q_start, 0), ki_prefill_ws(s, n_q, q_start, 1));
    case 4:  // decode mode: pooled score of every page
      return (size_t)batch * s.h_kv * max_pages * 4;
    case 1:
      if (n_q == 0) return 0;
      return msa::prefill_plan(s.dtype, n_q, q_start, n_kv, s.h_q, s.h_kv, s.d_h, s.top_k).total;
    case 2:
      return msa::decode_plan(batch, s.h_q, s.h_kv, s.d_h, s.top_k).total;
    case 5:
    case 6:
      if (n_q == 0) return 0;
      return msa::backward_plan(n_q, q_start, n_kv, s.h_q, s.h_kv, s.d_h, s.top_k, s.d_idx, op == 6).total;
    default:
      return 0;
  }
}

msa_status msa_index_topk(const msa_shape* shape, int32_t batch, int32_t n_q, int32_t q_start,
                          const void* q_idx, const msa_kv* kv, int32_t* block_idx, float* block_score,
                          void* workspace, size_t ws_bytes, void* hip_stream) {
  msa_status st = check_shape(shape, true, false);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if (!kv) return fail(MSA_ERR_INVALID_ARG, "kv is NULL");
  if (batch < 0 || n_q < 0 || q_start < 0) return fail(MSA_ERR_INVALID_ARG, "batch=%d n_q=%d q_start=%d", batch, n_q, q_start);
  if (!kv->k_idx) return fail(MSA_ERR_INVALID_ARG, "kv->k_idx is NULL");
  if (!aligned16(q_idx) || !aligned16(kv->k_idx)) return fail(MSA_ERR_INVALID_ARG, "q_idx/k_idx must be 16-byte aligned");
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const float idx_scale = idx_scale_of(s);
  // The diagonal block must be scored when its pooled score is reported, and
  // when it competes as an ordinary candidate (no forced local block).
  const int need_diag = (block_score != nullptr || !s.force_local) ? 1 : 0;

  if ((st = check_cache_dtype(s, true)) != MSA_OK) return st;
  if ((st = check_scales(s, kv, true, false)) != MSA_OK) return st;
  if (kv->seq_lens) {  // decode mode
    if (n_q != 1) return fail(MSA_ERR_INVALID_ARG, "decode mode (seq_lens given) needs n_q == 1, got %d", n_q);
    if (!kv->page_table) return fail(MSA_ERR_INVALID_ARG, "decode mode needs a page_table");
    if (kv->max_pages < 1 || kv->max_pages > msa::kMaxDecodePages)
      return fail(MSA_ERR_UNSUPPORTED, "max_pages=%d not in [1,%d]", kv->max_pages, msa::kMaxDecodePages);
    if (batch == 0) return ok();
    if (!q_idx || !block_idx) return fail(MSA_ERR_INVALID_ARG, "q_idx/block_idx is NULL");
    const size_t need = (size_t)batch * s.h_kv * kv->max_pages * 4;
    if ((st = check_ws(workspace, ws_bytes, need)) != MSA_OK) return st;
    return launch_index_decode(s, batch, q_idx, kv, block_idx, block_score, static_cast<float*>(workspace), stream,
                               "msa_index_topk(decode)");
  }

  if (batch != 1) return fail(MSA_ERR_INVALID_ARG, "prefill mode handles one sequence: batch must be 1, got %d", batch);
  if ((int64_t)q_start + n_q > kv->n_kv)
    return fail(MSA_ERR_INVALID_ARG, "q_start + n_q = %lld exceeds n_kv = %d", (long long)q_start + n_q, kv->n_kv);
  if (kv->page_table && (int64_t)kv->max_pages * MSA_BLOCK_SIZE < kv->n_kv)
    return fail(MSA_ERR_INVALID_ARG, "max_pages=%d too small for n_kv=%d", kv->max_pages, kv->n_kv);
  if ((int64_t)n_q * s.h_kv * s.top_k >= (int64_t(1) << 31)) return fail(MSA_ERR_UNSUPPORTED, "n_q too large");
  if (n_q == 0) return ok();
  if (!q_idx || !block_idx) return fail(MSA_ERR_INVALID_ARG, "q_idx/block_idx is NULL");
  const msa::KiPlan p = msa::ki_prefill_plan(n_q, s.h_kv, q_start, need_diag);
  const size_t need = ki_prefill_ws(s, n_q, q_start, need_diag);
  if ((st = check_ws(workspace, ws_bytes, need)) != MSA_OK) return st;
  msa::KiPrefillArgs a{};
  a.q_idx = q_idx;
  a.k_idx = kv->k_idx;
  a.k_idx_scale = mx_cache(s) ? kv->k_idx_scale : nullptr;
  a.page_table = kv->page_table;
  a.n_rows = p.n_rows;
  a.h_kv = s.h_kv;
  a.q_start = q_start;
  a.n_kv = kv->n_kv;
  a.chunk_blocks = p.chunk_blocks;
  a.n_chunks = p.n_chunks;
  a.grid_chunks = p.grid_chunks;
  a.xcd_major = p.xcd_major;
  a.n_tiles = p.n_tiles;
  a.idx_scale = idx_scale;
  a.force_local = s.force_local;
  a.pool = s.pool;
  a.top_k = s.top_k;
  a.need_diag = need_diag;
  a.block_idx = block_idx;
  a.block_score = block_score;
  if (p.n_chunks > 1) {
    char* ws = static_cast<char*>(workspace);
    const size_t keys = ((size_t)p.n_rows * p.n_chunks * 16 * 8 + 255) & ~size_t(255);
    a.part_keys = reinterpret_cast<uint64_t*>(ws);
    a.part_diag = reinterpret_cast<float*>(ws + keys);
  }
  return hip_status(msa::launch_ki_prefill(kernel_dtype(s), s.d_idx, a, stream), "msa_index_topk(prefill)");
}

msa_status msa_sparse_prefill(const msa_shape* shape, int32_t n_q, int32_t q_start, const void* q,
                              const msa_kv* kv, const int32_t* block_idx, void* o, float* lse,
                              void* workspace, size_t ws_bytes, void* hip_stream) {
  msa_status st = check_shape(shape, false, true);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if ((st = check_cache_dtype(s, true)) != MSA_OK) return st;
  if (!kv) return fail(MSA_ERR_INVALID_ARG, "kv is NULL");
  if ((st = check_scales(s, kv, false, true)) != MSA_OK) return st;
  if (kv->seq_lens) return fail(MSA_ERR_INVALID_ARG, "msa_sparse_prefill takes one sequence: seq_lens must be NULL");
  if (n_q < 0 || q_start < 0) return fail(MSA_ERR_INVALID_ARG, "n_q=%d q_start=%d", n_q, q_start);
  if ((int64_t)q_start + n_q > kv->n_kv)
    return fail(MSA_ERR_INVALID_ARG, "q_start + n_q = %lld exceeds n_kv = %d", (long long)q_start + n_q, kv->n_kv);
  if (kv->page_table && (int64_t)kv->max_pages * MSA_BLOCK_SIZE < kv->n_kv)
    return fail(MSA_ERR_INVALID_ARG, "max_pages=%d too small for n_kv=%d", kv->max_pages, kv->n_kv);
  if ((int64_t)n_q * s.h_kv * s.top_k >= (int64_t(1) << 27)) return fail(MSA_ERR_UNSUPPORTED, "n_q too large");
  if (n_q == 0) return ok();
  if (!q || !kv->k || !kv->v || !block_idx || !o) return fail(MSA_ERR_INVALID_ARG, "q/k/v/block_idx/o is NULL");
  if (!aligned16(q) || !aligned16(kv->k) || !aligned16(kv->v) || !aligned16(o))
    return fail(MSA_ERR_INVALID_ARG, "q/k/v/o must be 16-byte aligned");
  const msa::PrefillPlan pl = msa::prefill_plan(s.dtype, n_q, q_start, kv->n_kv, s.h_q, s.h_kv, s.d_h, s.top_k);
  if ((st = check_ws(workspace, ws_bytes, pl.total)) != MSA_OK) return st;
  msa::AttnArgs a{};
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.k_scale = mx_cache(s) ? kv->k_scale : nullptr;
  a.v_scale = mx_cache(s) ? kv->v_scale : nullptr;
  a.page_table = kv->page_table;
  a.block_idx = block_idx;
  a.o = o;
  a.lse = lse;
  a.n_q = n_q;
  a.q_start = q_start;
  a.n_kv = kv->n_kv;
  a.batch = 1;
  a.max_pages = kv->max_pages;
  a.h_q = s.h_q;
  a.h_kv = s.h_kv;
  a.group = s.h_q / s.h_kv;
  a.top_k = s.top_k;
  a.sm_scale = sm_scale_of(s);
  a.ws = workspace;
  a.ws_bytes = ws_bytes;
  return hip_status(msa::launch_sparse_prefill(kernel_dtype(s), s.d_h, a, pl, static_cast<hipStream_t>(hip_stream)),
                    "msa_sparse_prefill");
}

msa_status msa_index_project(const msa_shape* shape, int32_t n_tok, int32_t d_model, const void* x,
                             const void* w_q_idx, const void* w_k_idx, int32_t rope_dim, float rope_base,
                             const int32_t* positions, const int32_t* seq, const msa_kv* kv, void* q_idx_out,
                             void* workspace, size_t ws_bytes, void* hip_stream) {
  msa_status st = check_shape(shape, true, false);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if (s.dtype != MSA_BF16 || fp8_cache(s)) return fail(MSA_ERR_UNSUPPORTED, "msa_index_project is built for bf16");
  if (!kv) return fail(MSA_ERR_INVALID_ARG, "kv is NULL");
  if (n_tok < 0) return fail(MSA_ERR_INVALID_ARG, "n_tok=%d", n_tok);
  if (d_model <= 0 || d_model % 16 != 0) return fail(MSA_ERR_INVALID_ARG, "d_model=%d must be a positive multiple of 16", d_model);
  if (rope_dim != 0 && rope_dim != 32 && rope_dim != 64 && rope_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "rope_dim=%d not in {0,32,64,128}", rope_dim);
  if (rope_dim > s.d_idx) return fail(MSA_ERR_INVALID_ARG, "rope_dim=%d exceeds d_idx=%d", rope_dim, s.d_idx);
  if (rope_dim > 0 && !(rope_base > 1.0f)) return fail(MSA_ERR_INVALID_ARG, "rope_base must be > 1");
  if (kv->page_table && kv->max_pages < 1) return fail(MSA_ERR_INVALID_ARG, "max_pages=%d", kv->max_pages);
  if (n_tok == 0) return ok();
  if (!x || !w_q_idx || !w_k_idx || !positions || !kv->k_idx || !q_idx_out)
    return fail(MSA_ERR_INVALID_ARG, "x/w_q_idx/w_k_idx/positions/k_idx/q_idx_out is NULL");
  if (!aligned16(x) || !aligned16(w_q_idx) || !aligned16(w_k_idx) || !aligned16(kv->k_idx) || !aligned16(q_idx_out))
    return fail(MSA_ERR_INVALID_ARG, "x/w_q_idx/w_k_idx/k_idx/q_idx_out must be 16-byte aligned");
  msa::KxArgs a{};
  a.x = x;
  a.w_q = w_q_idx;
  a.w_k = w_k_idx;
  a.positions = positions;
  a.seq = seq;
  a.page_table = kv->page_table;
  a.k_cache = const_cast<void*>(kv->k_idx);
  a.q_out = q_idx_out;
  a.n_tok = n_tok;
  a.d_model = d_model;
  a.h_kv = s.h_kv;
  a.rope_dim = rope_dim;
  a.n_kv = kv->n_kv;
  a.max_pages = kv->max_pages;
  a.rope_base = rope_base;
  const msa::KxPlan pl = msa::kx_plan(n_tok, d_model, s.h_kv, s.d_idx);
  if ((st = check_ws(workspace, ws_bytes, pl.total)) != MSA_OK) return st;
  a.split = pl.split;
  a.k_per_split = pl.k_per_split;
  a.part = pl.split > 1 ? static_cast<float*>(workspace) : nullptr;
  return hip_status(msa::launch_index_project(s.d_idx, a, static_cast<hipStream_t>(hip_stream)), "msa_index_project");
}

msa_status msa_sparse_prefill_backward(const msa_shape* shape, int32_t n_q, int32_t q_start, const void* q,
                                       const msa_kv* kv, const int32_t* block_idx, const void* o, const float* lse,
                                       const void* d_o, void* dq, void* dk, void* dv, const msa_kl* kl,
                                       void* workspace, size_t ws_bytes, void* hip_stream) {
  msa_status st = check_shape(shape, kl != nullptr, true);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if ((st = check_cache_dtype(s, false)) != MSA_OK) return st;
  if (!msa::backward_supported(s.dtype, s.d_h))
    return fail(MSA_ERR_UNSUPPORTED, "the backward is built for dtype MSA_BF16 and d_h 64/128");
  if (!kv) return fail(MSA_ERR_INVALID_ARG, "kv is NULL");
  if (kv->seq_lens || kv->page_table)
    return fail(MSA_ERR_UNSUPPORTED, "the backward takes one contiguous sequence (no page_table, no seq_lens)");
  if (n_q < 0 || q_start < 0 || kv->n_kv < 0) return fail(MSA_ERR_INVALID_ARG, "n_q=%d q_start=%d", n_q, q_start);
  if ((int64_t)q_start + n_q > kv->n_kv)
    return fail(MSA_ERR_INVALID_ARG, "q_start + n_q = %lld exceeds n_kv = %d", (long long)q_start + n_q, kv->n_kv);
  if ((int64_t)n_q * s.h_kv * s.top_k >= (int64_t(1) << 27)) return fail(MSA_ERR_UNSUPPORTED, "n_q too large");
  if (kv->n_kv > 0 && (!dk || !dv)) return fail(MSA_ERR_INVALID_ARG, "dk/dv is NULL");
  if (n_q > 0 && (!q || !kv->k || !kv->v || !block_idx || !o || !lse || !d_o || !dq))
    return fail(MSA_ERR_INVALID_ARG, "q/k/v/block_idx/o/lse/d_o/dq is NULL");
  if (!aligned16(q) || !aligned16(kv->k) || !aligned16(kv->v) || !aligned16(o) || !aligned16(d_o) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(MSA_ERR_INVALID_ARG, "q/k/v/o/d_o/dq/dk/dv must be 16-byte aligned");
  if (kl) {
    if ((kv->n_kv > 0 && !kl->dk_idx) || (n_q > 0 && (!kl->q_idx || !kl->k_idx || !kl->dq_idx)))
      return fail(MSA_ERR_INVALID_ARG, "kl: q_idx/k_idx/dq_idx/dk_idx is NULL");
    if (!aligned16(kl->q_idx) || !aligned16(kl->k_idx) || !aligned16(kl->dq_idx) || !aligned16(kl->dk_idx))
      return fail(MSA_ERR_INVALID_ARG, "kl: q_idx/k_idx/dq_idx/dk_idx must be 16-byte aligned");
    if (!(kl->kl_scale == kl->kl_scale)) return fail(MSA_ERR_INVALID_ARG, "kl: kl_scale is NaN");
  }
  if (kv->n_kv == 0) return ok();
  const msa::BackwardPlan pl =
      msa::backward_plan(n_q, q_start, kv->n_kv, s.h_q, s.h_kv, s.d_h, s.top_k, s.d_idx, kl != nullptr);
  if (n_q > 0 && (st = check_ws(workspace, ws_bytes, pl.total)) != MSA_OK) return st;
  msa::BackwardArgs b{};
  msa::AttnArgs& a = b.attn;
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.block_idx = block_idx;
  a.o = const_cast<void*>(o);
  a.lse = const_cast<float*>(lse);
  a.n_q = n_q;
  a.q_start = q_start;
  a.n_kv = kv->n_kv;
  a.batch = 1;
  a.h_q = s.h_q;
  a.h_kv = s.h_kv;
  a.group = s.h_q / s.h_kv;
  a.top_k = s.top_k;
  a.sm_scale = sm_scale_of(s);
  a.ws = workspace;
  a.ws_bytes = ws_bytes;
  b.d_o = d_o;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  if (kl) {
    b.kl = 1;
    b.d_idx = s.d_idx;
    b.q_idx = kl->q_idx;
    b.k_idx = kl->k_idx;
    b.idx_scale = s.idx_scale > 0.f ? s.idx_scale : 1.0f / sqrtf((float)s.d_idx);
    b.kl_scale = kl->kl_scale;
    b.kl_out = kl->kl_out;
    b.dq_idx = kl->dq_idx;
    b.dk_idx = kl->dk_idx;
  }
  return hip_status(msa::launch_sparse_prefill_backward(s.d_h, b, pl, static_cast<hipStream_t>(hip_stream)),
                    "msa_sparse_prefill_backward");
}

msa_status msa_sparse_decode(const msa_shape* shape, int32_t batch, const void* q, const msa_kv* kv,
                             const int32_t* block_idx, void* o, float* lse, void* workspace, size_t ws_bytes,
                             void* hip_stream) {
  msa_status st = check_shape(shape, false, true);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if ((st = check_cache_dtype(s, true)) != MSA_OK) return st;
  if (!msa::decode_supported(kernel_dtype(s), s.d_h)) return fail(MSA_ERR_UNSUPPORTED, "decode is built for bf16 only");
  if (!kv) return fail(MSA_ERR_INVALID_ARG, "kv is NULL");
  if ((st = check_scales(s, kv, false, true)) != MSA_OK) return st;
  if (!kv->page_table || !kv->seq_lens) return fail(MSA_ERR_INVALID_ARG, "decode needs a paged cache with seq_lens");
  if (kv->max_pages < 1) return fail(MSA_ERR_INVALID_ARG, "max_pages=%d", kv->max_pages);
  if (batch < 0) return fail(MSA_ERR_INVALID_ARG, "batch=%d", batch);
  if (batch == 0) return ok();
  if (!q || !kv->k || !kv->v || !block_idx || !o) return fail(MSA_ERR_INVALID_ARG, "q/k/v/block_idx/o is NULL");
  if (!aligned16(q) || !aligned16(kv->k) || !aligned16(kv->v) || !aligned16(o))
    return fail(MSA_ERR_INVALID_ARG, "q/k/v/o must be 16-byte aligned");
  const msa::DecodePlan pl = msa::decode_plan(batch, s.h_q, s.h_kv, s.d_h, s.top_k);
  if ((st = check_ws(workspace, ws_bytes, pl.total)) != MSA_OK) return st;
  msa::AttnArgs a{};
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.k_scale = mx_cache(s) ? kv->k_scale : nullptr;
  a.v_scale = mx_cache(s) ? kv->v_scale : nullptr;
  a.page_table = kv->page_table;
  a.seq_lens = kv->seq_lens;
  a.block_idx = block_idx;
  a.o = o;
  a.lse = lse;
  a.batch = batch;
  a.max_pages = kv->max_pages;
  a.h_q = s.h_q;
  a.h_kv = s.h_kv;
  a.group = s.h_q / s.h_kv;
  a.top_k = s.top_k;
  a.sm_scale = sm_scale_of(s);
  a.ws = workspace;
  a.ws_bytes = ws_bytes;
  return hip_status(msa::launch_sparse_decode(kernel_dtype(s), s.d_h, a, pl, static_cast<hipStream_t>(hip_stream)),
                    "msa_sparse_decode");
}

msa_status msa_dense_prefill(const msa_shape* shape, int32_t n_q, int32_t q_start, const void* q,
                             const msa_kv* kv, void* o, float* lse, void* workspace, size_t ws_bytes,
                             void* hip_stream) {
  (void)workspace;
  (void)ws_bytes;
  msa_status st = check_shape(shape, false, true);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if ((st = check_cache_dtype(s, false)) != MSA_OK) return st;
  if (!kv) return fail(MSA_ERR_INVALID_ARG, "kv is NULL");
  if (kv->page_table || kv->seq_lens) return fail(MSA_ERR_UNSUPPORTED, "dense prefill takes a contiguous cache");
  if (n_q < 0 || q_start < 0 || (int64_t)q_start + n_q > kv->n_kv)
    return fail(MSA_ERR_INVALID_ARG, "n_q=%d q_start=%d n_kv=%d", n_q, q_start, kv->n_kv);
  if (n_q == 0) return ok();
  if (!q || !kv->k || !kv->v || !o) return fail(MSA_ERR_INVALID_ARG, "q/k/v/o is NULL");
  if (!aligned16(q) || !aligned16(kv->k) || !aligned16(kv->v) || !aligned16(o))
    return fail(MSA_ERR_INVALID_ARG, "q/k/v/o must be 16-byte aligned");
  msa::AttnArgs a{};
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.o = o;
  a.lse = lse;
  a.n_q = n_q;
  a.q_start = q_start;
  a.n_kv = kv->n_kv;
  a.h_q = s.h_q;
  a.h_kv = s.h_kv;
  a.group = s.h_q / s.h_kv;
  a.sm_scale = sm_scale_of(s);
  return hip_status(msa::launch_dense_prefill(s.dtype, s.d_h, a, static_cast<hipStream_t>(hip_stream)),
                    "msa_dense_prefill");
}

}  // extern "C"
