// msa_profile.hip - event pairs around timed kernel launches (diagnostics).
#include "msa_profile.hpp"

#include "msa_common.hpp"

#include <cstring>
#include <mutex>
#include <vector>

namespace msa {
namespace {

struct Rec {
  int kernel;
  hipEvent_t start, stop;
  bool used;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;   // events are kept for reuse once collected

const char* kNames[PK_COUNT] = {"ki_prefill_kernel", "kp_kernel",  "km_kernel",  "ki_decode_scan_kernel",
                                "kd_kernel",         "kbq_kernel", "kbkv_kernel"};

}  // namespace

bool profile_on() { return g_on; }

void profile_set(bool on) {
  std::lock_guard<std::mutex> g(g_mu);
  g_on = on;
}

int profile_kernel_id(const char* name) {
  for (int k = 0; k < PK_COUNT; ++k)
    if (name && std::strcmp(name, kNames[k]) == 0) return k;
  return -1;
}

int profile_begin(ProfKernel k, hipStream_t st) {
  if (!g_on) return -1;
  std::lock_guard<std::mutex> g(g_mu);
  int slot = -1;
  for (size_t i = 0; i < g_recs.size(); ++i)
    if (!g_recs[i].used) {
      slot = (int)i;
      break;
    }
  if (slot < 0) {
    Rec r{};
    if (hipEventCreate(&r.start) != hipSuccess) return -1;
    if (hipEventCreate(&r.stop) != hipSuccess) return -1;
    g_recs.push_back(r);
    slot = (int)g_recs.size() - 1;
  }
  Rec& r = g_recs[slot];
  r.kernel = k;
  r.used = true;
  if (hipEventRecord(r.start, st) != hipSuccess) {
    r.used = false;
    return -1;
  }
  return slot;
}

void profile_end(int slot, hipStream_t st) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> g(g_mu);
  (void)hipEventRecord(g_recs[slot].stop, st);
}

hipError_t profile_collect(ProfKernel k, double* total_ms, long long* launches) {
  std::lock_guard<std::mutex> g(g_mu);
  double tot = 0.0;
  long long n = 0;
  for (Rec& r : g_recs) {
    if (!r.used || r.kernel != k) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return e;
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return e;
    tot += ms;
    ++n;
    r.used = false;
  }
  *total_ms = tot;
  *launches = n;
  return hipSuccess;
}

// Dense bf16 MFMA throughput probe (measurement of the achievable peak): each
// wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 chains on
// operands made from the lane index (unknown at compile time); one sum per
// workgroup is written so that the work is kept.
__global__ __launch_bounds__(256) void kprobe_mfma_kernel(int32_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = from_f32<bf16_t>((float)(lane + e) * 1e-3f);
    b[e] = from_f32<bf16_t>((float)(3 * lane + e) * 1e-3f);
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) mma32(acc[j], a, b);
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) sum += acc[j][v];
  if (threadIdx.x == 0) out[blockIdx.x] = sum;
}

hipError_t launch_mfma_probe(int32_t n_wg, int32_t iters, float* out, hipStream_t st) {
  hipLaunchKernelGGL(kprobe_mfma_kernel, dim3((unsigned)n_wg), dim3(256), 0, st, iters, out);
  return hipGetLastError();
}

}  // namespace msa
