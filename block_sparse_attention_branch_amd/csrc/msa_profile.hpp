// msa_profile.hpp - optional per-kernel launch timing with HIP events.
//
// Off by default.  When enabled (msa_profile_enable), the launch code brackets
// every launch of a timed kernel with two events recorded on the launch
// stream; msa_profile_read() waits for them and returns the summed GPU time
// of a kernel's launches.  Used to time the dominant kernels live, on the
// stream they run on, without a profiler.
#pragma once

#include <hip/hip_runtime.h>

namespace msa {

enum ProfKernel { PK_KI_PREFILL = 0, PK_KP, PK_KM, PK_KI_DECODE_SCAN, PK_KD, PK_KBQ, PK_KBKV, PK_COUNT };

bool profile_on();
void profile_set(bool on);
// Returns a slot (or -1 when profiling is off / an event could not be made).
int profile_begin(ProfKernel k, hipStream_t st);
void profile_end(int slot, hipStream_t st);
int profile_kernel_id(const char* name);
// Sums the recorded durations of kernel k and forgets them.
hipError_t profile_collect(ProfKernel k, double* total_ms, long long* launches);
// n_wg workgroups of 4 waves, each wave `iters` rounds of 8 bf16 32x32x16 MFMAs.
hipError_t launch_mfma_probe(int32_t n_wg, int32_t iters, float* out, hipStream_t st);

}  // namespace msa
