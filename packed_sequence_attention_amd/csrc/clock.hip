// blockdiag_clock_probe: the engine clock a measurement ran at.  Each
// workgroup (one wave) reads the shader-clock counter (s_memtime, one count
// per engine clock cycle) and the constant 100 MHz real-time counter
// (s_memrealtime) before and after spinning for a given number of real-time
// ticks; the ratio of the two differences, times 100 MHz, is the clock its
// CU ran at meanwhile.  A measurement aid next to the attention calls, not
// part of the attention path.
#include <hip/hip_runtime.h>

#include "blockdiag.h"
#include "internal.h"

namespace {

// Bound on the spin loop's iterations, whatever the counters read: every
// wave leaves the loop.
constexpr int kMaxSpin = 1 << 22;

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* __restrict__ out, uint32_t ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0, c1 = c0;
  for (int i = 0; i < kMaxSpin && r1 - r0 < ticks; ++i) {
    r1 = __builtin_amdgcn_s_memrealtime();
    c1 = __builtin_amdgcn_s_memtime();
  }
  if (threadIdx.x < 2) out[2 * blockIdx.x + threadIdx.x] = threadIdx.x == 0 ? c1 - c0 : r1 - r0;
}

}  // namespace

extern "C" bd_status blockdiag_clock_probe(int32_t n_workgroups, uint32_t ticks, uint64_t* d_out, void* stream) {
  if (n_workgroups <= 0 || n_workgroups > 65536 || ticks == 0 || ticks > 10000000u || d_out == nullptr)
    return bd::fail(BD_ERR_INVALID_ARG, "clock_probe: n_workgroups %d, ticks %u, out %p", n_workgroups, ticks,
                    static_cast<void*>(d_out));
  hipLaunchKernelGGL(clock_probe_kernel, dim3(n_workgroups), dim3(64), 0, static_cast<hipStream_t>(stream), d_out,
                     ticks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return bd::fail(BD_ERR_HIP, "clock_probe launch: %s", hipGetErrorString(e));
  return BD_OK;
}
