// Shader-clock probe for throughput reports (not part of the attention path).
//
// One wave counts shader-clock cycles (s_memtime) and ticks of the device's
// constant-rate wall clock (s_memrealtime) over the same interval. Their ratio
// times the wall-clock rate is the shader clock over that interval, which is
// below the nominal clock when the chip throttles under load.
#include "sage_internal.h"

namespace sage {

namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(long long cycles, long long* out) {
  const long long w0 = static_cast<long long>(__builtin_amdgcn_s_memrealtime());
  const long long c0 = static_cast<long long>(__builtin_readcyclecounter());
  long long c1 = c0;
  // the counter advances every clock, so the loop ends after `cycles` clocks
  while (c1 - c0 < cycles) {
    __builtin_amdgcn_s_sleep(2);
    c1 = static_cast<long long>(__builtin_readcyclecounter());
  }
  const long long w1 = static_cast<long long>(__builtin_amdgcn_s_memrealtime());
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = w1 - w0;
  }
}

}  // namespace

hipError_t launch_clock_probe(long long cycles, long long* out, hipStream_t s) {
  clock_probe_kernel<<<1, 64, 0, s>>>(cycles, out);
  return hipGetLastError();
}

}  // namespace sage
