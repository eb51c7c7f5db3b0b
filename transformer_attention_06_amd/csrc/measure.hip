// Measurement aid: the average shader clock over a stretch of wall time.
//
// One wave reads the shader-clock counter (s_memtime) and the constant
// 100 MHz counter (s_memrealtime), sleeps until `ticks` of the latter have
// passed, and reads both again. Run on a second stream beside other
// kernels, the ratio is the clock those kernels ran at (the counters are
// chip-wide; the wave itself mostly sleeps and takes no LDS). The loop's
// exit depends only on the real-time counter, so it always ends.

#include "kernels.hpp"

namespace nc {
namespace {

__global__ __launch_bounds__(64) void shader_clock_kernel(unsigned long long* out, unsigned long long ticks) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r1 = r0;
  while (r1 - r0 < ticks) {
    __builtin_amdgcn_s_sleep(127);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_shader_clock(unsigned long long* out, unsigned long long ticks, hipStream_t s) {
  shader_clock_kernel<<<1, 64, 0, s>>>(out, ticks);
  return hipGetLastError();
}

}  // namespace nc
