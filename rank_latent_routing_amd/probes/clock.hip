// Shader-clock sampler: one wave per XCD (workgroup i of the 8 runs on XCD
// i mod 8) reads the shader clock counter (s_memtime) and the constant
// 100 MHz real-time counter (s_memrealtime) at the start and the end of a
// spin of a fixed real-time length.  Launched on a second stream beside
// back-to-back launches of a kernel, it gives the average shader clock of
// each XCD while that kernel runs (the clock under the kernel's power draw),
// in real time, without counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(64) void clock_sample_kernel(unsigned long long* out, unsigned long long ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0, c1 = c0;
  // Ends once `ticks` real-time ticks have passed: the counter runs at a
  // constant rate whatever the load, so every wave leaves the loop.
  while (r1 - r0 < ticks) {
    __builtin_amdgcn_s_sleep(32);
    r1 = __builtin_amdgcn_s_memrealtime();
    c1 = __builtin_amdgcn_s_memtime();
  }
  if (threadIdx.x == 0) {
    out[4 * blockIdx.x + 0] = r0;
    out[4 * blockIdx.x + 1] = r1;
    out[4 * blockIdx.x + 2] = c0;
    out[4 * blockIdx.x + 3] = c1;
  }
}

}  // namespace

extern "C" {

// Spins one wave per XCD (8 workgroups of one wave) for `ticks` ticks of the
// 100 MHz real-time counter (at most 10^7, 0.1 s) on `stream`, then writes
// four device integers per workgroup to out[4 i .. 4 i + 3] (32 in all): the
// real-time counter at the start and the end, and the shader clock counter at
// the start and the end.  Returns a hipError_t.
int clock_sample(unsigned long long* out, unsigned long long ticks, void* stream) {
  if (out == nullptr || ticks < 1 || ticks > 10000000ull) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(clock_sample_kernel, dim3(8), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), out, ticks);
  return (int)hipGetLastError();
}

}  // extern "C"
