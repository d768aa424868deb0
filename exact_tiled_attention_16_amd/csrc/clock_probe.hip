// Shader clock under load -- a measurement aid, built as its own library
// (libfa_probe.so), not part of the attention library's C ABI.
//
// One wave sleeps in short steps for a given wall-clock interval and records
// the shader-cycle counter and the constant-rate wall clock at both ends;
// the ratio of the two differences is the shader clock while whatever else
// is running on the device runs.  The loop is bounded by an iteration count
// as well as by the wall clock, so it always ends.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ void __launch_bounds__(64)
clock_probe_kernel(long long* out, long long wall_ticks, long long max_iter) {
  const long long w0 = wall_clock64();
  const long long c0 = clock64();
  long long w = w0;
  for (long long it = 0; it < max_iter && w - w0 < wall_ticks; ++it) {
    __builtin_amdgcn_s_sleep(32);  // 32 x 64 shader cycles
    w = wall_clock64();
  }
  const long long c1 = clock64();
  if (threadIdx.x == 0) {
    out[0] = w0;
    out[1] = w;
    out[2] = c0;
    out[3] = c1;
  }
}

}  // namespace

extern "C" {

// Wall-clock counter rate of the current device in kHz, or 0.
long long fa_probe_wall_rate_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

// Enqueue the probe on `stream` (a hipStream_t): it runs for about
// `wall_ticks` wall-clock ticks and writes {wall start, wall end, shader
// cycles start, shader cycles end} to out[0..3] (device memory, 4 int64).
// Returns 0, -1 on a bad argument, -3 if the launch fails.
int fa_probe_clock(long long* out, long long wall_ticks, void* stream) {
  if (out == nullptr || wall_ticks <= 0 || wall_ticks > (1LL << 40)) return -1;
  // Each step sleeps at least 2048 shader cycles (> 0.5 us below 4 GHz),
  // i.e. at least 50 ticks of a 100 MHz wall clock: this bound ends the loop
  // after about twice the requested interval even if the wall clock stalls.
  const long long max_iter = wall_ticks / 25 + 1024;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     out, wall_ticks, max_iter);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
