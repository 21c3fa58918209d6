// Diagnostics: the shader clock the GPU holds, measured on the device.
//
// One wave reads the shader-clock counter (s_memtime) and the constant
// 100 MHz counter (s_memrealtime) at the start and the end of a spin of
// about `ticks` wall-clock ticks. Launched between two kernels on one stream,
// it runs at the clock the chip holds for that load (clock changes take
// milliseconds, the probe tens of microseconds), and the ratio of the two
// counters' advances gives that clock. The spin ends on the wall-clock
// counter, so it always terminates.

#include "../../include/fp8gemm.h"
#include "internal.h"

namespace fp8g {
namespace {

__global__ void __launch_bounds__(64) clock_probe_kernel(uint64_t* out, int ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0;
  while (r1 - r0 < (uint64_t)ticks) r1 = __builtin_amdgcn_s_memrealtime();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = t1 - t0;
    out[1] = r1 - r0;
  }
}

}  // namespace
}  // namespace fp8g

extern "C" fp8g_status fp8g_clock_probe(uint64_t* out, int ticks, hipStream_t stream) {
  if (!out) return FP8G_ERR_NULL_PTR;
  if (((uintptr_t)out & 7) != 0) return FP8G_ERR_ALIGN;
  if (ticks < 1 || ticks > 1000000) return FP8G_ERR_SHAPE;
  fp8g::DeviceInfo dev;
  if (fp8g::current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  hipLaunchKernelGGL(fp8g::clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, ticks);
  return hipGetLastError() == hipSuccess ? FP8G_OK : FP8G_ERR_LAUNCH;
}
