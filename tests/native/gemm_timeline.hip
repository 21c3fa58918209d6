// Per-wave timeline of the persistent GEMM's main loop (a measurement
// build, not part of the library): gemm.hip compiled with FP8G_TRACE, whose
// kernels stamp the shader clock (s_memtime) from lane 0 of every wave of
// workgroups 0..3 at six points of each of the first 32 K steps:
//   0  start of the step (slice 0)
//   1  start of the slice holding the end-of-step barrier
//   2  after the wave's own LDS reads have completed (lgkmcnt(0))
//   3  after its own copies of the next stage have landed and the barrier
//   4  after the first part of the next refill has been issued (copy waves)
//   5  after the last part has been issued (copy waves)
// Runs the dense 4096x8192x8192 GEMM (block-scaled, or per-tensor with
// argument 3) 60 times and prints, per wave, the cycles per K step spent in
// each phase, averaged over steps 4..27 of workgroups 0..3.
//
// Build: hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature
//        -Xclang -packed-fp32-ops -I include -o gemm_timeline
//        tests/native/gemm_timeline.hip
#define FP8G_TRACE 1
#include "../../moe_grouped_gemm_quantizer_amd/csrc/gemm.hip"

#include <stdio.h>
#include <stdlib.h>

#include <vector>

#define CK(x)                                                                      \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);        \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

using namespace fp8g;

int main(int argc, char** argv) {
  const int mode = argc > 1 ? atoi(argv[1]) : 0;   // 0 block-scaled, 3 per-tensor
  const int64_t M = 4096, N = 8192, K = 8192;
  uint8_t *a, *b;
  float *sa, *sb;
  uint16_t* d;
  CK(hipMalloc(&a, M * K));
  CK(hipMalloc(&b, N * K));
  CK(hipMalloc(&sa, (K / 128) * M * 4));
  CK(hipMalloc(&sb, (N / 128) * (K / 128) * 4));
  CK(hipMalloc(&d, M * N * 2));
  // (operand values do not matter for the timing; small codes, unit scales)
  CK(hipMemset(a, 0x38, M * K));
  CK(hipMemset(b, 0x30, N * K));
  std::vector<float> ones((size_t)(K / 128) * M, 1.0f);
  CK(hipMemcpy(sa, ones.data(), (K / 128) * M * 4, hipMemcpyHostToDevice));
  CK(hipMemcpy(sb, ones.data(), (N / 128) * (K / 128) * 4, hipMemcpyHostToDevice));
  DeviceInfo dev{1, 0};
  CK(hipDeviceGetAttribute(&dev.cu_count, hipDeviceAttributeMultiprocessorCount, 0));
  GemmArgs args{a, sa, b, sb, d, nullptr, M, M, N, K, 1, mode == 3 ? MODE_PERTENSOR : MODE_DENSE};
  for (int i = 0; i < 60; ++i) CK(launch_gemm(args, dev, 0, nullptr, 0, 0));
  CK(hipDeviceSynchronize());
  std::vector<unsigned long long> h((size_t)TR_WG * 8 * TR_STEPS * TR_PTS);
  CK(hipMemcpyFromSymbol(h.data(), HIP_SYMBOL(fp8g_trace), h.size() * 8));
  auto at = [&](int wg, int w, int s, int pt) {
    return (double)h[(((size_t)wg * 8 + w) * TR_STEPS + s) * TR_PTS + pt];
  };
  printf("%s GEMM 4096x8192x8192, 256x256 tiles, 8 waves (4-7 issue the copies);\n",
         mode == 3 ? "per-tensor" : "block-scaled");
  printf("shader cycles per K step, mean over steps 4..27 of workgroups 0..3\n");
  printf("wave | step | to barrier slice | own LDS reads | copies landed + barrier | refill part 0 | "
         "refill part 1\n");
  for (int w = 0; w < 8; ++w) {
    double step = 0, c1 = 0, c2 = 0, c3 = 0, c4 = 0, c5 = 0;
    int n = 0;
    for (int wg = 0; wg < TR_WG; ++wg)
      for (int s = 4; s < 28; ++s) {
        step += at(wg, w, s + 1, 0) - at(wg, w, s, 0);
        c1 += at(wg, w, s, 1) - at(wg, w, s, 0);
        c2 += at(wg, w, s, 2) - at(wg, w, s, 1);
        c3 += at(wg, w, s, 3) - at(wg, w, s, 2);
        if (w >= 4) {
          c4 += at(wg, w, s, 4) - at(wg, w, s, 3);
          c5 += at(wg, w, s + 1, 5) - at(wg, w, s + 1, 0);
        }
        ++n;
      }
    printf("%4d | %4.0f | %16.0f | %13.0f | %23.0f | %13.0f | %13.0f\n", w, step / n, c1 / n, c2 / n,
           c3 / n, c4 / n, c5 / n);
  }
  return 0;
}
