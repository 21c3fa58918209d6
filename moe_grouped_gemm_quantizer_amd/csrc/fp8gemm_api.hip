// C entry points of libfp8gemm: argument validation, device facts, launch.
// Every host-checkable precondition is checked before any HIP call, so a
// rejected call neither launches nor touches the device.

#include <mutex>
#include <vector>
#include <stddef.h>
#include <string.h>

#include "../../include/fp8gemm.h"
#include "internal.h"

namespace fp8g {

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];

void query_device(int dev) {
  DeviceInfo info{0, 0};
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
    info.cu_count = prop.multiProcessorCount;
    info.ok = (strncmp(prop.gcnArchName, "gfx950", 6) == 0 && info.cu_count > 0) ? 1 : 0;
  }
  g_info[dev] = info;
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
constexpr int64_t kMaxK = int64_t(1) << 24;
}  // namespace

int current_device_info(DeviceInfo* info) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1;
  std::call_once(g_once[dev], query_device, dev);
  *info = g_info[dev];
  return info->ok ? 0 : 1;
}

// Shared by both quantiser entry points; x_align is the input vector width.
template <typename T>
fp8g_status quantize_checked(const T* x, int64_t rows, int64_t cols, int64_t ldx, int block_rows,
                             uint8_t* q, int64_t ldq, float* scales, int64_t s_stride_row,
                             int64_t s_stride_col, hipStream_t stream) {
  constexpr uintptr_t x_align = 4 * sizeof(T);
  if (rows < 0 || cols < 0) return FP8G_ERR_SHAPE;
  if (block_rows != 1 && block_rows != 128) return FP8G_ERR_SHAPE;
  if (rows == 0) return FP8G_OK;
  if (cols == 0 || cols % 16 != 0) return FP8G_ERR_SHAPE;
  if (!x || !q || !scales) return FP8G_ERR_NULL_PTR;
  if (ldx < cols || ldq < cols || s_stride_row < 1 || s_stride_col < 1) return FP8G_ERR_STRIDE;
  if (!aligned(x, x_align) || ldx % 4 != 0 || !aligned(q, 4) || ldq % 4 != 0 ||
      !aligned(scales, 4))
    return FP8G_ERR_ALIGN;
  if ((cols + 127) / 128 > 65535 || (block_rows == 1 && (rows + 7) / 8 > 0x7FFFFFFF) ||
      (block_rows == 128 && (rows + 127) / 128 > 0x7FFFFFFF))
    return FP8G_ERR_UNSUPPORTED;
  // the 128x128 kernel reaches 8 rows from one base through 32-bit offsets
  if (block_rows == 128 && (ldx > (int64_t(1) << 26) || ldq > (int64_t(1) << 28)))
    return FP8G_ERR_UNSUPPORTED;
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  hipError_t e = launch_quantize<T>(x, rows, cols, ldx, block_rows, q, ldq, scales, s_stride_row,
                                    s_stride_col, stream, dev.cu_count);
  return e == hipSuccess ? FP8G_OK : FP8G_ERR_LAUNCH;
}

}  // namespace fp8g

using namespace fp8g;

extern "C" {

const char* fp8g_status_string(fp8g_status status) {
  switch (status) {
    case FP8G_OK: return "ok";
    case FP8G_ERR_NULL_PTR: return "a required pointer is NULL";
    case FP8G_ERR_SHAPE: return "invalid size (negative, or not a required multiple)";
    case FP8G_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case FP8G_ERR_STRIDE: return "leading dimension or scale stride too small";
    case FP8G_ERR_DEVICE: return "no usable gfx950 device is current";
    case FP8G_ERR_LAUNCH: return "kernel launch failed";
    case FP8G_ERR_UNSUPPORTED: return "request not supported by the library";
    case FP8G_ERR_WORKSPACE: return "workspace too small for this call";
    default: return "unknown status";
  }
}

int fp8g_abi_version(void) { return 3; }

fp8g_status fp8g_warmup(void) {
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  std::vector<const void*> kernels;
  gemm_kernels(kernels);
  quantize_kernels(kernels);
  for (const void* k : kernels) {
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, k) != hipSuccess) {
      (void)hipGetLastError();
      return FP8G_ERR_LAUNCH;
    }
  }
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess || !scratch_ptr(device)) return FP8G_ERR_DEVICE;
  return FP8G_OK;
}

fp8g_status fp8g_set_shape_specialisation(int enable) {
  set_shape_specialisation(enable);
  return FP8G_OK;
}

fp8g_status fp8g_gemm_kernel_name(int layout, int64_t rows, int64_t N, int64_t K, int G,
                                  int expected_m, int quant, char* buf, size_t len) {
  if (!buf) return FP8G_ERR_NULL_PTR;
  if (len == 0) return FP8G_ERR_SHAPE;
  if (layout < FP8G_LAYOUT_DENSE || layout > FP8G_LAYOUT_PERTENSOR) return FP8G_ERR_SHAPE;
  if (rows < 0 || G < 0 || N <= 0 || K <= 0 || N % 16 != 0 || K % 16 != 0)
    return FP8G_ERR_SHAPE;
  if (quant && layout != FP8G_LAYOUT_DENSE) return FP8G_ERR_UNSUPPORTED;
  GemmArgs args{};
  args.mode = layout == FP8G_LAYOUT_DENSE        ? MODE_DENSE
              : layout == FP8G_LAYOUT_CONTIGUOUS ? MODE_CONTIGUOUS
              : layout == FP8G_LAYOUT_MASKED     ? MODE_MASKED
                                                 : MODE_PERTENSOR;
  args.rows = rows;
  args.N = N;
  args.K = K;
  args.G = layout == FP8G_LAYOUT_CONTIGUOUS || layout == FP8G_LAYOUT_MASKED ? G : 1;
  static uint8_t marker;
  args.qd = quant ? &marker : nullptr;      // (only tested for null by the selection)
  describe_gemm(args, expected_m, buf, len);
  return FP8G_OK;
}


fp8g_status fp8_quantize(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                         int block_rows, uint8_t* q, int64_t ldq, float* scales,
                         int64_t s_stride_row, int64_t s_stride_col, hipStream_t stream) {
  return quantize_checked(x, rows, cols, ldx, block_rows, q, ldq, scales, s_stride_row,
                          s_stride_col, stream);
}

fp8g_status fp8_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                              int block_rows, uint8_t* q, int64_t ldq, float* scales,
                              int64_t s_stride_row, int64_t s_stride_col, hipStream_t stream) {
  return quantize_checked(x, rows, cols, ldx, block_rows, q, ldq, scales, s_stride_row,
                          s_stride_col, stream);
}

fp8g_status fp8_quantize_tensor(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* q, int64_t ldq, float* scale, hipStream_t stream) {
  if (rows < 0 || cols < 0) return FP8G_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8G_OK;
  if (cols % 4 != 0) return FP8G_ERR_SHAPE;
  if (!x || !q || !scale) return FP8G_ERR_NULL_PTR;
  if (ldx < cols || ldq < cols) return FP8G_ERR_STRIDE;
  if (!aligned(x, 16) || ldx % 4 != 0 || !aligned(q, 4) || ldq % 4 != 0 || !aligned(scale, 4))
    return FP8G_ERR_ALIGN;
  if ((cols + 1023) / 1024 > 0x7FFFFFFF) return FP8G_ERR_UNSUPPORTED;
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  return launch_quantize_tensor(x, rows, cols, ldx, q, ldq, scale, stream) == hipSuccess
             ? FP8G_OK
             : FP8G_ERR_LAUNCH;
}

static fp8g_status check_nk(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % 16 != 0 || K % 16 != 0) return FP8G_ERR_SHAPE;
  // int32 tile bookkeeping inside the kernel; the operand copies address up
  // to 256 rows of a tile from one base with 32-bit byte offsets
  // (255 * K + 112 < 2^32 for K <= 2^24)
  if ((N + 127) / 128 > (1 << 20) || K > kMaxK) return FP8G_ERR_UNSUPPORTED;
  return FP8G_OK;
}

static fp8g_status check_ptrs(const uint8_t* a, const float* sa, const uint8_t* b,
                              const float* sb, uint16_t* d) {
  if (!a || !sa || !b || !sb || !d) return FP8G_ERR_NULL_PTR;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(sa, 4) ||
      !aligned(sb, 4))
    return FP8G_ERR_ALIGN;
  return FP8G_OK;
}

fp8g_status gemm_fp8_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b,
                                 const float* sb, uint16_t* d, int64_t M, int64_t N,
                                 int64_t K, hipStream_t stream) {
  if (M < 0) return FP8G_ERR_SHAPE;
  fp8g_status s = check_nk(N, K);
  if (s != FP8G_OK) return s;
  if (M == 0) return FP8G_OK;
  s = check_ptrs(a, sa, b, sb, d);
  if (s != FP8G_OK) return s;
  if ((M + 127) / 128 * ((N + 127) / 128) > 0x7FFFFFFF) return FP8G_ERR_UNSUPPORTED;
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  GemmArgs args{a, sa, b, sb, d, nullptr, M, M, N, K, 1, MODE_DENSE};
  return launch_gemm(args, dev, 0, nullptr, 0, stream) == hipSuccess ? FP8G_OK : FP8G_ERR_LAUNCH;
}

fp8g_status gemm_fp8_blockscaled_quant(const uint8_t* a, const float* sa, const uint8_t* b,
                                       const float* sb, uint16_t* d, uint8_t* qd, float* sd,
                                       int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M < 0) return FP8G_ERR_SHAPE;
  fp8g_status s = check_nk(N, K);
  if (s != FP8G_OK) return s;
  if (M == 0) return FP8G_OK;
  if (!a || !sa || !b || !sb || !qd || !sd) return FP8G_ERR_NULL_PTR;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(sa, 4) ||
      !aligned(sb, 4) || !aligned(qd, 4) || !aligned(sd, 4))
    return FP8G_ERR_ALIGN;
  if ((M + 127) / 128 * ((N + 127) / 128) > 0x7FFFFFFF) return FP8G_ERR_UNSUPPORTED;
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  GemmArgs args{a, sa, b, sb, d, nullptr, M, M, N, K, 1, MODE_DENSE};
  args.qd = qd;
  args.sd = sd;
  return launch_gemm(args, dev, 0, nullptr, 0, stream) == hipSuccess ? FP8G_OK : FP8G_ERR_LAUNCH;
}

fp8g_status gemm_fp8_pertensor_fmt(const uint8_t* a, int fmt_a, const float* scale_a,
                                   const uint8_t* b, int fmt_b, const float* scale_b,
                                   uint16_t* d, int64_t M, int64_t N, int64_t K,
                                   hipStream_t stream) {
  if (M < 0) return FP8G_ERR_SHAPE;
  if ((fmt_a != FP8G_FMT_E4M3 && fmt_a != FP8G_FMT_E5M2) ||
      (fmt_b != FP8G_FMT_E4M3 && fmt_b != FP8G_FMT_E5M2))
    return FP8G_ERR_UNSUPPORTED;
  fp8g_status s = check_nk(N, K);
  if (s != FP8G_OK) return s;
  if (M == 0) return FP8G_OK;
  s = check_ptrs(a, scale_a, b, scale_b, d);
  if (s != FP8G_OK) return s;
  if ((M + 127) / 128 * ((N + 127) / 128) > 0x7FFFFFFF) return FP8G_ERR_UNSUPPORTED;
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  GemmArgs args{a, scale_a, b, scale_b, d, nullptr, M, M, N, K, 1, MODE_PERTENSOR};
  args.fmts = fmt_a | (fmt_b << 4);
  return launch_gemm(args, dev, 0, nullptr, 0, stream) == hipSuccess ? FP8G_OK : FP8G_ERR_LAUNCH;
}

fp8g_status gemm_fp8_pertensor(const uint8_t* a, const float* scale_a, const uint8_t* b,
                               const float* scale_b, uint16_t* d, int64_t M, int64_t N,
                               int64_t K, hipStream_t stream) {
  return gemm_fp8_pertensor_fmt(a, FP8G_FMT_E4M3, scale_a, b, FP8G_FMT_E4M3, scale_b, d, M, N, K,
                                stream);
}

fp8g_status fp8_quantize_delayed(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                 int fmt, float* amax_history, int history_len, int slot,
                                 uint8_t* q, int64_t ldq, float* scale, hipStream_t stream) {
  if (rows < 0 || cols < 0) return FP8G_ERR_SHAPE;
  if (fmt != FP8G_FMT_E4M3 && fmt != FP8G_FMT_E5M2) return FP8G_ERR_UNSUPPORTED;
  if (history_len < 1 || history_len > 65536 || slot < 0 || slot >= history_len)
    return FP8G_ERR_SHAPE;
  if (!amax_history || !scale) return FP8G_ERR_NULL_PTR;
  if (!aligned(amax_history, 4) || !aligned(scale, 4)) return FP8G_ERR_ALIGN;
  const bool empty = rows == 0 || cols == 0;
  if (!empty) {
    if (cols % 4 != 0) return FP8G_ERR_SHAPE;
    if (!x || !q) return FP8G_ERR_NULL_PTR;
    if (ldx < cols || ldq < cols) return FP8G_ERR_STRIDE;
    if (!aligned(x, 16) || ldx % 4 != 0 || !aligned(q, 4) || ldq % 4 != 0) return FP8G_ERR_ALIGN;
    if ((cols + 1023) / 1024 > 0x7FFFFFFF) return FP8G_ERR_UNSUPPORTED;
  }
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  return launch_quantize_delayed(empty ? nullptr : x, empty ? 0 : rows, empty ? 0 : cols, ldx,
                                 fmt, amax_history, history_len, slot, q, ldq, scale,
                                 stream) == hipSuccess
             ? FP8G_OK
             : FP8G_ERR_LAUNCH;
}

static fp8g_status contiguous_checked(const uint8_t* a, const float* sa, const uint8_t* b,
                                      const float* sb, uint16_t* d,
                                      const int32_t* group_offsets, int G, int64_t M_total,
                                      int64_t N, int64_t K, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (G < 0 || M_total < 0 || M_total % 128 != 0) return FP8G_ERR_SHAPE;
  fp8g_status s = check_nk(N, K);
  if (s != FP8G_OK) return s;
  if (G == 0 || M_total == 0) return FP8G_OK;
  s = check_ptrs(a, sa, b, sb, d);
  if (s != FP8G_OK) return s;
  if (!group_offsets) return FP8G_ERR_NULL_PTR;
  if (!aligned(group_offsets, 4) || !aligned(workspace, 256)) return FP8G_ERR_ALIGN;
  if (M_total / 128 * ((N + 127) / 128) > 0x7FFFFFFF) return FP8G_ERR_UNSUPPORTED;
  if (!workspace && workspace_bytes != 0) return FP8G_ERR_NULL_PTR;
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  GemmArgs args{a, sa, b, sb, d, group_offsets, M_total, M_total, N, K, G, MODE_CONTIGUOUS};
  if (workspace) {
    const size_t need = contiguous_workspace_bytes(args, dev);
    if (workspace_bytes < need) return FP8G_ERR_WORKSPACE;
  }
  return launch_gemm(args, dev, 0, workspace, workspace_bytes, stream) == hipSuccess
             ? FP8G_OK
             : FP8G_ERR_LAUNCH;
}

fp8g_status grouped_gemm_fp8_contiguous(const uint8_t* a, const float* sa, const uint8_t* b,
                                        const float* sb, uint16_t* d,
                                        const int32_t* group_offsets, int G, int64_t M_total,
                                        int64_t N, int64_t K, hipStream_t stream) {
  return contiguous_checked(a, sa, b, sb, d, group_offsets, G, M_total, N, K, nullptr, 0, stream);
}

fp8g_status grouped_gemm_fp8_contiguous_workspace_size(int G, int64_t M_total, int64_t N,
                                                       int64_t K, size_t* bytes) {
  if (!bytes) return FP8G_ERR_NULL_PTR;
  *bytes = 0;
  if (G < 0 || M_total < 0 || M_total % 128 != 0) return FP8G_ERR_SHAPE;
  fp8g_status s = check_nk(N, K);
  if (s != FP8G_OK) return s;
  if (G == 0 || M_total == 0) return FP8G_OK;
  if (M_total / 128 * ((N + 127) / 128) > 0x7FFFFFFF) return FP8G_ERR_UNSUPPORTED;
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  GemmArgs args{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, M_total, M_total, N, K, G,
                MODE_CONTIGUOUS};
  *bytes = contiguous_workspace_bytes(args, dev);
  return FP8G_OK;
}

fp8g_status grouped_gemm_fp8_contiguous_ws(const uint8_t* a, const float* sa, const uint8_t* b,
                                           const float* sb, uint16_t* d,
                                           const int32_t* group_offsets, int G, int64_t M_total,
                                           int64_t N, int64_t K, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  return contiguous_checked(a, sa, b, sb, d, group_offsets, G, M_total, N, K, workspace,
                            workspace_bytes, stream);
}

fp8g_status grouped_gemm_fp8_contiguous_noalloc(const uint8_t* a, const float* sa,
                                                const uint8_t* b, const float* sb, uint16_t* d,
                                                const int32_t* group_offsets, int G,
                                                int64_t M_total, int64_t N, int64_t K,
                                                hipStream_t stream) {
  // every check of the workspace call, except that the workspace is the
  // library's scratch array: reject what it cannot hold, then look it up
  if (G < 0 || M_total < 0 || M_total % 128 != 0) return FP8G_ERR_SHAPE;
  fp8g_status s = check_nk(N, K);
  if (s != FP8G_OK) return s;
  if (G == 0 || M_total == 0) return FP8G_OK;
  s = check_ptrs(a, sa, b, sb, d);
  if (s != FP8G_OK) return s;
  if (!group_offsets) return FP8G_ERR_NULL_PTR;
  if (!aligned(group_offsets, 4)) return FP8G_ERR_ALIGN;
  if (M_total / 128 * ((N + 127) / 128) > 0x7FFFFFFF) return FP8G_ERR_UNSUPPORTED;
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  GemmArgs args{a, sa, b, sb, d, group_offsets, M_total, M_total, N, K, G, MODE_CONTIGUOUS};
  if (contiguous_workspace_bytes(args, dev) > noalloc_scratch_bytes()) return FP8G_ERR_WORKSPACE;
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) return FP8G_ERR_DEVICE;
  void* ws = scratch_ptr(device);
  if (!ws) return FP8G_ERR_DEVICE;
  return launch_gemm(args, dev, 0, ws, noalloc_scratch_bytes(), stream) == hipSuccess
             ? FP8G_OK
             : FP8G_ERR_LAUNCH;
}

fp8g_status grouped_gemm_fp8_masked(const uint8_t* a, const float* sa, const uint8_t* b,
                                    const float* sb, uint16_t* d, const int32_t* masked_m,
                                    int G, int64_t max_m, int64_t N, int64_t K,
                                    int expected_m, hipStream_t stream) {
  if (G < 0 || max_m < 0) return FP8G_ERR_SHAPE;
  fp8g_status s = check_nk(N, K);
  if (s != FP8G_OK) return s;
  if (G == 0 || max_m == 0) return FP8G_OK;
  s = check_ptrs(a, sa, b, sb, d);
  if (s != FP8G_OK) return s;
  if (!masked_m) return FP8G_ERR_NULL_PTR;
  if (!aligned(masked_m, 4)) return FP8G_ERR_ALIGN;
  if (G > 1024 || max_m > (1 << 30) ||
      (int64_t)G * ((max_m + 127) / 128) * ((N + 127) / 128) > 0x7FFFFFFF)
    return FP8G_ERR_UNSUPPORTED;
  DeviceInfo dev;
  if (current_device_info(&dev) != 0) return FP8G_ERR_DEVICE;
  GemmArgs args{a, sa, b, sb, d, masked_m, max_m, (int64_t)G * max_m, N, K, G, MODE_MASKED};
  return launch_gemm(args, dev, expected_m, nullptr, 0, stream) == hipSuccess ? FP8G_OK
                                                                         : FP8G_ERR_LAUNCH;
}

}  // extern "C"
