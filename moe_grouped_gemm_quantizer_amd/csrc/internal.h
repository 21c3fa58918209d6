// Internal declarations shared by the HIP translation units of libfp8gemm.
// Nothing here is part of the C ABI (include/fp8gemm.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <vector>
#include <stdint.h>

namespace fp8g {

// Per-device facts the launchers need, queried once per device.
struct DeviceInfo {
  int ok;          // 1 when the device is a usable gfx950
  int cu_count;    // compute units (256 on MI355X)
};
// Fills *info for the current device; returns 0 on success.
int current_device_info(DeviceInfo* info);

// Launchers (arguments already validated by the C entry points). The
// quantiser takes fp32 (T = float) or bf16 bit patterns (T = uint16_t).
template <typename T>
hipError_t launch_quantize(const T* x, int64_t rows, int64_t cols, int64_t ldx,
                           int block_rows, uint8_t* q, int64_t ldq, float* scales,
                           int64_t s_stride_row, int64_t s_stride_col, hipStream_t stream,
                           int cu_count);

// MODE_PERTENSOR: one scale per operand (sa, sb point at one float each);
// the MFMA accumulates over all of K and the epilogue applies sa * sb once.
// Per-tensor quantisation: one scale (written to *scale) for the whole matrix.
hipError_t launch_quantize_tensor(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* scale, hipStream_t stream);

enum GemmMode { MODE_DENSE = 0, MODE_CONTIGUOUS = 1, MODE_MASKED = 2, MODE_PERTENSOR = 3 };

struct GemmArgs {
  const uint8_t* a;        // e4m3 rows, K contiguous
  const float* sa;         // [K/128][sa_ld]
  const uint8_t* b;        // e4m3 [G][N][K]
  const float* sb;         // [G][N/128][K/128]
  uint16_t* d;             // bf16 bits, rows of N
  const int32_t* group;    // contiguous: offsets [G+1]; masked: counts [G]; dense: null
  int64_t rows;            // dense: M; contiguous: M_total; masked: max_m
  int64_t sa_ld;           // row count of the sa layout (M, M_total or G*max_m)
  int64_t N;
  int64_t K;
  int G;
  int mode;
  // Set by the launcher only (the entry points leave the defaults):
  int split_base = 0;      // contiguous, splits > 1: tiles from here on run as K pieces
  int splits = 1;          // contiguous: K pieces per tile past split_base (1: none)
  float* ws = nullptr;     // split workspace: fp32 partial tiles [piece][BM][BN]
  struct SplitMeta* ws_meta = nullptr;  // split workspace: what the reduction reads
  // Dense only, set by the fused entry point: the bf16 result is also
  // quantised per 1x128 block into qd [rows][N] (e4m3) with scales
  // sd [N/128][rows]; d may then be null (no bf16 output).
  uint8_t* qd = nullptr;
  float* sd = nullptr;
  // Per-tensor only: operand formats, fmt_a | fmt_b << 4 (Fp8Format codes).
  int fmts = 0;
};

// Written by the GEMM kernel for the reduction of its split tail: the
// number of tail tiles (0: nothing to reduce), the pieces per tile, and
// where each tail tile's output goes. SplitTile records follow the header.
struct SplitTile {
  int64_t d_off;           // offset of the tile's first output element in d
  int mvalid, nvalid;      // rows and columns of the tile that exist
};
struct SplitMeta {
  int tail;
  int splits;
  int pad[2];
};
// Launch of a validated GEMM call. ws/ws_bytes: caller-owned workspace for a
// contiguous call's split tail (null/0: the call runs unsplit; a workspace
// smaller than contiguous_workspace_bytes is not used).
hipError_t launch_gemm(const GemmArgs& args, const DeviceInfo& dev, int expected_m, void* ws,
                       size_t ws_bytes, hipStream_t stream);
// Workspace a contiguous call with these sizes can use (0: it never splits).
size_t contiguous_workspace_bytes(const GemmArgs& args, const DeviceInfo& dev);

// FP8 element formats (the MFMA's operand format codes).
enum Fp8Format { FMT_E4M3 = 0, FMT_E5M2 = 1 };

// Delayed-scaling quantiser (quantize.hip): scale from the amax window,
// codes in format fmt, this step's amax into history[slot].
hipError_t launch_quantize_delayed(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                   int fmt, float* history, int hist_len, int slot, uint8_t* q,
                                   int64_t ldq, float* scale, hipStream_t stream);

// Kernel table (gemm.hip): the text naming the kernel a GEMM call of these
// arguments launches (snprintf's return value), and the process-wide switch
// between the shape-specialised instantiations and the generic ones (on by
// default; both give the same bits).
int describe_gemm(const GemmArgs& args, int expected_m, char* buf, size_t len);
void set_shape_specialisation(int enable);
// Every kernel of the library (for warm-up: loading each one's code object
// onto the current device ahead of the first call).
void gemm_kernels(std::vector<const void*>& out);
void quantize_kernels(std::vector<const void*>& out);

// The allocation-free contiguous entry point's scratch: its size, and its
// device address on `device` (looked up once per device; nullptr on failure;
// call with that device current).
size_t noalloc_scratch_bytes();
void* scratch_ptr(int device);

}  // namespace fp8g
