/*
 * fp8gemm.h -- C ABI of the MI355X (gfx950) FP8 block-scaled GEMM library.
 *
 * The library quantises fp32 matrices to FP8 e4m3 with one fp32 scale per
 * block, and multiplies e4m3 operands with per-block scales into a bf16
 * result, densely or for every expert of a mixture-of-experts layer in one
 * launch. Method sources (the three pages the design follows):
 *   [czchanglian] m.czchanglian.com/news/60438 (DeepGEMM teardown essay)
 *   [gtnt]        www.gtnt.cn/news/117510, "生产级 FP8 GEMM 算子对齐与 Tensor Core 峰值利用率调优"
 *   [nxmr]        www.nxmr.cn/news/131680 (DeepGEMM explainer)
 *
 * Conventions shared by every entry point:
 *  - Every pointer is a device pointer on the current HIP device, owned by
 *    the caller. The library allocates no device memory, per call or
 *    otherwise; scratch memory (the split tail of the contiguous call) comes
 *    from the caller (grouped_gemm_fp8_contiguous_ws). Its only state is a
 *    per-device record of the architecture and compute-unit count, filled on
 *    first use.
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *    without waiting for it. The host never synchronises.
 *  - Scales are IEEE fp32; e4m3 codes are the OCP 8-bit float layout (sign,
 *    4 exponent bits biased by 7, 3 mantissa bits, max 448, NaN = 0x7F/0xFF);
 *    bf16 values are passed as their 16-bit patterns (uint16_t).
 *  - Every host-checkable precondition is checked before anything is
 *    launched; a failed check returns its status and launches nothing.
 *    Calls never abort the process.
 *  - A call with zero rows (or zero groups) is a no-op that returns FP8G_OK.
 */
#ifndef FP8GEMM_H
#define FP8GEMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int fp8g_status;
enum {
  FP8G_OK = 0,
  FP8G_ERR_NULL_PTR = 1,     /* a required pointer is NULL */
  FP8G_ERR_SHAPE = 2,        /* a size is negative or not a multiple it must be */
  FP8G_ERR_ALIGN = 3,        /* a pointer or leading dimension is misaligned */
  FP8G_ERR_STRIDE = 4,       /* a leading dimension or scale stride is too small */
  FP8G_ERR_DEVICE = 5,       /* no usable gfx950 device is current */
  FP8G_ERR_LAUNCH = 6,       /* the HIP launch reported an error */
  FP8G_ERR_UNSUPPORTED = 7,  /* a valid request the library does not handle */
  FP8G_ERR_WORKSPACE = 8     /* the workspace given is smaller than the call needs */
};

/* Static text for a status code (never NULL). */
const char* fp8g_status_string(fp8g_status status);

/* ABI version of this header; bumped on any signature change. */
int fp8g_abi_version(void);

/*
 * fp8_quantize -- blockwise e4m3 quantisation with fp32 scales.
 *
 * Source: nxmr §3.1 (block amax, scale = amax / FP8 max, divide to
 * quantise, multiply to dequantise); czchanglian §5.2 (initial scale
 * max_val / 448, independent per tensor); czchanglian §2.2 (activations
 * grouped per token, weights per channel, K cut into blocks); nxmr §5.1
 * (128x128 blocks, round to nearest by default).
 *
 * x      fp32 [rows][ldx], row-major; 16-byte aligned, ldx % 4 == 0, ldx >= cols.
 * rows   >= 0.  cols > 0 (when rows > 0), cols % 16 == 0.
 * block_rows  1 (1x128 per-token blocks, for the activation operand A) or
 *        128 (128x128 blocks, for the weight operand B). Block (i, j) covers
 *        rows [i*block_rows, min(rows, (i+1)*block_rows)) and columns
 *        [128 j, min(cols, 128 j + 128)). A last partial block (of rows, or
 *        of columns when cols is not a multiple of 128) takes the elements
 *        that are there (czchanglian §5.1: the same codes and scales as
 *        zero padding to a multiple of 128).
 * q      uint8 e4m3 codes [rows][ldq]; 4-byte aligned, ldq % 4 == 0, ldq >= cols.
 * scales fp32; the scale of block (i, j) is written to
 *        scales[i * s_stride_row + j * s_stride_col] (strides in elements,
 *        both >= 1). For a GEMM A operand use s_stride_row = 1,
 *        s_stride_col = rows (layout [ceil(cols/128)][rows]); for a B operand
 *        use s_stride_row = ceil(cols/128), s_stride_col = 1 (layout
 *        [ceil(rows/128)][ceil(cols/128)]). Stacked expert weights [G][N][K]
 *        are one call with rows = G*N (N a multiple of 128, so that no
 *        128-row block spans two experts).
 *
 * Per block: amax = max |x| (NaN skipped); s = fl32(amax / 448) by IEEE
 * division; every element becomes rne_e4m3(clamp(fl32(x / s), -448, 448)).
 * s == 0 gives signed-zero codes; NaN elements give 0x7F with their sign;
 * no denormal is flushed. Output is bit-exact with respect to this
 * definition.
 *
 * Errors (nothing is launched): FP8G_ERR_SHAPE, _NULL_PTR, _STRIDE, _ALIGN
 * as stated above; FP8G_ERR_UNSUPPORTED for more than 65535 column blocks,
 * or, with block_rows == 128, ldx > 2^26 or ldq > 2^28 (the 128x128 kernel
 * addresses 8 rows from one base with 32-bit offsets).
 */
fp8g_status fp8_quantize(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                         int block_rows, uint8_t* q, int64_t ldq, float* scales,
                         int64_t s_stride_row, int64_t s_stride_col, hipStream_t stream);

/*
 * fp8_quantize_bf16 -- fp8_quantize for a bf16 input (activations usually
 * arrive in bf16; czchanglian §5.1 and nxmr §3.1 have the scales computed
 * as the data is loaded rather than in a separate fp32 pass).
 *
 * x      bf16 bit patterns [rows][ldx] (uint16_t), row-major; 8-byte
 *        aligned, ldx % 4 == 0, ldx >= cols.
 * Every other argument, the blocking, the errors and the result are those
 * of fp8_quantize applied to the exact fp32 values of the bf16 inputs
 * (every bf16 value is an fp32 value): codes and scales are bit-identical
 * to fp8_quantize on the widened array.
 */
fp8g_status fp8_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                              int block_rows, uint8_t* q, int64_t ldq, float* scales,
                              int64_t s_stride_row, int64_t s_stride_col, hipStream_t stream);

/*
 * fp8_quantize_tensor -- e4m3 quantisation with ONE fp32 scale for the whole
 * matrix (per-tensor scaling).
 *
 * Source: gtnt, Triton kernel section (one scale_a and one scale_b per
 * operand, applied in the epilogue); czchanglian §2.2 (per-tensor scaling
 * is the coarse form that a single outlier channel spoils); czchanglian
 * §5.2 (initial scale max_val / 448).
 *
 * x      fp32 [rows][ldx], 16-byte aligned, ldx % 4 == 0, ldx >= cols.
 * rows, cols >= 0; cols % 4 == 0 (when the matrix is not empty).
 * q      uint8 e4m3 codes [rows][ldq], 4-byte aligned, ldq % 4 == 0.
 * scale  DEVICE float [1], 4-byte aligned: receives s = fl32(amax / 448).
 * The result is fp8_quantize's element rule with a single block covering
 * every element: amax over the whole matrix (NaN skipped), one IEEE
 * division for s, q = rne_e4m3(clamp(fl32(x / s), -448, 448)); bit-exact.
 * Three kernels are enqueued on `stream` (amax reduction into *scale,
 * encoding, scale); *scale holds the amax in between.
 *
 * Errors (nothing is launched): FP8G_ERR_SHAPE (negative sizes, cols % 4),
 * FP8G_ERR_NULL_PTR, FP8G_ERR_STRIDE, FP8G_ERR_ALIGN as stated,
 * FP8G_ERR_DEVICE. An empty matrix is a no-op and leaves *scale unchanged.
 */
fp8g_status fp8_quantize_tensor(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* q, int64_t ldq, float* scale, hipStream_t stream);

/*
 * gemm_fp8_blockscaled -- D = bf16( sum_kb sa[kb][m] * sb[n/128][kb] *
 *                                   sum_{k in block kb} a[m][k] * b[n][k] )
 *
 * Source: czchanglian §2.2-§2.3 (fine-grained scales handled inside the
 * GEMM pipeline, FP32 accumulation over all of K, rounding only on
 * write-back); gtnt pipeline figure and Triton kernel (scale multiply fused
 * into the epilogue, bf16 output); nxmr §3.3 (operands used without a
 * transpose: both K-contiguous).
 *
 * a   e4m3 [M][K] row-major (K contiguous), 16-byte aligned.
 * sa  fp32 [KB][M], KB = ceil(K/128): sa[kb*M + m] is the scale of row m,
 *     K block kb.
 * b   e4m3 [N][K] row-major (K contiguous), 16-byte aligned.
 * sb  fp32 [ceil(N/128)][KB]: sb[(n/128)*KB + kb].
 * d   bf16 bits [M][N] row-major, 16-byte aligned; fully overwritten.
 * M >= 0 (any value); N > 0, N % 16 == 0; K > 0, K % 16 == 0. N and K need
 * not be multiples of 128 (czchanglian §5.1 pads outside and slices the
 * padding off; the library does that in the kernel): the last K block, and
 * the last 128-row block of b, hold the elements that are there, which is
 * the zero-padded product exactly. Multiples of 16 keep operand rows
 * 16-byte aligned for the vector copies.
 * Accumulation is fp32 per 128-wide K block, promoted into an fp32
 * accumulator with the block's scale product; output rounds to nearest even.
 *
 * Errors (nothing is launched): FP8G_ERR_SHAPE for M < 0 or N, K not
 * positive multiples of 16; FP8G_ERR_NULL_PTR, FP8G_ERR_ALIGN for the
 * pointers above; FP8G_ERR_UNSUPPORTED for K > 2^24 (operand rows are
 * addressed with 32-bit offsets from a tile's first row), ceil(N/128) > 2^20,
 * or more than 2^31 - 1 tiles of 128x128; FP8G_ERR_DEVICE when the current
 * device is not a gfx950.
 */
fp8g_status gemm_fp8_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b,
                                 const float* sb, uint16_t* d, int64_t M, int64_t N,
                                 int64_t K, hipStream_t stream);

/*
 * gemm_fp8_blockscaled_quant -- gemm_fp8_blockscaled whose epilogue also
 * quantises its own bf16 result for the next GEMM (the quantiser fused into
 * the producer of the activations).
 *
 * Source: nxmr §3.1 (the scale is computed while the data is loaded, not in
 * a separate pass) and czchanglian §2.2 (per-token activation scales, K cut
 * into blocks); the result is gemm_fp8_blockscaled's, then fp8_quantize_bf16
 * with block_rows = 1 applied to it, in one kernel.
 *
 * a, sa, b, sb, M, N, K as for gemm_fp8_blockscaled.
 * d    bf16 bits [M][N] (16-byte aligned), or NULL: the bf16 result is then
 *      not stored (it is still what is quantised).
 * qd   uint8 e4m3 codes [M][N], 4-byte aligned: row m's 128-column block nb
 *      quantised with one scale (the next GEMM's A operand).
 * sd   fp32 [ceil(N/128)][M], 4-byte aligned: sd[nb * M + m] is that block's scale
 *      (the next GEMM's sa layout).
 * Codes and scales are bit-identical to fp8_quantize_bf16(d, ..., block_rows
 * = 1, s_stride_row = 1, s_stride_col = M) on the bf16 result.
 * Errors: those of gemm_fp8_blockscaled, FP8G_ERR_NULL_PTR for qd or sd,
 * FP8G_ERR_ALIGN for the alignments above.
 */
fp8g_status gemm_fp8_blockscaled_quant(const uint8_t* a, const float* sa, const uint8_t* b,
                                       const float* sb, uint16_t* d, uint8_t* qd, float* sd,
                                       int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * gemm_fp8_pertensor -- D = bf16( fl32(scale_a * scale_b) * acc ),
 *   acc[m][n] = fp32 sum over all of K of a[m][k] * b[n][k]
 *
 * Source: gtnt, Triton kernel section (acc += dot over K blocks in fp32,
 * then acc * (scale_a * scale_b) cast to bf16) and its H100 table (the
 * 4096x8192x8192 shape); czchanglian §2.3 (fp32 accumulation, rounding only
 * on write-back). The block-scaled call with every scale equal computes the
 * same value; this one needs no per-block promotion, so the MFMA keeps the
 * running sum itself.
 *
 * a, b, d, M, N, K as for gemm_fp8_blockscaled (same layouts, alignment and
 * limits). scale_a, scale_b: DEVICE float [1] each, 4-byte aligned.
 * Errors: those of gemm_fp8_blockscaled.
 */
fp8g_status gemm_fp8_pertensor(const uint8_t* a, const float* scale_a, const uint8_t* b,
                               const float* scale_b, uint16_t* d, int64_t M, int64_t N,
                               int64_t K, hipStream_t stream);

/* ---- e5m2 operands and delayed scaling (czchanglian §2.1, §2.3; gtnt
 * E4M3-vs-E5M2 part) ---------------------------------------------------------
 * e5m2 (5 exponent bits, 2 mantissa bits, largest finite value 57344, with
 * infinities) is the pages' format for gradients and other wide-range data;
 * delayed scaling quantises a step with a scale gathered before it, instead
 * of a statistics pass over the data being quantised. */

/* Format codes. */
enum { FP8G_FMT_E4M3 = 0, FP8G_FMT_E5M2 = 1 };

/*
 * gemm_fp8_pertensor_fmt -- gemm_fp8_pertensor with each operand's format
 * given: fmt_a, fmt_b in { FP8G_FMT_E4M3, FP8G_FMT_E5M2 } (a backward GEMM
 * takes its gradient operand in e5m2). D = bf16( fl32(scale_a * scale_b) *
 * acc ), acc the fp32 sum over K of dec_a(a[m][k]) * dec_b(b[n][k]).
 * Arguments, layouts and errors as for gemm_fp8_pertensor, plus
 * FP8G_ERR_UNSUPPORTED for an unknown format code.
 */
fp8g_status gemm_fp8_pertensor_fmt(const uint8_t* a, int fmt_a, const float* scale_a,
                                   const uint8_t* b, int fmt_b, const float* scale_b,
                                   uint16_t* d, int64_t M, int64_t N, int64_t K,
                                   hipStream_t stream);

/*
 * fp8_quantize_delayed -- one step of delayed (amax-history) per-tensor
 * scaling:
 *   s = RN(max(amax_history[0..history_len)) / FP8max)   (1 if no entry > 0;
 *        NaN entries skipped; FP8max 448 for e4m3, 57344 for e5m2)
 *   q[r][c] = enc(sat(RN(x[r][c] / s)))                   (codes in fmt)
 *   amax_history[slot] = max |x| over the matrix          (NaN skipped)
 * The scale is taken from the history as it was before the call; *scale
 * receives it. Finite quotients saturate to +-FP8max (the data may have
 * outgrown the scale); an infinite element gives the e5m2 infinity code,
 * or the e4m3 NaN code of its sign; a NaN element gives 0x7F with its sign.
 * s == 0 (a history whose max underflows) gives signed zeros.
 *
 * x: DEVICE float [rows][ldx], 16-byte aligned, ldx % 4 == 0, cols % 4 == 0.
 * q: DEVICE uint8 [rows][ldq], 4-byte aligned, ldq % 4 == 0.
 * amax_history: DEVICE float [history_len] (1..65536), read and written;
 * slot in [0, history_len): the entry this step's amax replaces (the caller
 * rotates it). scale: DEVICE float [1]. All 4-byte aligned. An empty matrix
 * still takes its step (scale written, history[slot] = 0).
 * Errors (nothing is launched): FP8G_ERR_SHAPE (negative sizes, cols % 4,
 * history_len or slot out of range), FP8G_ERR_NULL_PTR, FP8G_ERR_STRIDE,
 * FP8G_ERR_ALIGN as stated, FP8G_ERR_UNSUPPORTED (unknown format),
 * FP8G_ERR_DEVICE.
 */
fp8g_status fp8_quantize_delayed(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                 int fmt, float* amax_history, int history_len, int slot,
                                 uint8_t* q, int64_t ldq, float* scale, hipStream_t stream);

/*
 * grouped_gemm_fp8_contiguous -- every expert's GEMM in one launch,
 * contiguous layout.
 *
 * Source: nxmr §3.2 (grouped GEMM of several experts packed into one
 * kernel, each expert's work mapped to its own workgroups); czchanglian
 * §1.2 (one launch instead of one per expert) and §5.3 (group id plus
 * token offsets; each expert's rows contiguous and movable in blocks);
 * czchanglian §5.1 (padding done outside the library).
 *
 * a    e4m3 [M_total][K]; expert g owns rows
 *      [group_offsets[g], group_offsets[g+1]).
 * sa   fp32 [ceil(K/128)][M_total] (as for the dense call, with M = M_total).
 * b    e4m3 [G][N][K]: expert g's weights at b + g*N*K.
 * sb   fp32 [G][ceil(N/128)][ceil(K/128)].
 * d    bf16 bits [M_total][N]; every row is written.
 * group_offsets  DEVICE int32 [G+1]: group_offsets[0] = 0,
 *      group_offsets[G] = M_total, non-decreasing, every entry a multiple
 *      of 128. The kernel reads it; the host cannot check it without a
 *      synchronisation, so an array breaking these rules is undefined
 *      behaviour (the kernel clamps every row index it derives into
 *      [0, M_total) and never reads or writes out of bounds).
 * G >= 0; M_total >= 0, M_total % 128 == 0; N, K as for the dense call.
 *
 *
 * This call uses no scratch memory: every tile runs over all of K in one
 * workgroup. grouped_gemm_fp8_contiguous_ws is the same call with a
 * caller-owned workspace, which lets it split a part-full last round of
 * tiles along K (faster when the tile count is just above a multiple of
 * the compute-unit count).
 *
 * Errors (nothing is launched): as for the dense call, plus FP8G_ERR_SHAPE
 * for G < 0 or M_total not a non-negative multiple of 128,
 * FP8G_ERR_NULL_PTR / FP8G_ERR_ALIGN for group_offsets (4-byte aligned),
 * FP8G_ERR_UNSUPPORTED for more than 2^31 - 1 tiles of 128x128.
 */
fp8g_status grouped_gemm_fp8_contiguous(const uint8_t* a, const float* sa, const uint8_t* b,
                                        const float* sb, uint16_t* d,
                                        const int32_t* group_offsets, int G, int64_t M_total,
                                        int64_t N, int64_t K, hipStream_t stream);

/*
 * grouped_gemm_fp8_contiguous_workspace_size -- bytes of workspace that
 * grouped_gemm_fp8_contiguous_ws needs for these sizes on the current
 * device (0: the call never splits, any workspace is ignored).
 *
 * Errors: FP8G_ERR_NULL_PTR for bytes == NULL, otherwise those of the
 * contiguous call for the same sizes (*bytes is then 0).
 */
fp8g_status grouped_gemm_fp8_contiguous_workspace_size(int G, int64_t M_total, int64_t N,
                                                       int64_t K, size_t* bytes);

/*
 * grouped_gemm_fp8_contiguous_ws -- grouped_gemm_fp8_contiguous with a
 * caller-owned device workspace for a split tail.
 *
 * Source: as for grouped_gemm_fp8_contiguous. The split keeps the method:
 * each K piece sums its K blocks with the same per-block promotion in fp32,
 * the pieces are added in fp32 in a fixed order, and the sum is rounded once
 * to bf16 (czchanglian §2.3: fp32 accumulation, rounding only on
 * write-back); only the order of the fp32 additions differs from the
 * unsplit call.
 *
 * workspace        device memory, 256-byte aligned, at least
 *                  grouped_gemm_fp8_contiguous_workspace_size bytes, or NULL
 *                  (then workspace_bytes must be 0 and the call runs as
 *                  grouped_gemm_fp8_contiguous). Its contents need no
 *                  initialisation and are garbage afterwards. The call uses
 *                  it until its last kernel has run on `stream`: calls that
 *                  share one workspace must be ordered (same stream, or
 *                  synchronised), or they race.
 * workspace_bytes  its size.
 * Every other argument as for grouped_gemm_fp8_contiguous.
 *
 * Errors: those of grouped_gemm_fp8_contiguous; FP8G_ERR_ALIGN for a
 * misaligned workspace; FP8G_ERR_NULL_PTR for workspace == NULL with
 * workspace_bytes != 0; FP8G_ERR_WORKSPACE for a workspace smaller than the
 * size query returns.
 */
fp8g_status grouped_gemm_fp8_contiguous_ws(const uint8_t* a, const float* sa, const uint8_t* b,
                                           const float* sb, uint16_t* d,
                                           const int32_t* group_offsets, int G, int64_t M_total,
                                           int64_t N, int64_t K, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream);

/*
 * grouped_gemm_fp8_contiguous_noalloc -- grouped_gemm_fp8_contiguous_ws
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the split
 * tail's workspace is a fixed array inside the library's code object (one
 * copy per GPU, 64 MiB plus a 4 KiB header, enough for launches of up to 256
 * workgroups, held until the process ends). The call allocates nothing and
 * calls no allocating routine; the first call on a device looks up that
 * device's copy of the array.
 *
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, not synchronised) race on it and must not be
 * issued. Nothing in it needs clearing between calls (every value the
 * reduction reads is written by the same call), and it keeps the last
 * call's contents.
 *
 * Arguments, results and errors are those of grouped_gemm_fp8_contiguous,
 * plus FP8G_ERR_WORKSPACE when a call would need more scratch than the
 * array holds (a GPU with more than 256 compute units), and FP8G_ERR_DEVICE
 * when the array's device address cannot be looked up.
 */
fp8g_status grouped_gemm_fp8_contiguous_noalloc(const uint8_t* a, const float* sa,
                                                const uint8_t* b, const float* sb, uint16_t* d,
                                                const int32_t* group_offsets, int G,
                                                int64_t M_total, int64_t N, int64_t K,
                                                hipStream_t stream);

/*
 * grouped_gemm_fp8_masked -- every expert's GEMM in one launch, masked
 * layout: each expert has a fixed slab of max_m rows, of which the first
 * masked_m[g] are valid.
 *
 * Source: as for the contiguous call (nxmr §3.2, czchanglian §1.2); the
 * per-expert valid-row count replaces the offsets.
 *
 * a    e4m3 [G][max_m][K].
 * sa   fp32 [ceil(K/128)][G*max_m]: sa[kb*(G*max_m) + g*max_m + r].
 * b    e4m3 [G][N][K];  sb fp32 [G][ceil(N/128)][ceil(K/128)].
 * d    bf16 bits [G][max_m][N]. Rows r < masked_m[g] of expert g are
 *      written; every other row of d is left untouched.
 * masked_m  DEVICE int32 [G]; each value is clamped to [0, max_m] by the
 *      kernel. Experts with no valid row read none of their weights.
 * expected_m  host hint of the typical masked_m (0 = unknown); it may only
 *      change the tile configuration, never the result.
 * G >= 0; max_m >= 0; N, K as for the dense call.
 *
 * Errors (nothing is launched): as for the dense call, plus FP8G_ERR_SHAPE
 * for G < 0 or max_m < 0, FP8G_ERR_NULL_PTR / FP8G_ERR_ALIGN for masked_m
 * (4-byte aligned), FP8G_ERR_UNSUPPORTED for G > 1024 (the per-expert
 * schedule lives in LDS), max_m > 2^30, or more than 2^31 - 1 tiles of
 * 128x128 over all experts.
 */
fp8g_status grouped_gemm_fp8_masked(const uint8_t* a, const float* sa, const uint8_t* b,
                                    const float* sb, uint16_t* d, const int32_t* masked_m,
                                    int G, int64_t max_m, int64_t N, int64_t K,
                                    int expected_m, hipStream_t stream);

/*
 * fp8g_clock_probe -- diagnostic: the shader clock the GPU holds right now.
 *
 * Enqueues one wave that counts shader-clock cycles over `ticks` ticks of
 * the GPU's constant 100 MHz counter and writes out[0] = shader cycles,
 * out[1] = 100 MHz ticks elapsed (clock in Hz = out[0] / out[1] * 1e8).
 * Placed between kernels on a stream, it reads the clock the chip holds
 * under that load (the benchmark's hygiene of knowing the clock: czchanglian
 * §4.3). Not part of the method; it computes nothing else.
 *
 * out    DEVICE uint64 [2], 8-byte aligned.  ticks  1 .. 1000000 (10 ms).
 * Errors: FP8G_ERR_NULL_PTR, FP8G_ERR_ALIGN, FP8G_ERR_SHAPE (ticks out of
 * range), FP8G_ERR_DEVICE, FP8G_ERR_LAUNCH.
 */
fp8g_status fp8g_clock_probe(uint64_t* out, int ticks, hipStream_t stream);

/* ---- Kernel table and warm-up (nxmr §2.3) ----------------------------------
 * The pages' library compiles a kernel per GEMM shape at run time and caches
 * it, so the first call of a shape pays for compilation, and advises warming
 * the common shapes up when a service starts. This library compiles every
 * kernel ahead of time: a generic kernel per layout and tile configuration,
 * plus kernels with N and K fixed at compile time for the hot shapes
 * (4096x8192x8192 block-scaled and per-tensor; contiguous
 * experts N4096 K7168; masked experts N7168 K2048; small-M K7168). A call
 * whose shape matches an entry runs the specialised kernel; both give the
 * same bits. What remains of the first-call cost is loading the code
 * objects onto the device, which fp8g_warmup does ahead of time. */

/* Layout codes of fp8g_gemm_kernel_name. */
enum {
  FP8G_LAYOUT_DENSE = 0,       /* gemm_fp8_blockscaled (and _quant) */
  FP8G_LAYOUT_CONTIGUOUS = 1,  /* grouped_gemm_fp8_contiguous* */
  FP8G_LAYOUT_MASKED = 2,      /* grouped_gemm_fp8_masked */
  FP8G_LAYOUT_PERTENSOR = 3    /* gemm_fp8_pertensor */
};

/* Loads the code object of every kernel of the library onto the current
 * device (and resolves the allocation-free entry point's scratch array), so
 * that no later call pays for it. Synchronous, host-side only: launches
 * nothing and allocates nothing. Safe to call more than once.
 * Errors: FP8G_ERR_DEVICE (no gfx950 device current), FP8G_ERR_LAUNCH (the
 * runtime could not load a kernel). */
fp8g_status fp8g_warmup(void);

/* Process-wide switch between the shape-specialised kernels (enable != 0,
 * the default) and the generic ones for every shape. The results are
 * bit-identical either way; the switch exists to measure the difference.
 * Takes effect for calls made after it returns. Always FP8G_OK. */
fp8g_status fp8g_set_shape_specialisation(int enable);

/* The kernel a GEMM call of this shape would launch, as text into buf (at
 * most len bytes including the terminating NUL; truncated like snprintf).
 * layout: FP8G_LAYOUT_*; rows: M (dense, per-tensor), M_total
 * (contiguous) or max_m (masked); G experts (grouped layouts);
 * expected_m: the masked call's hint (0 = none); quant != 0: the dense
 * call with the quantising epilogue. Launches nothing.
 * Errors: FP8G_ERR_NULL_PTR (buf), FP8G_ERR_SHAPE (len 0, unknown layout,
 * negative rows or G, N or K not positive multiples of 16),
 * FP8G_ERR_UNSUPPORTED (quant with a layout other than dense). */
fp8g_status fp8g_gemm_kernel_name(int layout, int64_t rows, int64_t N, int64_t K, int G,
                                  int expected_m, int quant, char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* FP8GEMM_H */
