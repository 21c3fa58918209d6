// FP8 block-scaled GEMM for gfx950: dense, grouped-contiguous and
// grouped-masked, sharing one persistent mainloop.
//
// Method (czchanglian §2.2-§2.3, gtnt pipeline figure and Triton kernel,
// nxmr §3.1-§3.3): e4m3 operands, a 1x128 scale per (row, K block) of A and
// a 128x128 scale per (N block, K block) of B; fp32 accumulation over all of
// K with each 128-wide K block's partial sum multiplied by its two scales
// before it is added ("promotion"); bf16 output rounded once at the end.
//
// Mapping onto CDNA4:
//  * One v_mfma_f32_16x16x128_f8f6f4 covers a 16x16 output over a whole
//    128-wide K block, so each MFMA's fp32 result is exactly one block's
//    partial sum: it is promoted with one FMA per element,
//    acc += part * (sa[row] * sb), with sa*sb formed once per row and block.
//    The promotion needs the accumulator in VGPRs (the VALU cannot read
//    AGPRs), which caps a wave's tile at 64x128 (128 fp32 accumulators per
//    lane). Such a tile reads (64 + 128) * 128 bytes of LDS per 32 MFMAs,
//    about 94 B/clk per CU with every MFMA pipe busy, under the LDS's 128.
//  * B is the MFMA's first operand, so each result is the transposed 16x16
//    tile: a lane holds one output row and four adjacent columns, which
//    makes the promotion factor one value per lane and MFMA tile and the
//    bf16 store one 8-byte write.
//  * Workgroup tiles: 256x256 with 8 waves of 64x128 (two per SIMD, so one
//    wave's promotion FMAs and LDS reads fill the other's MFMA shadow) where
//    rows come in large blocks, including contiguous experts (m-blocks
//    enumerated expert by expert); 128x256 with 8 waves of 64x64 and three
//    LDS stages where M is small, or for more than 1024 contiguous experts.
//  * Grouped layouts whose last round of tiles would run at most half full
//    (contiguous) cut those tiles into K pieces: fp32 partials in a
//    per-device workspace, summed in order by reduce_split_kernel.
//  * Operand tiles are copied global -> LDS directly (global_load_lds, no
//    staging registers) into STAGES buffers, the copies of the next K blocks
//    in flight while the current one is multiplied. The copy and the reads
//    of one K step go through restrict-qualified stage pointers so that the
//    compiler knows they do not overlap and does not wait for the copies
//    before reading; each wave instead waits for its own copies of the stage
//    it is about to read, right before the barrier that publishes them.
//    LDS rows are 128 bytes (one K block of one row); the 16-byte chunk
//    index is XOR-swizzled (see swz) so that the MFMA fragment reads of 8 or
//    16 consecutive lanes spread over all LDS banks.
//  * Persistent grid of one workgroup per CU. Tile indices are remapped so
//    that each XCD (workgroups are dealt round-robin to the 8 XCDs) walks a
//    contiguous run of tiles, grouped GROUP_M m-blocks at a time (the tile
//    swizzle of the gtnt Triton kernel), so that the tiles an XCD runs
//    together share A rows and B columns in its L2.
//  * Grouped layouts decode the tile index on the device from the group
//    metadata (offsets or valid counts), so the host never synchronises
//    (nxmr §3.2: each expert's work goes to its own workgroups, one launch).
//    Where m-blocks are enumerated per expert, MFMA row tiles past the
//    expert's rows skip the arithmetic (16 rows at a time); rows past them
//    are never stored.

#include <atomic>
#include <mutex>
#include <stdio.h>
#include <type_traits>
#include <vector>

#include "e4m3.h"
#include "gemm_index.h"
#include "internal.h"

namespace fp8g {
namespace {

using namespace gidx;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Build-time timeline trace (-DFP8G_TRACE, off in the library): lane 0 of
// each wave of workgroups 0..3 stamps the shader clock at fixed points of
// the first 32 K steps into spare LDS, copied to fp8g_trace at the end.
#ifdef FP8G_TRACE
constexpr int TR_STEPS = 32, TR_PTS = 6, TR_WG = 4;
__device__ unsigned long long fp8g_trace[TR_WG][8][TR_STEPS][TR_PTS];
#define FP8G_TR(step_, pt_)                                                                   \
  do {                                                                                        \
    if (tr_on && (step_) < TR_STEPS && (threadIdx.x & 63) == 0)                               \
      trace_lds[(threadIdx.x >> 6) * TR_STEPS * TR_PTS + (step_) * TR_PTS + (pt_)] =          \
          __builtin_amdgcn_s_memtime();                                                       \
  } while (0)
#else
#define FP8G_TR(step_, pt_) do {} while (0)
#endif

// Two floats -> packed bf16 bits (a in the low half), round to nearest even,
// NaN -> 0x7FC0: gfx950's v_cvt_pk_bf16_f32 after mapping NaN inputs to
// +qNaN. One instruction for two values, where rounding the bit pattern in
// integer arithmetic ((u + 0x7FFF + lsb) >> 16, NaN tested first) takes
// about seven per value; the two agree on all 2^32 fp32 patterns (compared
// exhaustively on the GPU, in the kernels' default float mode, subnormals
// included).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const float qnan = __uint_as_float(0x7FC00000u);
  const f32x2_t v = {a != a ? qnan : a, b != b ? qnan : b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// s_waitcnt immediate that waits for vmcnt <= n only (expcnt, lgkmcnt free).
constexpr int vmcnt_only(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }

// Direct global -> LDS copies (global_load_lds_dword[x4]): each lane's 4 or 16
// bytes at base + voff land in LDS at M0 + lane * size (M0 = wave-uniform LDS
// byte address). Issued through inline assembly so that the compiler does
// not track them: it would otherwise wait for every copy in flight before
// the next LDS read of any stage. The waits these copies need are explicit
// (wait_stage before the barrier that publishes a stage); the memory clobber
// keeps LDS accesses from moving across the copy. s_nop 0 covers the
// M0-write -> LDS-DMA hazard.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)p);
}
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds)
               : "memory");
}
// The same with the non-temporal cache policy (the lines are streamed, not
// kept): for weights that one tile reads once.
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "{m0}"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds)
               : "memory");
}

// Global -> LDS copy of one K block of the A and B tiles and of the A row
// and B column-block scales. One 16-byte copy moves 8 rows x 128 bytes:
// lane l takes row base + (l >> 3) and, because its destination chunk is
// fixed to (l & 7), reads the logical chunk (l & 7) ^ (l >> 3) ^ parity so
// that the LDS image is the swizzled layout (swz). Copy wave cw issues the
// copies for the 8-row groups cw, cw + COPY_WAVES, ...; the first A_COPIES
// of them are A rows. Everything but the K offset is fixed for a tile, so it
// is computed once per tile (CopyPlan). Copy i of a wave moves rows
// row0 + i * 8 * COPY_WAVES of its operand (row0 = cw * 8 + (l >> 3)), so
// on a full tile one per-lane offset serves every copy and the rest of the
// offset is wave-uniform. On a ragged tile (rows past mvalid or columns past
// nvalid) each copy's row is clamped to the last row that exists (read in
// bounds, never stored). A K step then only advances the base pointers and
// issues the copies. Every copy wave issues the same number of copies
// whatever the tile, which the counted waits rely on.
template <class C>
__device__ __forceinline__ void make_plan(CopyPlan<C>& pl, const TileInfo& ti, int64_t K) {
  make_plan_at<C>(pl, ti, K, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), threadIdx.x & 63);
}

// Copies [c0, c1) of this wave's share of one stage, and with `scales` the
// scale copies too, so that a stage's copies can be spread between MFMAs.
// vsub: subtracted from every lane offset; for the partial last K block of a
// K that is not a multiple of 128, a lane whose 16-byte chunk lies past K
// passes its chunk offset here and so reads chunk 0 of the same row (in
// bounds; the consumer zeroes those bytes of its fragments).
// The A and B copies of one stage part; NT: the B copies with the
// non-temporal policy (dma16_nt).
template <class C, bool NT>
__device__ __forceinline__ void issue_tile_copies(const CopyPlan<C>& pl, const TileInfo& ti,
                                                  int64_t K, int kb, uint32_t stage_lds, int c0,
                                                  int c1, uint32_t vsub) {
  const int lane = threadIdx.x & 63;
  if (!pl.ragged) {
#pragma unroll
    for (int i = c0; i < c1; ++i) {
      const uint8_t* base;
      uint32_t voff;
      copy_source_full<C>(pl, ti, K, kb, i, vsub, base, voff);
      const uint32_t dst = stage_lds + pl.dst0 + (uint32_t)(i * C::COPY_WAVES * 8 * BK);
      if (NT && i >= C::A_COPIES) dma16_nt(base, voff, dst);
      else dma16(base, voff, dst);
    }
  } else {
#pragma unroll
    for (int i = c0; i < c1; ++i) {
      const uint8_t* base;
      uint32_t voff;
      copy_source_ragged<C>(pl, ti, K, kb, i, lane, vsub, base, voff);
      const uint32_t dst = stage_lds + pl.dst0 + (uint32_t)(i * C::COPY_WAVES * 8 * BK);
      if (NT && i >= C::A_COPIES) dma16_nt(base, voff, dst);
      else dma16(base, voff, dst);
    }
  }
}
// STREAM: 0 the B copies are cached; 1 every tile streams them (the masked
// layout); 2 a tile streams them when no other tile reads its B rows
// (ti.b_once; one wave-uniform branch per call, none between the copies)
template <class C, int STREAM = 0>
__device__ __forceinline__ void issue_copies(const CopyPlan<C>& pl, const TileInfo& ti,
                                             int64_t sa_ld, int64_t K, int kb, uint32_t stage_lds,
                                             int c0, int c1, bool scales, uint32_t vsub = 0) {
  if (pl.cw < 0) return;
  const int lane = threadIdx.x & 63;
  if (STREAM == 1 || (STREAM == 2 && ti.b_once))
    issue_tile_copies<C, STREAM != 0>(pl, ti, K, kb, stage_lds, c0, c1, vsub);
  else
    issue_tile_copies<C, false>(pl, ti, K, kb, stage_lds, c0, c1, vsub);
  if (scales) {
    if (pl.cw < C::SA_WAVES)
      dma4(ti.sa + (int64_t)kb * sa_ld, pl.sa_voff, stage_lds + C::SA_OFFSET + pl.cw * 256);
    // lane n < NB128 copies the scale of the tile's n-th 128-column block
    if (pl.cw == C::SB_WAVE && lane < C::NB128)
      dma4(ti.sb + kb, pl.sb_voff, stage_lds + C::SB_OFFSET);
  }
}

template <class C, int STREAM = 0>
__device__ __forceinline__ void issue_stage(const CopyPlan<C>& pl, const TileInfo& ti,
                                            int64_t sa_ld, int64_t K, int kb, uint32_t stage_lds,
                                            bool scales, uint32_t vsub = 0) {
  issue_copies<C, STREAM>(pl, ti, sa_ld, K, kb, stage_lds, 0, C::COPIES_PER_WAVE, scales, vsub);
}

// Wait until this wave's copies of the stage about to be read have landed,
// allowing the copies of `newer` later-issued stages to stay in flight.
// A copy wave issues COPIES_PER_WAVE copies per stage, plus one if it copies
// row scales and one if it copies the B scales; a wave that copies nothing
// has nothing to wait for.
template <class C, int PER>
__device__ __forceinline__ void wait_newer(int newer) {
  if (newer <= 0) __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  else if (newer == 1) __builtin_amdgcn_s_waitcnt(vmcnt_only(PER));
  else __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * PER));
}
template <class C, bool SCALES = true>
__device__ __forceinline__ void wait_stage(int newer) {
  const int cw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) - C::FIRST_COPY_WAVE;
  if (cw < 0) return;
  const bool sa = SCALES && cw < C::SA_WAVES, sb = SCALES && cw == C::SB_WAVE;
  if (sa && sb) wait_newer<C, C::COPIES_PER_WAVE + 2>(newer);
  else if (sa || sb) wait_newer<C, C::COPIES_PER_WAVE + 1>(newer);
  else wait_newer<C, C::COPIES_PER_WAVE>(newer);
}

// Workgroup barrier without the memory fences of __syncthreads(), which
// would drain every copy in flight. Visibility is handled explicitly: each
// wave waits for its own copies of the stage to be read (wait_stage) before
// arriving, and every LDS read of a stage has completed (its value fed an
// MFMA) before the wave arrives at the barrier after which that stage is
// refilled. The memory clobber keeps the compiler from moving LDS accesses
// across it; the scheduling barrier keeps other instructions in place.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// MFMA operand fragment: lane l holds row (l & 15) of the 16-row slice
// starting at `row0`, bytes [(l >> 4) * 32, +32) of the K block. A and B use
// the same lane -> K assignment, so the product sums over the full block
// whatever order the hardware takes the K elements in.
__device__ __forceinline__ v8i load_frag(const uint8_t* __restrict__ tile, int row0, int lane) {
  const int r = row0 + (lane & 15);
  const int c0 = (lane >> 4) * 2;
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + r * BK + swz(r, c0) * 16);
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + r * BK + swz(r, c0 + 1) * 16);
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// Zeroes the chunks past K of one stage's A and B rows (the partial last K
// block; its copies put each row's chunk 0 there), so that the block's
// products past K are 0 x 0. Every thread of the workgroup takes a share;
// the caller waits for the writes and synchronises before the stage is read.
template <class C>
__device__ __forceinline__ void zero_past_k(uint8_t* __restrict__ stage, int kr) {
  const int n = past_k_items<C>(kr);
  for (int i = (int)threadIdx.x; i < n; i += C::THREADS)
    *reinterpret_cast<uint4*>(stage + past_k_offset<C>(i, kr)) = make_uint4(0u, 0u, 0u, 0u);
}

// Materialises a value at this point of the program: the optimiser may not
// sink the arithmetic that produces it past later synchronisation (which
// would keep every slice's MFMA results alive until then).
__device__ __forceinline__ void pin(v4f& v) { asm volatile("" : "+v"(v)); }

// Fragment and scale reads of one K step from its LDS stage.
template <class C>
__device__ __forceinline__ void read_frags(const uint8_t* __restrict__ st, int wm, int wn,
                                           int lane, v8i (&af)[C::TM], v8i& b0) {
#pragma unroll
  for (int i = 0; i < C::TM; ++i) af[i] = load_frag(st, (wm + i * C::WAVES_M) * 16, lane);
  b0 = load_frag(st + C::BM * BK, wn * C::WN, lane);
}
// A row scale of each of this lane's rows (row rlane + i * RSTEP) and the B
// block scale of the wave's columns.
template <class C>
__device__ __forceinline__ void read_scales(const uint8_t* __restrict__ st, int wn, int rlane,
                                            float (&sa1)[C::TM], float& sbv) {
  const float* sas = reinterpret_cast<const float*>(st + C::SA_OFFSET);
#pragma unroll
  for (int i = 0; i < C::TM; ++i) sa1[i] = sas[rlane + i * C::RSTEP];
  sbv = reinterpret_cast<const float*>(st + C::SB_OFFSET)[(wn * C::WN) / 128];
}

// bf16 store of a wave's accumulators in whole 128-byte lines. The MFMA
// layout gives lane l four adjacent columns 4g .. 4g + 3 (g = l >> 4) of row
// r = l & 15 in every 16x16 tile, so a direct store writes 32-byte pieces of
// 16 rows. Two register exchanges regroup each 64-column block (four tiles):
//  * lanes l and l ^ 16 hold the two halves of columns 8 (g >> 1) .. +7 of
//    a tile; for each pair of adjacent tiles they swap one half, after
//    which the even lane holds those 8 columns of the first tile and the
//    odd lane those of the second: 16 bytes, piece (g >> 1) + 2 (g & 1) of
//    the pair's 64 bytes of row r;
//  * lanes l and l ^ 8 (rows r and r ^ 8) then swap one of their two tile
//    pairs' pieces: the lanes of rows 0-7 keep their first pair's piece and
//    take their partner's (row r + 8) first-pair piece, the lanes of rows
//    8-15 keep their second pair's piece and take their partner's (row
//    r - 8) second-pair piece.
// Each of the two stores per block then covers 8 whole rows x 128 bytes.
// The stores are non-temporal (the kernel never reads its output): the
// masked layout, bound by its weight stream, spent 17% of its time writing
// its 62 MB of output 8 bytes per lane; whole lines, non-temporal, recover
// most of that. Rows past mvalid and columns past nvalid are not written.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Value of lane l ^ 16 (ds_swizzle in bitmask mode within each 32 lanes:
// and-mask 31, or-mask 0, xor-mask 16) and of lane l ^ 8 (DPP row rotate by
// 8 within each row of 16 lanes); neither needs an address register.
__device__ __forceinline__ int swap_lane16(int x) {
  return __builtin_amdgcn_ds_swizzle(x, (16 << 10) | 31);
}
__device__ __forceinline__ int swap_lane8(int x) {
  return __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);
}
// One MFMA row tile i (rows trow .. trow + 15 of the workgroup tile) of the
// wave's columns; every lane of the wave takes part (lane exchanges).
template <class C>
__device__ __forceinline__ void store_rows_lines(const v4f (&acc)[C::TN], const TileInfo& ti,
                                                 int64_t N, int trow, int wn, int lane) {
  static_assert(C::TN % 4 == 0, "64-column blocks of four tiles");
  const int g = lane >> 4, r = lane & 15;
  const bool odd = (g & 1) != 0, hi = r >= 8;
  // the 16-byte piece this lane stores within a 128-byte row segment: the
  // first tile pair's (pieces 0-3) for rows 0-7 lanes, the second's (4-7)
  // for rows 8-15 lanes
  const int piece = (hi ? 4 : 0) + (g >> 1) + (odd ? 2 : 0);
  // Store address: a wave-uniform base (row 8 k of the tile, the 64-column
  // block) plus one per-lane 32-bit element offset that is the same for
  // every store, (r mod 8) N + 8 piece (N <= 2^27, so 7 N + 56 < 2^32).
  // 64-bit per-row addresses held across the stores would not fit the
  // register budget and be spilled.
  const uint32_t loff = (uint32_t)(r & 7) * (uint32_t)N + (uint32_t)(piece * 8);
#pragma unroll
  for (int h = 0; h < C::TN / 4; ++h) {
    const int c64 = wn * C::WN + h * 64;
    if (c64 >= ti.nvalid) continue;                     // (wave-uniform)
    u32x4 pc[2];        // row r's 16 bytes of tile pair 0 and tile pair 1
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int j = h * 4 + pr * 2;
      uint2 a, b;
      a.x = bf16x2_rne(acc[j][0], acc[j][1]);
      a.y = bf16x2_rne(acc[j][2], acc[j][3]);
      b.x = bf16x2_rne(acc[j + 1][0], acc[j + 1][1]);
      b.y = bf16x2_rne(acc[j + 1][2], acc[j + 1][3]);
      const uint2 keep = odd ? b : a, send = odd ? a : b;
      const uint32_t rx = (uint32_t)swap_lane16((int)send.x);
      const uint32_t ry = (uint32_t)swap_lane16((int)send.y);
      // even lane: own columns first, partner's after; odd lane reversed
      pc[pr] = odd ? u32x4{rx, ry, keep.x, keep.y} : u32x4{keep.x, keep.y, rx, ry};
    }
    // rows r and r ^ 8: the lower lane sends its second pair's piece, the
    // upper one its first pair's
    const u32x4 snd = hi ? pc[0] : pc[1];
    u32x4 rcv;
#pragma unroll
    for (int k = 0; k < 4; ++k) rcv[k] = (uint32_t)swap_lane8((int)snd[k]);
    // store 0: rows 0-7 of the tile (lower lanes their own first-pair
    // piece, upper lanes the one received from row r - 8); store 1: rows
    // 8-15 (lower lanes the one received from row r + 8, upper lanes their
    // own second-pair piece)
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const u32x4 v = part == 0 ? (hi ? rcv : pc[0]) : (hi ? pc[1] : rcv);
      const int row = trow + part * 8 + (r & 7);
      const int col = c64 + piece * 8;
      uint16_t* const base = ti.d + (int64_t)(trow + part * 8) * N + c64;
      if (row < ti.mvalid && col < ti.nvalid)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(base + loff));
    }
    // (one block at a time: converting later blocks early would only hold
    // more registers)
    __builtin_amdgcn_sched_barrier(0);
  }
}
template <class C>
__device__ __forceinline__ void store_tile_lines(const v4f (&acc)[C::TM][C::TN], const TileInfo& ti,
                                                 int64_t N, int wm, int wn, int lane) {
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
    store_rows_lines<C>(acc[i], ti, N, (wm + i * C::WAVES_M) * 16, wn, lane);
}

// Fused quantising epilogue (the producer of the next layer's activations
// quantises them as it writes them): the bf16 result of each row's
// 128-column block (one wave's columns) is quantised 1x128 exactly as the
// quantiser does it for a bf16 input -- amax over the 128 bf16 values, one
// scale, the e4m3 element rule -- and stored as codes qd [rows][N] and
// scales sd [N/128][rows]; the bf16 values themselves are stored too when d
// is wanted. A row's 128 values sit in lanes l, l^16, l^32, l^48 (four
// columns per lane and MFMA tile), so the block amax is two lane shuffles.
template <class C>
__device__ __forceinline__ void store_tile_quant(v4f (&acc)[C::TM][C::TN], const TileInfo& ti,
                                                 const GemmArgs& args, int wm, int wn, int rlane,
                                                 int lane) {
  static_assert(C::WN == 128, "one 128-column scale block per wave and row");
  const int64_t N = args.N;
  const int64_t cb = (ti.col0 >> 7) + wn;                  // this wave's column block
  const int64_t col = ti.col0 + wn * C::WN + (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int r = rlane + i * C::RSTEP;
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      // each value replaced by its bf16 rounding, held exactly as fp32;
      // columns past N (a partial last block) are zeros, which leave the
      // block amax alone, and are not stored
      const bool jok = wn * C::WN + j * 16 < ti.nvalid;
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const uint32_t pk = bf16x2_rne(acc[i][j][e], acc[i][j][e + 1]);
        acc[i][j][e] = jok ? __uint_as_float(pk << 16) : 0.0f;
        acc[i][j][e + 1] = jok ? __uint_as_float(pk & 0xFFFF0000u) : 0.0f;
      }
      m = e4m3::amax4(make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]), m);
    }
    m = __builtin_fmaxf(m, __shfl_xor(m, 16));
    m = __builtin_fmaxf(m, __shfl_xor(m, 32));
    const e4m3::Divisor dv = e4m3::make_divisor(e4m3::scale_of(m));
    if (r < ti.mvalid) {
      const int64_t row = ti.row0 + r;
      uint8_t* qrow = args.qd + row * N + col;
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        if (wn * C::WN + j * 16 < ti.nvalid)
          *reinterpret_cast<uint32_t*>(qrow + j * 16) = e4m3::encode4(
              make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]), dv);
      if ((lane >> 4) == 0) args.sd[cb * args.rows + row] = dv.s;
    }
    // the bf16 values themselves, when wanted: acc[i] now holds each one
    // exactly (bf16 rounding of them changes nothing), stored as whole lines
    // like the plain epilogue's, row tile by row tile so that each tile's
    // registers are free once it is stored
    if (args.d) store_rows_lines<C>(acc[i], ti, N, (wm + i * C::WAVES_M) * 16, wn, lane);
  }
}

// fp32 store of a wave's accumulators into a K piece's partial tile
// (row-major BM x BN floats), same lane layout as store_tile; MFMA row
// tiles past ntiles (no row of the tile) are not stored.
template <class C>
__device__ __forceinline__ void store_partial(const v4f (&acc)[C::TM][C::TN], float* part, int wn,
                                              int rlane, int lane, int ntiles) {
  float* base = part + (int64_t)rlane * C::BN + wn * C::WN + (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
    if (i < ntiles) {
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        *reinterpret_cast<float4*>(base + (int64_t)(i * C::RSTEP) * C::BN + j * 16) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
}

// Persistent block-scaled GEMM. Workgroup w owns the tile slots
// first, first + grid, ...; their K steps form one continuous sequence
// (tile-major) that a single copy ring serves: the copies of step s + STAGES
// are issued as soon as every wave has finished reading step s, whether or
// not s + STAGES belongs to the same tile, so the next tile's first operands
// arrive while the current tile's last K blocks are multiplied.
//
// A K step on one wave (TM x TN MFMA tiles, 16-column slices j):
//   for j: read B fragment j+1 | MFMAs of slice j | promote slice j-1
//   wait for own copies of step s+1, barrier, issue the copies of step
//   s+STAGES, read the A fragments and first B fragment of step s+1,
//   promote slice TN-1, read the scales of step s+1.
// The fragment reads of the next step are thus in flight while the last
// slice's MFMAs and promotions run, and the barrier sits where the LDS has
// nothing left to give the current step.
//
// K pieces (contiguous layout, planned by the host with choose_splits): a
// piece's fp32 sum over its K blocks goes to args.ws instead of D, the
// first piece of each tile records where the tile's output goes, and
// reduce_split_kernel adds the pieces and stores bf16.
//
// QUANT (dense layout only) swaps the bf16 epilogue for the quantising one
// (store_tile_quant). It is a separate instantiation because the quantising
// epilogue's extra registers would otherwise raise the plain kernel's
// allocation past 256 VGPRs and spill inside its main loop.
//
// NS, KS > 0: an instantiation for one hot shape (N = NS, K = KS known at
// compile time), the ahead-of-time counterpart of compiling a kernel per
// shape; the arithmetic is the generic kernel's, so the choice never
// changes bits (the scalar address and tile arithmetic folds into
// constants, which frees the scalar registers the generic kernel spills).
//
// FMTS (per-tensor layout only): the operands' 8-bit formats, A's in bits
// 0-3 and B's in bits 4-7, 0 = e4m3, 1 = e5m2 -- the MFMA's own operand
// format codes (it takes both formats, and mixed pairs, at the same rate).
//
// KTAIL: K is not a multiple of 128. The last K block is partial: its
// copies read the chunks past K from chunk 0 of the same row instead (in
// bounds), and once its stage has landed, the workgroup zeroes those chunks
// in LDS, in both operands (a stray NaN code would otherwise poison the
// products), and synchronises once more before reading it. The main loop
// is then the aligned kernel's; a separate instantiation all the same, so
// that the aligned kernels carry none of it.
template <class C, int MODE, bool QUANT = false, int NS = 0, int KS = 0, int FMTS = 0,
          bool KTAIL = false>
__global__ void __launch_bounds__(C::THREADS, 1)
gemm_fp8_bs_kernel(GemmArgs args, int xcd_remap) {
  static_assert(!QUANT || (MODE == MODE_DENSE && C::WN == 128),
                "the quantising epilogue needs one 128-column block per wave");
  static_assert(FMTS == 0 || MODE == MODE_PERTENSOR, "operand formats: per-tensor layout only");
  // (B is the MFMA's first operand)
  constexpr int kFmtFirst = (FMTS >> 4) & 15, kFmtSecond = FMTS & 15;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
  // (per-expert metadata; a placeholder word in the other layouts)
  __shared__ int meta_lds[per_expert<C, MODE>() ? sizeof(MaskedMeta) / sizeof(int) : 1];
#ifdef FP8G_TRACE
  constexpr bool tr_on = MODE == MODE_DENSE || MODE == MODE_PERTENSOR;
  __shared__ unsigned long long trace_lds[tr_on ? 8 * TR_STEPS * TR_PTS : 1];
#endif
  MaskedMeta* const meta = reinterpret_cast<MaskedMeta*>(meta_lds);

  const int64_t N = NS > 0 ? (int64_t)NS : args.N;
  const int64_t K = KS > 0 ? (int64_t)KS : args.K;
  // per-tensor scales: the MFMA accumulates over all of K, no promotion
  constexpr bool PT = MODE == MODE_PERTENSOR;
  // Weight panels that one tile alone reads are streamed with the
  // non-temporal policy, which leaves the L2 to the A rows an expert's
  // column blocks share: the masked layout streams every tile's (an
  // expert's m-blocks are at most max_m rows; G32 maxm256 N7168 K2048:
  // 129-131 -> 123-129 us on three boxes), the contiguous layout those of
  // experts with a single m-block, the split tail's pieces among them
  // (G8 T4096 N4096 K7168: 160 -> 158 us; deciding per tile in the masked
  // layout too measured 2% slower there). Panels several tiles read stay
  // cached: with the policy on the dense weights, 221 -> 238 us.
  constexpr int kStream = MODE == MODE_MASKED ? 1 : (MODE == MODE_CONTIGUOUS ? 2 : 0);
  Sched sc;
  sc.nblocks128 = (int)((N + 127) / 128);
  sc.nblocks = (int)((N + C::BN - 1) / C::BN);
  if constexpr (per_expert<C, MODE>()) {
    // clamped counts; masked: rank of each expert by decreasing count
    // (ties by index, so the ranks are a permutation), contiguous: expert
    // order; then wave 0 scans the m-block counts in rank order, 64 ranks
    // at a time
    const int G = args.G;
    for (int g = threadIdx.x; g < G; g += C::THREADS) {
      if constexpr (MODE == MODE_MASKED) {
        const int m = args.group[g];
        meta->cnt[g] = m < 0 ? 0 : (m > args.rows ? (int)args.rows : m);
      } else {
        int64_t lo = args.group[g], hi = args.group[g + 1];
        lo = lo < 0 ? 0 : (lo > args.rows ? args.rows : lo);
        hi = hi < 0 ? 0 : (hi > args.rows ? args.rows : hi);
        meta->cnt[g] = hi > lo ? (int)(hi - lo) : 0;
        meta->order[g] = g;
      }
    }
    __syncthreads();
    if constexpr (MODE == MODE_MASKED) {
      for (int t = threadIdx.x; t < G; t += C::THREADS) {
        const int key = meta->cnt[t];
        int r = 0;
        for (int g = 0; g < G; ++g) {
          const int kg = meta->cnt[g];
          r += (kg > key || (kg == key && g < t)) ? 1 : 0;
        }
        meta->order[r] = t;
      }
      __syncthreads();
    }
    if (threadIdx.x < 64) {
      const int l = threadIdx.x;
      int carry = 0;
      for (int r0 = 0; r0 < G; r0 += 64) {
        const int r = r0 + l;
        int v = r < G ? (meta->cnt[meta->order[r]] + C::BM - 1) / C::BM : 0;
        for (int o = 1; o < 64; o <<= 1) {
          const int x = __shfl_up(v, o);
          if (l >= o) v += x;
        }
        if (r < G) meta->prefix[r + 1] = carry + v;
        carry += __shfl(v, 63);
      }
      if (l == 0) meta->prefix[0] = 0;
    }
    __syncthreads();
    sc.mblocks = __builtin_amdgcn_readfirstlane(meta->prefix[G]);
  } else {
    sc.mblocks = (int)((args.rows + C::BM - 1) / C::BM);
  }
  sc.tiles = sc.mblocks * sc.nblocks;
  const int grid = gridDim.x;
  const int nkb = (int)((K + BK - 1) / BK);
  // the partial last K block's valid bytes
  const int kr = (int)(K % BK);
  SplitPlan spl{args.split_base, args.splits};
  if constexpr (MODE == MODE_CONTIGUOUS && per_expert<C, MODE>()) {
    // the tile count is known here only: plan the split tail on the device
    // (every workgroup alike)
    spl.splits = args.ws ? choose_splits(sc.tiles, grid, nkb) : 1;
    spl.base = spl.splits > 1 ? (sc.tiles / grid) * grid : 0;
  }
  // (every lane of wave 0 writes the same values: a wave-uniform branch)
  if (args.ws && blockIdx.x == 0 && __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0) {
    args.ws_meta->tail = spl.splits > 1 ? sc.tiles - spl.base : 0;
    args.ws_meta->splits = spl.splits;
  }
  // work slots of this launch
  const int nwork = spl.splits > 1 ? spl.base + (sc.tiles - spl.base) * spl.splits : sc.tiles;
  const int w = blockIdx.x;
  const int first = xcd_remap ? (w & 7) * (grid >> 3) + (w >> 3) : w;
  const int nslots = slot_count<MODE>(first, grid, nwork);
  if (nslots == 0) return;                               // uniform over the workgroup

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the younger wave of each SIMD (waves WAVES/2 ..) issues the copies; by
  // default the SIMD favours the older wave, which starves the copy issuer
  if (C::PRIO_YOUNG == 1 && wave >= C::WAVES / 2) __builtin_amdgcn_s_setprio(1);
  const int wm = wave / C::WAVES_N;
  const int wn = wave % C::WAVES_N;
  const int rlane = wm * 16 + (lane & 15);               // this lane's row in MFMA tile 0
  const int kpt = nkb / spl.splits;                      // K steps of a piece
  int total = 0;                                         // K steps of this workgroup
  for (int k = 0, w2 = first; k < nslots; ++k, w2 = next_slot<MODE>(w2, first, grid))
    total += work_steps(spl, w2, nkb, kpt);
  const uint32_t lds_base = lds_addr(lds);

  // copy cursor: the (tile, K block) whose copies are issued next
  int p_slot = first, p_kb = 0, issued = 0;
  int p_k0 = work_k0(spl, p_slot, kpt);                 // first K block of the slot
  int p_steps = work_steps(spl, p_slot, nkb, kpt);      // its K steps
  TileInfo tp;
  decode_tile<C, MODE>(args, meta, sc, work_tile(spl, p_slot), tp, N, K);
  CopyPlan<C> pl;
  make_plan<C>(pl, tp, K);
#pragma unroll
  for (int s = 0; s < C::STAGES; ++s) {
    if (issued < total) {
      issue_stage<C, kStream>(pl, tp, args.sa_ld, K, p_k0 + p_kb, lds_base + s * C::STAGE_BYTES, !PT,
                     (KTAIL && p_k0 + p_kb == nkb - 1 && (int)pl.ch16 >= kr) ? pl.ch16 : 0u);
      ++issued;
      if (++p_kb == p_steps) {
        p_kb = 0;
        p_slot = next_slot<MODE>(p_slot, first, grid);
        if (p_slot < nwork) {
          decode_tile<C, MODE>(args, meta, sc, work_tile(spl, p_slot), tp, N, K);
          p_k0 = work_k0(spl, p_slot, kpt);
          p_steps = work_steps(spl, p_slot, nkb, kpt);
          make_plan<C>(pl, tp, K);
        }
      }
    }
  }

  // compute cursor
  int c_slot = first, c_kb = 0;
  TileInfo tc;
  int c_steps = work_steps(spl, c_slot, nkb, kpt);
  decode_tile<C, MODE>(args, meta, sc, work_tile(spl, c_slot), tc, N, K);
  int nact = active_tiles<C>(tc, wm, wn);     // MFMA row tiles of this wave in use

  v4f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // per-tensor: the product of the two scales, formed once in fp32
  float ptc = 0.f;
  if constexpr (PT) ptc = args.sa[0] * args.sb[0];
  v8i af[C::TM];        // A fragments of the K step
  v8i bf[C::NBF];       // B fragments: slices j .. j + PF in flight (slice j in bf[j % NBF])
  float sa1[C::TM];     // A row scales of the K step (this lane's row per MFMA tile)
  float sbv = 0.f;      // B block scale of the K step
  float cs[C::TM];      // promotion factors sa * sb of the K step
  v4f p[C::TM];         // MFMA results of the current slice

  wait_stage<C, !PT>(min(C::STAGES - 1, issued - 1));
  wg_barrier();
  if constexpr (KTAIL) {
    if (work_k0(spl, first, kpt) == nkb - 1) {         // the first step reads the last block
      zero_past_k<C>(lds, kr);
      __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0)
      wg_barrier();
    }
  }
  read_frags<C>(lds, wm, wn, lane, af, bf[0]);
#pragma unroll
  for (int k = 1; k < C::PF; ++k) bf[k] = load_frag(lds + C::BM * BK, wn * C::WN + k * 16, lane);

  // Everything a wave does at the end of a K step before it may read the
  // next one: its copies of the next stage have landed (own wait), every
  // wave is done reading this stage (barrier), then this stage's buffer is
  // refilled with the stage STAGES steps ahead. (At the last step there is
  // nothing left to copy; the barrier is then harmless, as every wave of
  // the workgroup takes it.)
#define FP8G_SYNC(s_)                                                                         \
  do {                                                                                        \
    __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0): own LDS reads done */                  \
    wait_stage<C, !PT>(min(C::STAGES - 2, issued - ((s_) + 2)));                              \
    wg_barrier();                                                                             \
  } while (0)
  // part q (of SPREAD) of the next stage's copies, into the buffer the
  // barrier freed; the last part also copies the scales
#define FP8G_REFILL_PART(q_)                                                                  \
  do {                                                                                        \
    constexpr int CPS_ = C::COPIES_PER_SLICE;                                                 \
    const int c0_ = min((q_) * CPS_, C::COPIES_PER_WAVE);                                     \
    const int c1_ = (q_) == C::SPREAD - 1 ? C::COPIES_PER_WAVE                                \
                                          : min(((q_) + 1) * CPS_, C::COPIES_PER_WAVE);       \
    if (issued < total)                                                                       \
      issue_copies<C, kStream>(pl, tp, args.sa_ld, K, p_k0 + p_kb,                            \
                      lds_base + (issued % C::STAGES) * C::STAGE_BYTES, c0_, c1_,             \
                      !PT && (q_) == C::SPREAD - 1,                                           \
                      (KTAIL && p_k0 + p_kb == nkb - 1 && (int)pl.ch16 >= kr) ? pl.ch16 : 0u); \
  } while (0)
  // after the last part: advance the copy cursor
#define FP8G_REFILL_DONE()                                                                    \
  do {                                                                                        \
    if (issued < total) {                                                                     \
      ++issued;                                                                               \
      if (++p_kb == p_steps) {                                                                \
        p_kb = 0;                                                                             \
        p_slot = next_slot<MODE>(p_slot, first, grid);                                        \
        if (p_slot < nwork) {                                                                 \
          decode_tile<C, MODE>(args, meta, sc, work_tile(spl, p_slot), tp, N, K);                  \
          p_k0 = work_k0(spl, p_slot, kpt);                                                  \
          p_steps = work_steps(spl, p_slot, nkb, kpt);                                       \
          make_plan<C>(pl, tp, K);                                                            \
        }                                                                                     \
      }                                                                                       \
    }                                                                                         \
  } while (0)

  // MFMA row tiles that hold no row of the tile skip their arithmetic only
  // where m-blocks are enumerated per expert (masked: an expert's valid
  // rows often end early in its 256-row block; contiguous with 256-row
  // tiles: an expert's last block may hold 128 rows); elsewhere every wave
  // computes every tile (rows past the tile are clamped copies, never
  // stored), which keeps the loop free of per-tile branches.
  constexpr bool SKIP_IDLE = per_expert<C, MODE>();
  // The slice whose start holds the end-of-step barrier. Every LDS read of
  // a step's stage has been issued by the start of slice TN - PF (the B
  // fragments are read PF slices ahead), so the barrier, and the refill of
  // the stage it frees, can come that early. The masked layout, whose time
  // is the weight stream rather than the MFMAs, takes it there so that
  // each stage's copies have PF - 1 more slices to land (141 -> 137 us on
  // G32 maxm256 N7168 K2048); the others keep it in the last slice, which
  // measured 1.5-2% faster for them.
  constexpr int SYNC_J = MODE == MODE_MASKED ? C::TN - C::PF : C::TN - 1;
  static_assert(SYNC_J == C::TN - 1 || C::SPREAD <= C::TN - SYNC_J,
                "a stage's copies are issued within the step of its barrier");
  bool refill = false;   // a stage's copies are being issued, part by part
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    p[i] = v4f{0.f, 0.f, 0.f, 0.f};
    cs[i] = 0.f;
  }
  for (int s = 0; s < total; ++s) {
    const uint8_t* __restrict__ cur = lds + (s % C::STAGES) * C::STAGE_BYTES;
    const uint8_t* __restrict__ btile = cur + C::BM * BK;
    const uint8_t* __restrict__ nxt = lds + ((s + 1) % C::STAGES) * C::STAGE_BYTES;
    const bool last_of_tile = c_kb == c_steps - 1;
    // Slice j: prefetch B slice j+2, then per MFMA tile i promote tile i of
    // the previous slice (for j = 0: the previous step's last slice, with
    // that step's promotion factors; p and cs are zero at the start of a
    // tile, so that adds exactly nothing) and reuse its result registers for
    // slice j. Slice 0 also reads this step's scales; slice 1 forms the new
    // promotion factors before its first promotion. The last slice starts
    // with the end-of-step synchronisation, reads the next step's first B
    // fragment at once, and follows each MFMA with the read of the next
    // step's A fragment whose register it has just freed, so that the first
    // MFMAs of the next step find their operands arriving in the order they
    // need them.
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      // part q of the refill: the slice with the barrier issues part 0 right
      // after it, the following slices (of this step or the next) the rest
      const int q = j >= SYNC_J ? j - SYNC_J : (SYNC_J == C::TN - 1 ? j + 1 : C::SPREAD);
      if (j == 0) FP8G_TR(s, 0);
      if (j == SYNC_J) {
        FP8G_TR(s, 1);
#ifdef FP8G_TRACE
        __builtin_amdgcn_s_waitcnt(0xC07F);     // (split the own-read wait from the rest)
#endif
        FP8G_TR(s, 2);
        FP8G_SYNC(s);
        FP8G_TR(s, 3);
        refill = issued < total;
        if constexpr (KTAIL) {
          // the next step reads the partial last K block: its stage has
          // landed (the barrier above), zero it past K before anyone reads it
          const int next_kb = last_of_tile ? work_k0(spl, next_slot<MODE>(c_slot, first, grid), kpt)
                                           : work_k0(spl, c_slot, kpt) + c_kb + 1;
          if (s + 1 < total && next_kb == nkb - 1) {
            zero_past_k<C>(lds + ((s + 1) % C::STAGES) * C::STAGE_BYTES, kr);
            __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0)
            wg_barrier();
          }
        }
      }
      if (q < C::SPREAD && refill) {
        FP8G_REFILL_PART(q);
        if (q == 0) FP8G_TR(s, 4);
        if (q == C::SPREAD - 1) {
          FP8G_TR(s, 5);
          FP8G_REFILL_DONE();
          refill = false;
        }
      }
      if (j == C::TN - 1) {
        __builtin_amdgcn_sched_barrier(0);
        // the next step's first PF slices: read them now, except one whose
        // register this last slice is still using
#pragma unroll
        for (int k = 0; k < C::PF; ++k)
          if (k % C::NBF != (C::TN - 1) % C::NBF)
            bf[k % C::NBF] = load_frag(nxt + C::BM * BK, wn * C::WN + k * 16, lane);
      }
      if (j + C::PF < C::TN)
        bf[(j + C::PF) % C::NBF] = load_frag(btile, wn * C::WN + (j + C::PF) * 16, lane);
      if (!PT && j == 0) read_scales<C>(cur, wn, rlane, sa1, sbv);
      if (!PT && j == 1) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i) cs[i] = sa1[i] * sbv;
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        if constexpr (PT) {
          // one K block's products added into the running fp32 sum
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bf[j % C::NBF], af[i], acc[i][j], kFmtFirst, kFmtSecond, 0, 0, 0, 0);
        } else if (!SKIP_IDLE || i < nact) {       // (wave-uniform)
          const int jp = j > 0 ? j - 1 : C::TN - 1;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][jp][e] = __builtin_fmaf(p[i][e], cs[i], acc[i][jp][e]);
          pin(acc[i][jp]);
          // B as the first operand: the result is the transposed 16x16
          // tile, so lane l holds row (l & 15), columns 4 (l >> 4) .. +3
          p[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bf[j % C::NBF], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        }
        if (j == C::TN - 1) {
          // next step's A fragment i, after the last use of its register
          // (the last step reads a stale stage: in bounds and unused)
          __builtin_amdgcn_sched_barrier(0);
          af[i] = load_frag(nxt, (wm + i * C::WAVES_M) * 16, lane);
        }
      }
      if (j == C::TN - 1) {
#pragma unroll
        for (int k = 0; k < C::PF; ++k)
          if (k % C::NBF == (C::TN - 1) % C::NBF)
            bf[k % C::NBF] = load_frag(nxt + C::BM * BK, wn * C::WN + k * 16, lane);
      }
      // Issue order of a full slice: one B fragment read, then per MFMA tile
      // its four promotion FMAs followed by its MFMA (the second fragment
      // read after the first tile). Left to itself the scheduler bunches
      // the FMAs of three tiles and then issues their MFMAs back to back, so
      // a wave's FMAs no longer sit in the shadow of its own MFMAs (3.7%
      // slower on the dense 4096x8192x8192 shape).
      if (!PT && j < SYNC_J) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // DS read
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);        // VALU
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
          if (i == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      // keep each slice's instructions together: the scheduler may
      // interleave them but not pull later loads forward (register
      // pressure) or move promotions across the reuse of their registers
      __builtin_amdgcn_sched_barrier(0);
    }
    if (last_of_tile) {
      const bool has_next = s + 1 < total;
      TileInfo tn = tc;
      const int nxt_slot = next_slot<MODE>(c_slot, first, grid);
      if (has_next) decode_tile<C, MODE>(args, meta, sc, work_tile(spl, nxt_slot), tn, N, K);
      if constexpr (PT) {
        // epilogue: the fp32 sum times scale_a * scale_b, rounded once to bf16
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] *= ptc;
        if (nact > 0) store_tile_lines<C>(acc, tc, N, wm, wn, lane);
      } else if (!SKIP_IDLE || nact > 0) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][C::TN - 1][e] = __builtin_fmaf(p[i][e], cs[i], acc[i][C::TN - 1][e]);
        if (nact > 0) {
          if (is_piece(spl, c_slot)) {        // (workgroup-uniform)
            const int piece = c_slot - spl.base;
            store_partial<C>(acc, args.ws + (int64_t)piece * (C::BM * C::BN), wn, rlane, lane,
                             SKIP_IDLE ? nact : C::TM);
            if (piece % spl.splits == 0 && wave == 0) {     // (all its lanes write the same)
              SplitTile* rec = reinterpret_cast<SplitTile*>(args.ws_meta + 1) + piece / spl.splits;
              rec->d_off = tc.d - args.d;
              rec->mvalid = tc.mvalid;
              rec->nvalid = tc.nvalid;
            }
          } else if constexpr (QUANT) {
            store_tile_quant<C>(acc, tc, args, wm, wn, rlane, lane);
          } else {
            store_tile_lines<C>(acc, tc, N, wm, wn, lane);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        p[i] = v4f{0.f, 0.f, 0.f, 0.f};
        cs[i] = 0.f;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      }
      tc = tn;
      nact = active_tiles<C>(tc, wm, wn);
      c_slot = nxt_slot;
      c_steps = work_steps(spl, c_slot, nkb, kpt);
      c_kb = 0;
    } else {
      ++c_kb;
    }
  }
#ifdef FP8G_TRACE
  __syncthreads();
  if (tr_on && blockIdx.x < TR_WG)
    for (int i = threadIdx.x; i < 8 * TR_STEPS * TR_PTS; i += C::THREADS)
      (&fp8g_trace[blockIdx.x][0][0][0])[i] = trace_lds[i];
#endif
}

// Sum of the K pieces of the split tail tiles recorded in meta, in piece
// order, rounded once to bf16; only the rows and columns that exist are
// stored. Work item b covers rows 8 (b % (BM / 8)) .. +7 of tail tile
// b / (BM / 8) (grid-stride over the items); each thread issues the loads
// of all pieces of its four columns before adding.
constexpr int RED_ROWS = 8;
template <class C>
__global__ void __launch_bounds__(256)
reduce_split_kernel(uint16_t* __restrict__ d, int64_t N, const float* __restrict__ ws,
                    const SplitMeta* __restrict__ meta) {
  static_assert(RED_ROWS * C::BN / 4 == 2 * 256, "two float4 columns per thread");
  constexpr int PARTS = C::BM / RED_ROWS;
  const int tail = meta->tail;
  const int splits = meta->splits;
  const SplitTile* recs = reinterpret_cast<const SplitTile*>(meta + 1);
  for (int item = (int)blockIdx.x; item < tail * PARTS; item += (int)gridDim.x) {
    const int t = item / PARTS;
    const int r0 = (item % PARTS) * RED_ROWS;
    const SplitTile rec = recs[t];
    if (r0 >= rec.mvalid) continue;                      // (workgroup-uniform)
    const float* part = ws + (int64_t)t * splits * (C::BM * C::BN);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = (int)threadIdx.x + h * 256;
      const int r = r0 + e / (C::BN / 4);
      const int c = (e % (C::BN / 4)) * 4;
      if (r >= rec.mvalid || c >= rec.nvalid) continue;
      float4 x[MAX_SPLITS];
#pragma unroll
      for (int q = 0; q < MAX_SPLITS; ++q)
        if (q < splits)
          x[q] = *reinterpret_cast<const float4*>(part + (int64_t)q * (C::BM * C::BN) +
                                                  r * C::BN + c);
      float4 sum = x[0];
#pragma unroll
      for (int q = 1; q < MAX_SPLITS; ++q)
        if (q < splits) {
          sum.x += x[q].x; sum.y += x[q].y; sum.z += x[q].z; sum.w += x[q].w;
        }
      uint2 v;
      v.x = bf16x2_rne(sum.x, sum.y);
      v.y = bf16x2_rne(sum.z, sum.w);
      *reinterpret_cast<uint2*>(d + rec.d_off + (int64_t)r * N + c) = v;
    }
  }
}

// Workspace of a split tail: the SplitMeta header and one SplitTile record
// per workgroup of the launch, then fp32 partial tiles for at most one round
// of pieces (grid tiles of BM x BN floats). Every byte the reduction reads is
// written by the GEMM kernel of the same call, so the workspace needs no
// clearing between calls.
template <class C>
size_t split_head_bytes(int64_t grid) {
  return ((sizeof(SplitMeta) + (size_t)grid * sizeof(SplitTile)) + 255) / 256 * 256;
}
template <class C>
size_t split_bytes(int64_t grid) {
  return split_head_bytes<C>(grid) + (size_t)grid * C::BM * C::BN * sizeof(float);
}

// Workspace a contiguous call can use for a split tail (0: it never splits).
template <class C>
size_t contiguous_ws_bytes(const GemmArgs& args, const DeviceInfo& dev) {
  int64_t tiles_max;
  const int64_t grid = launch_grid<C>(args, dev, &tiles_max);
  if (tiles_max <= 0) return 0;
  const bool expert_blocks = C::BM > 128;
  if (expert_blocks) return tiles_max > grid ? split_bytes<C>(grid) : 0;
  return choose_splits(tiles_max, grid, (args.K + BK - 1) / BK) > 1 ? split_bytes<C>(grid) : 0;
}

// ---------------------------------------------------------------------------
// Kernel table. The pages' library compiles a kernel for each GEMM shape at
// run time and keeps it in a cache, so that a shape pays for compilation
// once (nxmr §2.3). Here every kernel is compiled ahead of time: a generic
// instantiation per layout and tile configuration, plus instantiations with
// N and K fixed at compile time for the hot shapes below; a call takes the
// specialised kernel when its shape matches an entry. The entries are the
// shapes the pages measure: the 4096x8192x8192 GEMM of the gtnt page's
// table (block and per-tensor scaling), MoE experts of 4096x7168 for the
// contiguous (prefill) layout and 7168x2048 for the masked (decode) layout,
// and the decode-shaped small-M product with K = 7168. (The quantising
// epilogue has no entry: its specialised kernel spilled more registers and
// measured slower than the generic one.)
struct HotShape {
  int mode;       // GemmMode
  bool quant;     // dense: the quantising epilogue
  bool small_m;   // the small-M kernel (N is not fixed there)
  int n, k;
};
constexpr int kSmallMHotK = 7168;
constexpr HotShape kHotShapes[] = {
    {MODE_DENSE, false, false, 8192, 8192},
    {MODE_PERTENSOR, false, false, 8192, 8192},
    {MODE_CONTIGUOUS, false, false, 4096, 7168},
    {MODE_MASKED, false, false, 7168, 2048},
    {MODE_DENSE, false, true, 0, kSmallMHotK},
};
constexpr int kNumHot = sizeof(kHotShapes) / sizeof(kHotShapes[0]);
std::atomic<int> g_specialise{1};

// Index of the table entry a persistent launch with configuration C uses
// (specialised kernels exist for the 256x256 configuration only), -1 for the
// generic kernel.
template <class C>
int hot_index(const GemmArgs& a) {
  if (!std::is_same<C, CfgLarge>::value || !g_specialise.load(std::memory_order_relaxed))
    return -1;
  for (int i = 0; i < kNumHot; ++i) {
    const HotShape& h = kHotShapes[i];
    if (!h.small_m && h.mode == a.mode && h.quant == (a.qd != nullptr) && a.fmts == 0 &&
        h.n == a.N && h.k == a.K)
      return i;
  }
  return -1;
}

// (a K that is not a multiple of 128 takes the KTAIL instantiation; the
// table's shapes all have K % 128 == 0)
template <class C, int MODE, bool QUANT, int FMTS = 0, int I = 0>
void launch_persistent(const GemmArgs& a, int hot, int64_t grid, int remap, hipStream_t stream) {
  if (a.K % BK != 0) {
    hipLaunchKernelGGL((gemm_fp8_bs_kernel<C, MODE, QUANT, 0, 0, FMTS, true>),
                       dim3((unsigned)grid), dim3(C::THREADS), 0, stream, a, remap);
    return;
  }
  if constexpr (FMTS != 0) {
    hipLaunchKernelGGL((gemm_fp8_bs_kernel<C, MODE, QUANT, 0, 0, FMTS>), dim3((unsigned)grid),
                       dim3(C::THREADS), 0, stream, a, remap);
  } else if constexpr (I < kNumHot) {
    constexpr HotShape h = kHotShapes[I];
    if constexpr (std::is_same<C, CfgLarge>::value && !h.small_m && h.mode == MODE &&
                  h.quant == QUANT) {
      if (hot == I) {
        hipLaunchKernelGGL((gemm_fp8_bs_kernel<C, MODE, QUANT, h.n, h.k>), dim3((unsigned)grid),
                           dim3(C::THREADS), 0, stream, a, remap);
        return;
      }
    }
    launch_persistent<C, MODE, QUANT, 0, I + 1>(a, hot, grid, remap, stream);
  } else {
    hipLaunchKernelGGL((gemm_fp8_bs_kernel<C, MODE, QUANT>), dim3((unsigned)grid),
                       dim3(C::THREADS), 0, stream, a, remap);
  }
}

template <class C>
hipError_t launch_cfg(const GemmArgs& args, const DeviceInfo& dev, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  const bool expert_blocks = args.mode == MODE_CONTIGUOUS && C::BM > 128;
  int64_t tiles_max;
  const int64_t grid = launch_grid<C>(args, dev, &tiles_max);
  if (tiles_max <= 0) return hipSuccess;
  const int remap = (grid % 8 == 0) ? 1 : 0;
  const int64_t nkb = (args.K + BK - 1) / BK;
  constexpr int PARTS = C::BM / RED_ROWS;
  const int hot = hot_index<C>(args);
  if (args.mode == MODE_DENSE && args.qd) {
    if constexpr (C::WN == 128) {
      launch_persistent<C, MODE_DENSE, true>(args, hot, grid, remap, stream);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;     // (choose_cfg gives the quantising epilogue 128-column waves)
  }
  if (args.mode == MODE_DENSE) {
    launch_persistent<C, MODE_DENSE, false>(args, hot, grid, remap, stream);
    return hipGetLastError();
  }
  if (args.mode == MODE_PERTENSOR) {
    switch (args.fmts) {
      case FMT_E4M3 | FMT_E4M3 << 4:
        launch_persistent<C, MODE_PERTENSOR, false>(args, hot, grid, remap, stream);
        break;
      case FMT_E5M2 | FMT_E4M3 << 4:
        launch_persistent<C, MODE_PERTENSOR, false, 0x01>(args, hot, grid, remap, stream);
        break;
      case FMT_E4M3 | FMT_E5M2 << 4:
        launch_persistent<C, MODE_PERTENSOR, false, 0x10>(args, hot, grid, remap, stream);
        break;
      case FMT_E5M2 | FMT_E5M2 << 4:
        launch_persistent<C, MODE_PERTENSOR, false, 0x11>(args, hot, grid, remap, stream);
        break;
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // Contiguous layout: its tiles (nearly) all cost the same. When the last
  // round of the persistent walk would run at most half full, its tiles are
  // cut into K pieces that fill that round instead (in the same launch:
  // every workgroup runs its full tiles, then at most one piece), and
  // reduce_split_kernel sums the pieces. With 128-row tiles tiles_max is
  // exact and the host plans the split; with 256-row tiles the count
  // depends on the device-side offsets and the kernel plans it (the host
  // only supplies the workspace when more than one round is possible). (The
  // masked layout gains nothing from it: its last-round tiles are the
  // smallest experts', which already cost less; measured 136.4 us unsplit
  // against 139.7 us.)
  int splits = 1;
  if (args.mode == MODE_CONTIGUOUS && !expert_blocks) splits = choose_splits(tiles_max, grid, nkb);
  const bool device_plan = expert_blocks && tiles_max > grid;
  const int64_t full = (tiles_max / grid) * grid;
  if ((splits > 1 || device_plan) && ws && ws_bytes >= split_bytes<C>(grid)) {
    GemmArgs sp = args;
    sp.ws_meta = static_cast<SplitMeta*>(ws);
    sp.ws = reinterpret_cast<float*>(static_cast<char*>(ws) + split_head_bytes<C>(grid));
    sp.split_base = (int)full;
    sp.splits = splits;
    // reduction work items: host-planned, exact; device-planned, at most
    // half a round of tail tiles, walked grid-stride
    const int64_t red_grid = device_plan ? (int64_t)dev.cu_count * 4 : (tiles_max - full) * PARTS;
    launch_persistent<C, MODE_CONTIGUOUS, false>(sp, hot, grid, remap, stream);
    hipLaunchKernelGGL((reduce_split_kernel<C>), dim3((unsigned)red_grid), dim3(256), 0, stream,
                       args.d, args.N, (const float*)sp.ws, (const SplitMeta*)sp.ws_meta);
    return hipGetLastError();
  }
  if (args.mode == MODE_CONTIGUOUS)
    launch_persistent<C, MODE_CONTIGUOUS, false>(args, hot, grid, remap, stream);
  else
    launch_persistent<C, MODE_MASKED, false>(args, hot, grid, remap, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small-M (decode-shaped) dense GEMM, M <= 32: every output row fits in one
// or two 16-row MFMA tiles, so the work is B streaming. One workgroup owns
// 16 output columns (grid = N / 16) and splits K over its 8 waves: wave v
// takes K blocks [v * kpw, (v + 1) * kpw) of each chunk of 8 * kpw blocks.
// Each element of B is used by exactly one MFMA, so fragments go straight
// from global memory into VGPRs (no LDS staging), and a wave issues all of a
// chunk's loads before its first MFMA to keep many bytes in flight. The
// same promotion as the main kernel is applied per K block; the eight waves'
// fp32 partial tiles are then summed through LDS (a fixed order, so the
// result is deterministic) and stored as bf16.
constexpr int SM_WAVES = 8;

// (KS > 0: K fixed at compile time, the kernel table's decode entry;
// KTAIL: K is not a multiple of 128, so the last block's fragments are
// loaded half by half, a half past K as zeros; a separate instantiation, so
// that the aligned kernel carries no per-load selects.)
template <int MT, int KPW, int KS = 0, bool KTAIL = false>
__global__ void __launch_bounds__(SM_WAVES * 64, 1)
gemm_smallm_kernel(const uint8_t* __restrict__ a, const float* __restrict__ sa,
                   const uint8_t* __restrict__ b, const float* __restrict__ sb,
                   uint16_t* __restrict__ d, int M, int64_t N, int64_t K_arg) {
  const int64_t K = KS > 0 ? (int64_t)KS : K_arg;
  // B is the MFMA's first operand (as in the main kernel), so lane l holds
  // output row mt * 16 + (l & 15) and columns n0 + 4 (l >> 4) .. +3: one A
  // row scale per lane and K block, and one 8-byte store per lane.
  __shared__ float4 red[SM_WAVES][MT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nkb = (int)((K + BK - 1) / BK);
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int kbyte = (lane >> 4) * 32;
  // (K % 16 == 0: each 16-byte half of a lane's 32 fragment bytes lies
  // wholly inside or wholly past K; past K it is zero, its bytes never used)
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
  const float* sbn = sb + (n0 / 128) * nkb;
  const uint8_t* brow = b + (n0 + (lane & 15)) * K;
  const uint8_t* arow[MT];
  int srow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    srow[mt] = min(mt * 16 + (lane & 15), M - 1);
    arow[mt] = a + (int64_t)srow[mt] * K;
  }
  v4f acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < nkb; c0 += SM_WAVES * KPW) {
    const int kb0 = c0 + wave * KPW;
    // (wave-uniform; a constant KPW where K is fixed and a whole number of
    // chunks)
    constexpr bool kWhole = KS > 0 && (KS / BK) % (SM_WAVES * KPW) == 0;
    const int cnt = kWhole ? KPW : smallm_count(nkb, c0, wave, KPW);
    uint4 bf[KPW][2];
    uint4 af[KPW][MT][2];
    float sav[KPW][MT];
    float sbv[KPW];
    // A wave with blocks in this chunk issues all KPW slots' loads, none
    // behind a branch of its own (branches between them serialise the
    // loads, ~3x slower): slots past the chunk's end load the last block
    // again and are not used, and a 16-byte half that lies past K (ragged K)
    // loads the row's last 16 bytes, which exist, and is replaced by zeros.
    // A wave without blocks in the chunk loads nothing.
    if (cnt > 0) {
#pragma unroll
      for (int t = 0; t < KPW; ++t) {
        const SmallMSlot sl = smallm_slot<KTAIL>(K, nkb, kb0, t, kbyte);
        const uint4 b0 = *reinterpret_cast<const uint4*>(brow + sl.o0);
        const uint4 b1 = *reinterpret_cast<const uint4*>(brow + sl.o1);
        bf[t][0] = sl.h0 ? b0 : z4;
        bf[t][1] = sl.h1 ? b1 : z4;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint4 a0 = *reinterpret_cast<const uint4*>(arow[mt] + sl.o0);
          const uint4 a1 = *reinterpret_cast<const uint4*>(arow[mt] + sl.o1);
          af[t][mt][0] = sl.h0 ? a0 : z4;
          af[t][mt][1] = sl.h1 ? a1 : z4;
          sav[t][mt] = sa[(int64_t)sl.kb * M + srow[mt]];
        }
        sbv[t] = sbn[sl.kb];
      }
    }
    // (every load of the chunk issued before the first MFMA: the scheduler
    // would otherwise trade bytes in flight for registers)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < KPW; ++t) {
      if (t < cnt) {
        v8i bv;
        bv[0] = (int)bf[t][0].x; bv[1] = (int)bf[t][0].y; bv[2] = (int)bf[t][0].z;
        bv[3] = (int)bf[t][0].w; bv[4] = (int)bf[t][1].x; bv[5] = (int)bf[t][1].y;
        bv[6] = (int)bf[t][1].z; bv[7] = (int)bf[t][1].w;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          v8i av;
          av[0] = (int)af[t][mt][0].x; av[1] = (int)af[t][mt][0].y; av[2] = (int)af[t][mt][0].z;
          av[3] = (int)af[t][mt][0].w; av[4] = (int)af[t][mt][1].x; av[5] = (int)af[t][mt][1].y;
          av[6] = (int)af[t][mt][1].z; av[7] = (int)af[t][mt][1].w;
          const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bv, av, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
          const float c = sav[t][mt] * sbv[t];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[mt][e] = __builtin_fmaf(p[e], c, acc[mt][e]);
        }
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    red[wave][mt][lane] = make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
  __syncthreads();
  if (wave < MT) {
    // wave mt sums the eight partial tiles of MFMA row tile mt in wave order
    const int mt = wave;
    float4 sum = red[0][mt][lane];
#pragma unroll
    for (int v = 1; v < SM_WAVES; ++v) {
      const float4 x = red[v][mt][lane];
      sum.x += x.x; sum.y += x.y; sum.z += x.z; sum.w += x.w;
    }
    const int r = mt * 16 + (lane & 15);
    if (r < M) {
      uint2 v;
      v.x = bf16x2_rne(sum.x, sum.y);
      v.y = bf16x2_rne(sum.z, sum.w);
      *reinterpret_cast<uint2*>(d + (int64_t)r * N + n0 + (lane >> 4) * 4) = v;
    }
  }
}

template <int MT, int KPW, int KS = 0>
hipError_t launch_smallm(const GemmArgs& args, hipStream_t stream) {
  if (KS == 0 && args.K % BK != 0) {
    hipLaunchKernelGGL((gemm_smallm_kernel<MT, KPW, 0, true>), dim3((unsigned)(args.N / 16)),
                       dim3(SM_WAVES * 64), 0, stream, args.a, args.sa, args.b, args.sb, args.d,
                       (int)args.rows, args.N, args.K);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_smallm_kernel<MT, KPW, KS>), dim3((unsigned)(args.N / 16)),
                     dim3(SM_WAVES * 64), 0, stream, args.a, args.sa, args.b, args.sb, args.d,
                     (int)args.rows, args.N, args.K);
  return hipGetLastError();
}

// Tile configuration: the split-K small-M kernel for M <= 32 (dense),
// 256-row tiles where rows come in large blocks (contiguous experts:
// enumerated expert by expert, up to 1024 experts), 128-row tiles where M is
// small or the experts too many for the per-expert metadata. Every
// configuration applies the same per-element arithmetic (one 16x16x128 MFMA
// per output tile and K block, the same lane -> K assignment, the same
// promotion order), so the choice changes speed, never bits, except that the
// small-M kernel sums its K split in a fixed order of its own.
enum CfgChoice { CFG_SMALL, CFG_MID, CFG_LARGE };
CfgChoice choose_cfg(const GemmArgs& args, int expected_m) {
  if (args.mode == MODE_DENSE && args.qd) return CFG_LARGE;    // fused epilogue: 128-column waves
  if (args.mode == MODE_DENSE && args.rows <= 32) return CFG_SMALL;
  if (args.mode == MODE_PERTENSOR) return args.rows > 128 ? CFG_LARGE : CFG_MID;
  bool large;
  if (args.mode == MODE_CONTIGUOUS)
    large = args.G <= MAX_MASKED_GROUPS;   // 256-row tiles enumerated per expert
  else if (args.mode == MODE_MASKED)
    large = (expected_m > 0 ? expected_m : args.rows) > 128;
  else
    large = args.rows > 128;
  return large ? CFG_LARGE : CFG_MID;
}

// Scratch of the allocation-free contiguous entry point: a split-tail
// workspace (header plus one fp32 256x256 partial tile per workgroup) for
// launches of up to kScratchCUs workgroups, part of the code object, so that
// the call needs no allocation. Each device holds its own copy at its own
// address; host code must use the address hipGetSymbolAddress returns for
// the current device (scratch_ptr), never the array's name.
constexpr int kScratchCUs = 256;
constexpr size_t kScratchBytes = ((sizeof(SplitMeta) + kScratchCUs * sizeof(SplitTile) + 255) /
                                  256 * 256) +
                                 (size_t)kScratchCUs * CfgLarge::BM * CfgLarge::BN * sizeof(float);
static_assert(kScratchBytes >= (size_t)kScratchCUs * CfgMid::BM * CfgMid::BN * sizeof(float),
              "the 128-row configuration's pieces fit as well");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

// Device address of this device's scratch array (nullptr if the symbol
// cannot be resolved), looked up once per device with that device current.
void* scratch_ptr(int device) {
  constexpr int kMaxDev = 64;
  static std::once_flag once[kMaxDev];
  static void* ptr[kMaxDev];
  if (device < 0 || device >= kMaxDev) return nullptr;
  std::call_once(once[device], [device] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) ptr[device] = p;
    else (void)hipGetLastError();
  });
  return ptr[device];
}

size_t contiguous_workspace_bytes(const GemmArgs& args, const DeviceInfo& dev) {
  return choose_cfg(args, 0) == CFG_LARGE ? contiguous_ws_bytes<CfgLarge>(args, dev)
                                          : contiguous_ws_bytes<CfgMid>(args, dev);
}

// Which kernel a call runs: the configuration, the kernel table entry (-1:
// generic) and, for the small-M kernel, its template arguments.
struct Selection {
  CfgChoice cfg;
  int hot;
  int mt, kpw;
};

Selection select_kernel(const GemmArgs& args, int expected_m) {
  Selection sel{choose_cfg(args, expected_m), -1, 0, 0};
  if (sel.cfg == CFG_SMALL) {
    // K blocks per wave: enough that 8 waves cover K in one chunk, capped by
    // the registers the fragments need
    const int64_t nkb = (args.K + BK - 1) / BK;
    sel.mt = args.rows <= 16 ? 1 : 2;
    sel.kpw = sel.mt == 2 ? 4 : (nkb <= 8 * 4 ? 4 : (nkb <= 8 * 7 ? 7 : 8));
    if (g_specialise.load(std::memory_order_relaxed))
      for (int i = 0; i < kNumHot; ++i)
        if (kHotShapes[i].small_m && kHotShapes[i].k == args.K && sel.mt == 1 && sel.kpw == 7)
          sel.hot = i;
  } else if (sel.cfg == CFG_LARGE) {
    sel.hot = hot_index<CfgLarge>(args);
  }
  return sel;
}

hipError_t launch_gemm(const GemmArgs& args, const DeviceInfo& dev, int expected_m, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  const Selection sel = select_kernel(args, expected_m);
  if (sel.cfg == CFG_SMALL) {
    if (sel.mt == 2) return launch_smallm<2, 4>(args, stream);
    if (sel.kpw == 4) return launch_smallm<1, 4>(args, stream);
    if (sel.kpw == 8) return launch_smallm<1, 8>(args, stream);
    if (sel.hot >= 0) return launch_smallm<1, 7, kSmallMHotK>(args, stream);
    return launch_smallm<1, 7>(args, stream);
  }
  return sel.cfg == CFG_LARGE ? launch_cfg<CfgLarge>(args, dev, ws, ws_bytes, stream)
                              : launch_cfg<CfgMid>(args, dev, ws, ws_bytes, stream);
}

int describe_gemm(const GemmArgs& args, int expected_m, char* buf, size_t len) {
  static const char* const kLayout[] = {"dense", "contiguous", "masked", "per-tensor"};
  const Selection sel = select_kernel(args, expected_m);
  const char* layout = kLayout[args.mode];
  char spec[64] = "generic";
  if (sel.hot >= 0) {
    const HotShape& h = kHotShapes[sel.hot];
    if (h.small_m) snprintf(spec, sizeof spec, "specialised K%d", h.k);
    else snprintf(spec, sizeof spec, "specialised N%d K%d", h.n, h.k);
  }
  int n;
  if (sel.cfg == CFG_SMALL)
    n = snprintf(buf, len, "small-M split-K, %d row tile(s), %d K blocks per wave, %s", sel.mt,
                 sel.kpw, spec);
  else
    n = snprintf(buf, len, "persistent %dx%d%s, %s, %s", sel.cfg == CFG_LARGE ? 256 : 128, 256,
                 args.qd ? " quantising epilogue" : "", layout, spec);
  return n;
}

void set_shape_specialisation(int enable) {
  g_specialise.store(enable ? 1 : 0, std::memory_order_relaxed);
}

// Every GEMM kernel of the library, generic and specialised, for warm-up.
template <class C, int MODE, bool QUANT, int I = 0>
void collect_persistent(std::vector<const void*>& out) {
  if constexpr (I == 0)
    out.push_back(reinterpret_cast<const void*>(&gemm_fp8_bs_kernel<C, MODE, QUANT, 0, 0, 0, true>));
  if constexpr (I < kNumHot) {
    constexpr HotShape h = kHotShapes[I];
    if constexpr (std::is_same<C, CfgLarge>::value && !h.small_m && h.mode == MODE &&
                  h.quant == QUANT)
      out.push_back(reinterpret_cast<const void*>(&gemm_fp8_bs_kernel<C, MODE, QUANT, h.n, h.k>));
    collect_persistent<C, MODE, QUANT, I + 1>(out);
  } else {
    out.push_back(reinterpret_cast<const void*>(&gemm_fp8_bs_kernel<C, MODE, QUANT>));
  }
}

void gemm_kernels(std::vector<const void*>& out) {
  collect_persistent<CfgLarge, MODE_DENSE, false>(out);
  collect_persistent<CfgLarge, MODE_DENSE, true>(out);
  collect_persistent<CfgLarge, MODE_PERTENSOR, false>(out);
  collect_persistent<CfgLarge, MODE_CONTIGUOUS, false>(out);
  collect_persistent<CfgLarge, MODE_MASKED, false>(out);
  collect_persistent<CfgMid, MODE_DENSE, false>(out);
  collect_persistent<CfgMid, MODE_PERTENSOR, false>(out);
  collect_persistent<CfgMid, MODE_CONTIGUOUS, false>(out);
  collect_persistent<CfgMid, MODE_MASKED, false>(out);
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgLarge, MODE_PERTENSOR, false, 0, 0, 0x01>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgLarge, MODE_PERTENSOR, false, 0, 0, 0x10>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgLarge, MODE_PERTENSOR, false, 0, 0, 0x11>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgMid, MODE_PERTENSOR, false, 0, 0, 0x01>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgMid, MODE_PERTENSOR, false, 0, 0, 0x10>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgMid, MODE_PERTENSOR, false, 0, 0, 0x11>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgLarge, MODE_PERTENSOR, false, 0, 0, 0x01, true>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgLarge, MODE_PERTENSOR, false, 0, 0, 0x10, true>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgLarge, MODE_PERTENSOR, false, 0, 0, 0x11, true>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgMid, MODE_PERTENSOR, false, 0, 0, 0x01, true>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgMid, MODE_PERTENSOR, false, 0, 0, 0x10, true>));
  out.push_back(reinterpret_cast<const void*>(
      &gemm_fp8_bs_kernel<CfgMid, MODE_PERTENSOR, false, 0, 0, 0x11, true>));
  out.push_back(reinterpret_cast<const void*>(&reduce_split_kernel<CfgLarge>));
  out.push_back(reinterpret_cast<const void*>(&reduce_split_kernel<CfgMid>));
  out.push_back(reinterpret_cast<const void*>(&gemm_smallm_kernel<1, 4>));
  out.push_back(reinterpret_cast<const void*>(&gemm_smallm_kernel<1, 7>));
  out.push_back(reinterpret_cast<const void*>(&gemm_smallm_kernel<1, 8>));
  out.push_back(reinterpret_cast<const void*>(&gemm_smallm_kernel<2, 4>));
  out.push_back(reinterpret_cast<const void*>(&gemm_smallm_kernel<1, 4, 0, true>));
  out.push_back(reinterpret_cast<const void*>(&gemm_smallm_kernel<1, 7, 0, true>));
  out.push_back(reinterpret_cast<const void*>(&gemm_smallm_kernel<1, 8, 0, true>));
  out.push_back(reinterpret_cast<const void*>(&gemm_smallm_kernel<2, 4, 0, true>));
  out.push_back(
      reinterpret_cast<const void*>(&gemm_smallm_kernel<1, 7, kSmallMHotK>));
}

}  // namespace fp8g
