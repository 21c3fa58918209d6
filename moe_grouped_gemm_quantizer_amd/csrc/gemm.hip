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
//  * Workgroup tiles are BM x BN with (BM/64) x (BN/128) waves: 256x256 with
//    8 waves (two per SIMD, so one wave's promotion FMAs and LDS reads fill
//    the other's MFMA shadow) where rows come in large blocks; 128x256 with
//    4 waves and three LDS stages where M is cut into 128-row blocks.
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
//    Waves whose 64 rows hold no valid row skip the arithmetic; rows past an
//    expert's valid count are never stored.

#include <stdlib.h>
#include <string.h>

#include "internal.h"

namespace fp8g {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BK = 128;            // K block = one scale block = one MFMA K
constexpr int MAX_MASKED_GROUPS = 1024;

template <int BM_, int BN_, int STAGES_, int GROUP_M_, int PBUF_, int WM_, int WN_>
struct Cfg {
  static constexpr int PBUF = PBUF_;                    // MFMA result buffers (1 or 2)
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int STAGES = STAGES_;
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int WM = WM_;                        // wave tile rows
  static constexpr int WN = WN_;                        // wave tile columns (64 or 128)
  static constexpr int TM = WM / 16;                    // MFMA tiles per wave, M
  static constexpr int TN = WN / 16;                    // MFMA tiles per wave, N
  static constexpr int WAVES_M = BM / WM;
  static constexpr int WAVES_N = BN / WN;
  static constexpr int NB128 = BN / 128;                // 128-column scale blocks per tile
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int SA_OFFSET = (BM + BN) * BK;     // A row scales of the K block
  static constexpr int SB_OFFSET = SA_OFFSET + BM * 4; // B scales of the K block, per 128 cols
  static constexpr int STAGE_BYTES = SB_OFFSET + 16;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int COPIES = (BM + BN) / 8;         // 8-row copy instructions per stage
  static constexpr int COPIES_PER_WAVE = COPIES / WAVES;
  static constexpr int SA_WAVES = BM / 64;             // waves that also copy 64 row scales
  static constexpr int SB_WAVE = WAVES - 1;            // the wave that copies the B scales
  static constexpr int A_COPIES = BM / (8 * WAVES);     // copies per wave that move A rows
  static_assert(COPIES % WAVES == 0, "copies must split evenly over the waves");
  static_assert((BM / 8) % WAVES == 0 && WAVES % 2 == 0, "A/B split and swizzle parity per wave");
  static_assert(SA_WAVES < WAVES, "one wave per 64 row scales, another for the B scales");
  static_assert(NB128 <= 4 && 128 % WN == 0, "B scales of a stage fit in 16 bytes");
  static_assert(LDS_BYTES + 4 * (MAX_MASKED_GROUPS + 1) <= 160 * 1024, "LDS budget");
};

#ifndef LARGE_PBUF
#define LARGE_PBUF 1
#endif
// dense / masked with large M: 8 waves of 64x128
using CfgLarge = Cfg<256, 256, 2, 4, LARGE_PBUF, 64, 128>;
// 128-row blocks (contiguous experts, M <= 128): 8 waves of 64x64
using CfgMid = Cfg<128, 256, 3, 8, 2, 64, 64>;

struct TileInfo {
  const uint8_t* a;      // first row of the tile's A rows
  const float* sa;       // scale of the tile's first row, K block 0
  const uint8_t* b;      // first row of the tile's B rows (expert applied)
  const float* sb;       // scale of the tile's first N block, K block 0
  uint16_t* d;           // first output row of the tile, column n0
  int mvalid;            // rows of the tile that exist (1..BM)
  int nvalid;            // columns of the tile that exist (multiple of 128, 128..BN)
  int kblocks;           // K / 128 (row length of the B scale array)
};

// LDS swizzle of the 16-byte chunk index within a 128-byte row:
// chunk ^ (row & 7) ^ ((row >> 3) & 1). Any 8 consecutive rows then use 8
// distinct chunks (conflict-free for 8 lanes x 16 B on 32 banks), and so do
// the even rows and the odd rows of any 16 consecutive rows (conflict-free
// for 16 lanes x 16 B on 64 banks, where rows r and r+2 share banks).
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ (row & 7) ^ ((row >> 3) & 1);
}

// float -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds)
               : "memory");
}

// Global -> LDS copy of one K block of the A and B tiles and of the A row
// and B column-block scales. One 16-byte copy moves 8 rows x 128 bytes:
// lane l takes row base + (l >> 3) and, because its destination chunk is
// fixed to (l & 7), reads the logical chunk (l & 7) ^ (l >> 3) ^ parity so
// that the LDS image is the swizzled layout (swz). Wave w issues copies for
// the 8-row groups w, w + WAVES, ...; the first A_COPIES of them are A rows.
// Everything but the K offset is fixed for a tile, so it is computed once
// per tile (CopyPlan): each copy's per-lane byte offset from the tile's A or
// B base, with rows past mvalid (A) or nvalid (B) clamped to the last row
// that exists (read in bounds, never stored). A K step then only advances
// the base pointers and issues the copies. Every wave issues the same number
// of copies whatever the tile, which the counted waits rely on.
template <class C>
struct CopyPlan {
  uint32_t voff[C::COPIES_PER_WAVE];   // per-lane offsets from the A / B tile base
  uint32_t sa_voff;                    // per-lane offset of this lane's A row scale
  uint32_t sb_voff;                    // per-lane offset of this lane's B block scale
  uint32_t dst0;                       // LDS offset of this wave's first 8-row group
  int wave;
};

template <class C>
__device__ __forceinline__ void make_plan(CopyPlan<C>& pl, const TileInfo& ti, int64_t K) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // swizzle: row & 7 = lane >> 3, and (row >> 3) & 1 = wave & 1 for every
  // group of this wave (WAVES is even)
  const uint32_t ch = (uint32_t)((lane & 7) ^ (lane >> 3) ^ (wave & 1));
  const uint32_t Ku = (uint32_t)K;
#pragma unroll
  for (int i = 0; i < C::COPIES_PER_WAVE; ++i) {
    const int grp = wave + i * C::WAVES;
    int r;
    if (i < C::A_COPIES) {
      r = grp * 8 + (lane >> 3);
      r = r < ti.mvalid ? r : ti.mvalid - 1;
    } else {
      r = grp * 8 - C::BM + (lane >> 3);
      r = r < ti.nvalid ? r : ti.nvalid - 1;
    }
    pl.voff[i] = (uint32_t)r * Ku + ch * 16u;
  }
  const int ra = wave * 64 + lane;
  pl.sa_voff = (uint32_t)(ra < ti.mvalid ? ra : ti.mvalid - 1) * 4u;
  const int nb = lane * 128 < ti.nvalid ? lane : (ti.nvalid / 128) - 1;
  pl.sb_voff = (uint32_t)nb * (uint32_t)ti.kblocks * 4u;
  pl.dst0 = (uint32_t)wave * 8u * BK;
  pl.wave = wave;
}

template <class C>
__device__ __forceinline__ void issue_stage(const CopyPlan<C>& pl, const TileInfo& ti,
                                            int64_t sa_ld, int kb, uint32_t stage_lds) {
  const int lane = threadIdx.x & 63;
  const uint8_t* abase = ti.a + (int64_t)kb * BK;
  const uint8_t* bbase = ti.b + (int64_t)kb * BK;
#pragma unroll
  for (int i = 0; i < C::COPIES_PER_WAVE; ++i)
    dma16(i < C::A_COPIES ? abase : bbase, pl.voff[i],
          stage_lds + pl.dst0 + (uint32_t)(i * C::WAVES * 8 * BK));
  if (pl.wave < C::SA_WAVES)
    dma4(ti.sa + (int64_t)kb * sa_ld, pl.sa_voff, stage_lds + C::SA_OFFSET + pl.wave * 256);
  // lane n < NB128 copies the scale of the tile's n-th 128-column block
  if (pl.wave == C::SB_WAVE && lane < C::NB128)
    dma4(ti.sb + kb, pl.sb_voff, stage_lds + C::SB_OFFSET);
}

// Wait until this wave's copies of the stage about to be read have landed,
// allowing `newer` later-issued stages to stay in flight.
template <class C>
__device__ __forceinline__ void wait_stage(int newer) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (newer == 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  } else if (wave < C::SA_WAVES || wave == C::SB_WAVE) {
    __builtin_amdgcn_s_waitcnt(vmcnt_only(C::COPIES_PER_WAVE + 1));
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_only(C::COPIES_PER_WAVE));
  }
}

// Workgroup barrier without the memory fences of __syncthreads(), which
// would drain every copy in flight. Visibility is handled explicitly: each
// wave waits for its own copies of the stage to be read (wait_stage) before
// arriving, and every LDS read of a stage feeds an MFMA or FMA before the
// wave leaves the K step, so no read is pending when a stage is refilled.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

// One K step: start the copy of K block `kb_next` into `nxt` (if any) and
// multiply the K block held in `cur` into the accumulators. The 16-column
// slices of the wave tile are software-pipelined: the MFMAs of slice j run
// while the promotion FMAs of slice j-1 (whose MFMA results are ready by
// then) and the LDS reads of slice j+1 issue, so the VALU work and the
// fragment loads hide in the MFMA shadow instead of waiting on it.
template <class C>
__device__ __forceinline__ void k_step(v4f (&acc)[C::TM][C::TN], const CopyPlan<C>& pl,
                                       const TileInfo& ti, int64_t sa_ld, int kb_next,
                                       bool do_copy, uint32_t nxt_lds,
                                       const uint8_t* __restrict__ cur, int wm, int wn, int rlane,
                                       bool active) {
  const int lane = threadIdx.x & 63;
  if (do_copy) issue_stage<C>(pl, ti, sa_ld, kb_next, nxt_lds);
  if (!active) return;
  const float* sas = reinterpret_cast<const float*>(cur + C::SA_OFFSET);
  const float sbv = reinterpret_cast<const float*>(cur + C::SB_OFFSET)[(wn * C::WN) / 128];
  const uint8_t* btile = cur + C::BM * BK;
  float cs[C::TM][4];
  v8i af[C::TM];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const float4 sa4 = *reinterpret_cast<const float4*>(sas + rlane + i * 16);
    cs[i][0] = sa4.x * sbv; cs[i][1] = sa4.y * sbv;
    cs[i][2] = sa4.z * sbv; cs[i][3] = sa4.w * sbv;
    af[i] = load_frag(cur, wm * C::WM + i * 16, lane);
  }
  v8i bf = load_frag(btile, wn * C::WN, lane);
  if constexpr (C::PBUF == 2) {
    // MFMA results double-buffered: slice j's MFMAs issue while slice j-1's
    // results (ready by then) are promoted
    v4f p[2][C::TM];
#pragma unroll
    for (int j = 0; j <= C::TN; ++j) {
      v8i bnext;
      if (j + 1 < C::TN) bnext = load_frag(btile, wn * C::WN + (j + 1) * 16, lane);
      if (j < C::TN) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
          p[j & 1][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[i], bf, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
      }
      if (j > 0) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j - 1][e] = __builtin_fmaf(p[(j - 1) & 1][i][e], cs[i][e], acc[i][j - 1][e]);
      }
      if (j + 1 < C::TN) bf = bnext;
    }
  } else {
    // single-buffered: each slice is promoted right after its MFMAs; the
    // other wave on the SIMD covers the wait for the results
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      v8i bnext;
      if (j + 1 < C::TN) bnext = load_frag(btile, wn * C::WN + (j + 1) * 16, lane);
      v4f p[C::TM];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        p[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf,
                                                                v4f{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(p[i][e], cs[i][e], acc[i][j][e]);
      if (j + 1 < C::TN) bf = bnext;
    }
  }
}

template <class C>
__device__ void run_tile(const TileInfo& ti, int64_t N, int64_t K, int64_t sa_ld,
                         int64_t kblocks, uint8_t* lds) {
  const int lane = threadIdx.x & 63;
  // wave index through readfirstlane so that everything derived from it
  // (notably the B scale address) is known to be wave-uniform (SGPRs)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WAVES_N;
  const int wn = wave % C::WAVES_N;
  const int nkb = (int)(K / BK);
  const int rlane = wm * C::WM + (lane >> 4) * 4;   // first accumulator row of this lane
  // 16-row MFMA tiles of this wave that hold valid rows (wave-uniform); a
  // wave with none skips the K loop's arithmetic, a partly valid wave
  // multiplies its clamped duplicate rows too and drops them at the store
  const int tm_active = min(C::TM, max(0, (ti.mvalid - wm * C::WM + 15) / 16));
  const bool active = tm_active > 0 && wn * C::WN < ti.nvalid;

  v4f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // prologue: the first STAGES-1 K blocks in flight
  const uint32_t lds_base = lds_addr(lds);
  CopyPlan<C> pl;
  make_plan<C>(pl, ti, K);
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < nkb) issue_stage<C>(pl, ti, sa_ld, s, lds_base + s * C::STAGE_BYTES);

  for (int kb = 0; kb < nkb; ++kb) {
    // copies of later stages that may stay in flight past this wait
    wait_stage<C>(min(C::STAGES - 2, nkb - 1 - kb));
    wg_barrier();                    // every wave's copies of stage kb are visible
    const int kn = kb + C::STAGES - 1;
    k_step<C>(acc, pl, ti, sa_ld, kn, kn < nkb, lds_base + (kn % C::STAGES) * C::STAGE_BYTES,
              lds + (kb % C::STAGES) * C::STAGE_BYTES, wm, wn, rlane, active);
  }
  // all waves are done reading the last stage before the next tile reuses LDS
  wg_barrier();

  if (!active) return;
  // epilogue: bf16 RNE, rows past mvalid are not written
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rlane + i * 16 + e;
      if (r < ti.mvalid) {
        uint16_t* drow = ti.d + (int64_t)r * N + wn * C::WN + (lane & 15);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) drow[j * 16] = (uint16_t)bf16_rne(acc[i][j][e]);
      }
    }
  }
}

// Tile order: slot -> (m-block, n-block) with group_m m-blocks per group.
__device__ __forceinline__ void swizzle_tile(int slot, int mblocks, int nblocks, int group_m,
                                             int& mb, int& nb) {
  const int per_group = group_m * nblocks;
  const int group = slot / per_group;
  const int first_m = group * group_m;
  const int gsize = min(mblocks - first_m, group_m);
  const int in_group = slot - group * per_group;
  mb = first_m + in_group % gsize;
  nb = in_group / gsize;
}

template <class C>
__global__ void __launch_bounds__(C::THREADS, 1)
gemm_fp8_bs_kernel(GemmArgs args, int xcd_remap) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS_BYTES];
  __shared__ int prefix[MAX_MASKED_GROUPS + 1];

  const int64_t N = args.N;
  const int64_t K = args.K;
  const int64_t kblocks = K / BK;
  const int nblocks128 = (int)(N / 128);
  const int nblocks = (int)((N + C::BN - 1) / C::BN);
  int mblocks;

  if (args.mode == MODE_MASKED) {
    // per-expert m-block counts -> prefix sums, computed by thread 0
    if (threadIdx.x == 0) {
      int acc = 0;
      prefix[0] = 0;
      for (int g = 0; g < args.G; ++g) {
        int m = args.group[g];
        m = m < 0 ? 0 : (m > args.rows ? (int)args.rows : m);
        acc += (m + C::BM - 1) / C::BM;
        prefix[g + 1] = acc;
      }
    }
    __syncthreads();
    mblocks = prefix[args.G];
  } else {
    mblocks = (int)((args.rows + C::BM - 1) / C::BM);
  }
  const int tiles = mblocks * nblocks;
  const int grid = gridDim.x;
  const int w = blockIdx.x;
  const int lane_slot = xcd_remap ? (w & 7) * (grid >> 3) + (w >> 3) : w;

  for (int base = 0;; base += grid) {
    const int slot = base + lane_slot;
    if (slot >= tiles) break;
    int mb, nb;
    swizzle_tile(slot, mblocks, nblocks, C::GROUP_M, mb, nb);

    TileInfo ti;
    int g = 0;
    int64_t row_start;
    if (args.mode == MODE_DENSE) {
      row_start = (int64_t)mb * C::BM;
      ti.mvalid = (int)min((int64_t)C::BM, args.rows - row_start);
    } else if (args.mode == MODE_CONTIGUOUS) {
      row_start = (int64_t)mb * C::BM;
      // expert g: the last g with offsets[g] <= row_start (binary search)
      int lo = 0, hi = args.G - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if ((int64_t)args.group[mid] <= row_start) lo = mid; else hi = mid - 1;
      }
      g = lo;
      ti.mvalid = (int)min((int64_t)C::BM, args.rows - row_start);
    } else {
      int lo = 0, hi = args.G - 1;       // the last g with prefix[g] <= mb
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= mb) lo = mid; else hi = mid - 1;
      }
      g = lo;
      const int local = mb - prefix[g];
      int m = args.group[g];
      m = m < 0 ? 0 : (m > args.rows ? (int)args.rows : m);
      row_start = (int64_t)g * args.rows + (int64_t)local * C::BM;
      ti.mvalid = min(C::BM, m - local * C::BM);
    }
    const int64_t n0 = (int64_t)nb * C::BN;
    ti.nvalid = (int)min((int64_t)C::BN, N - n0);
    ti.a = args.a + row_start * K;
    ti.sa = args.sa + row_start;
    ti.b = args.b + ((int64_t)g * N + n0) * K;
    ti.sb = args.sb + ((int64_t)g * nblocks128 + n0 / 128) * kblocks;
    ti.kblocks = (int)kblocks;
    ti.d = args.d + row_start * N + n0;
    run_tile<C>(ti, N, K, args.sa_ld, kblocks, lds);
  }
}

template <class C>
hipError_t launch_cfg(const GemmArgs& args, const DeviceInfo& dev, hipStream_t stream) {
  const int64_t nblocks = (args.N + C::BN - 1) / C::BN;
  int64_t mblocks_max;
  if (args.mode == MODE_MASKED)
    mblocks_max = (int64_t)args.G * ((args.rows + C::BM - 1) / C::BM);
  else
    mblocks_max = (args.rows + C::BM - 1) / C::BM;
  const int64_t tiles_max = mblocks_max * nblocks;
  if (tiles_max <= 0) return hipSuccess;
  int64_t grid = dev.cu_count;
  if (grid > tiles_max) grid = tiles_max;
  const int remap = (grid % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(gemm_fp8_bs_kernel<C>, dim3((unsigned)grid), dim3(C::THREADS), 0, stream,
                     args, remap);
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

template <int MT, int KPW>
__global__ void __launch_bounds__(SM_WAVES * 64, 1)
gemm_smallm_kernel(const uint8_t* __restrict__ a, const float* __restrict__ sa,
                   const uint8_t* __restrict__ b, const float* __restrict__ sb,
                   uint16_t* __restrict__ d, int M, int64_t N, int64_t K) {
  __shared__ float4 red[SM_WAVES][MT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nkb = (int)(K / BK);
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t col = n0 + (lane & 15);
  const int kbyte = (lane >> 4) * 32;
  const float* sbn = sb + (n0 / 128) * nkb;
  const uint8_t* brow = b + col * K + kbyte;
  const uint8_t* arow[MT];
  int srow[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(mt * 16 + (lane & 15), M - 1);
    arow[mt] = a + (int64_t)r * K + kbyte;
#pragma unroll
    for (int e = 0; e < 4; ++e) srow[mt][e] = min(mt * 16 + (lane >> 4) * 4 + e, M - 1);
  }
  v4f acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < nkb; c0 += SM_WAVES * KPW) {
    const int kb0 = c0 + wave * KPW;
    const int cnt = max(0, min(KPW, nkb - kb0));      // wave-uniform
    uint4 bf[KPW][2];
    uint4 af[KPW][MT][2];
    float sav[KPW][MT][4];
    float sbv[KPW];
#pragma unroll
    for (int t = 0; t < KPW; ++t) {
      if (t < cnt) {
        const int64_t ko = (int64_t)(kb0 + t) * BK;
        bf[t][0] = *reinterpret_cast<const uint4*>(brow + ko);
        bf[t][1] = *reinterpret_cast<const uint4*>(brow + ko + 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          af[t][mt][0] = *reinterpret_cast<const uint4*>(arow[mt] + ko);
          af[t][mt][1] = *reinterpret_cast<const uint4*>(arow[mt] + ko + 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) sav[t][mt][e] = sa[(int64_t)(kb0 + t) * M + srow[mt][e]];
        }
        sbv[t] = sbn[kb0 + t];
      }
    }
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
              av, bv, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[mt][e] = __builtin_fmaf(p[e], sav[t][mt][e] * sbv[t], acc[mt][e]);
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
    const float vals[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = mt * 16 + (lane >> 4) * 4 + e;
      if (r < M) d[(int64_t)r * N + col] = (uint16_t)bf16_rne(vals[e]);
    }
  }
}

template <int MT, int KPW>
hipError_t launch_smallm(const GemmArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_smallm_kernel<MT, KPW>), dim3((unsigned)(args.N / 16)),
                     dim3(SM_WAVES * 64), 0, stream, args.a, args.sa, args.b, args.sb, args.d,
                     (int)args.rows, args.N, args.K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& args, const DeviceInfo& dev, int expected_m,
                       hipStream_t stream) {
  // Tile configuration: the split-K small-M kernel for M <= 32 (dense),
  // 256-row tiles where rows come in large blocks, 128-row tiles where M is
  // cut at multiples of 128 (contiguous experts) or is small.
  // FP8G_FORCE_CFG=large|mid overrides the choice (tuning only).
  static const char* force = getenv("FP8G_FORCE_CFG");
  bool large;
  if (args.mode == MODE_CONTIGUOUS)
    large = false;
  else if (args.mode == MODE_MASKED)
    large = (expected_m > 0 ? expected_m : args.rows) > 128;
  else
    large = args.rows > 128;
  bool small = args.mode == MODE_DENSE && args.rows <= 32;
  if (force && args.mode != MODE_CONTIGUOUS) {
    if (!strcmp(force, "large")) { large = true; small = false; }
    if (!strcmp(force, "mid")) { large = false; small = false; }
  }
  if (small) {
    // K blocks per wave: enough that 8 waves cover K in one chunk, capped by
    // the registers the fragments need
    const int64_t nkb = args.K / BK;
    if (args.rows <= 16) {
      if (nkb <= 8 * 4) return launch_smallm<1, 4>(args, stream);
      return launch_smallm<1, 8>(args, stream);
    }
    return launch_smallm<2, 4>(args, stream);
  }
  return large ? launch_cfg<CfgLarge>(args, dev, stream) : launch_cfg<CfgMid>(args, dev, stream);
}

}  // namespace fp8g
