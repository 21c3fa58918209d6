// Tile and copy index arithmetic of the persistent GEMM kernel (gemm.hip),
// written as functions that compile for the host as well as the device, so
// that a host build (tests/native/gemm_index_check.cpp) can enumerate every
// tile, copy source, scale read and store of a launch with these same
// functions and check each against the bounds of its buffer. Device-only
// details stay in gemm.hip; here a workgroup-uniform value goes through
// uniform(), which is readfirstlane on the device and the value itself on
// the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

#define FP8G_HD __host__ __device__ __forceinline__

namespace fp8g {
namespace gidx {

FP8G_HD int uniform(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_readfirstlane(x);
#else
  return x;
#endif
}
FP8G_HD int imin(int a, int b) { return a < b ? a : b; }
FP8G_HD int imax(int a, int b) { return a > b ? a : b; }
FP8G_HD int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }

constexpr int BK = 128;            // K block = one scale block = one MFMA K
constexpr int MAX_MASKED_GROUPS = 1024;

template <int BM_, int BN_, int STAGES_, int GROUP_M_, int PBUF_, int WM_, int WN_, int SPREAD_,
          int COPY_WAVES_, int PF_, int PRIO_>
struct Cfg {
  // issue priority (s_setprio) of the younger wave of each SIMD's pair, the
  // one that issues the copies; the older waves keep priority 0
  static constexpr int PRIO_YOUNG = PRIO_;
  static constexpr int PF = PF_;                        // B fragments read PF slices ahead
  static constexpr int NBF = PF + 1;                    // B fragment registers (ring)
  static constexpr int PBUF = PBUF_;                    // MFMA result buffers (1 or 2)
  static constexpr int SPREAD = SPREAD_;                // slices a stage's copies are spread over
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int STAGES = STAGES_;
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int WM = WM_;                        // wave tile rows
  static constexpr int WN = WN_;                        // wave tile columns (64 or 128)
  static constexpr int TM = WM / 16;                    // MFMA tiles per wave, M
  static constexpr int TN = WN / 16;                    // MFMA tiles per wave, N
  static constexpr int WAVES_M = BM / WM;
  // A wave's MFMA row tiles are interleaved with the other row bands': tile
  // i of band wm covers rows (wm + i * WAVES_M) * 16 .. +15, so a tile whose
  // first u 16-row slices hold rows spreads them evenly over the bands (and
  // over both SIMDs' wave pairs) when the rest is skipped.
  static constexpr int RSTEP = 16 * WAVES_M;
  static constexpr int WAVES_N = BN / WN;
  static constexpr int NB128 = BN / 128;                // 128-column scale blocks per tile
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int SA_OFFSET = (BM + BN) * BK;     // A row scales of the K block
  static constexpr int SB_OFFSET = SA_OFFSET + BM * 4; // B scales of the K block, per 128 cols
  static constexpr int STAGE_BYTES = SB_OFFSET + 16;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // The copies are issued by the last COPY_WAVES waves (copy wave index
  // cw = wave - FIRST_COPY_WAVE); the others only read and multiply.
  static constexpr int COPY_WAVES = COPY_WAVES_;
  static constexpr int FIRST_COPY_WAVE = WAVES - COPY_WAVES;
  static constexpr int COPIES = (BM + BN) / 8;         // 8-row copy instructions per stage
  static constexpr int COPIES_PER_WAVE = COPIES / COPY_WAVES;
  static constexpr int SA_WAVES = BM / 64;             // copy waves that also copy 64 row scales
  static constexpr int SB_WAVE = COPY_WAVES - 1;       // the copy wave that copies the B scales
  static constexpr int A_COPIES = BM / (8 * COPY_WAVES);  // copies per wave that move A rows
  static constexpr int COPIES_PER_SLICE = (COPIES_PER_WAVE + SPREAD - 1) / SPREAD;
  static_assert(COPY_WAVES >= 2 && COPY_WAVES <= WAVES, "copy waves");
  static_assert(COPIES % COPY_WAVES == 0, "copies must split evenly over the copy waves");
  static_assert((BM / 8) % COPY_WAVES == 0 && COPY_WAVES % 2 == 0,
                "A/B split and swizzle parity per copy wave");
  static_assert(SA_WAVES <= COPY_WAVES, "one copy wave per 64 row scales");
  static_assert(2 * (COPIES_PER_WAVE + 2) <= 63, "counted waits fit in vmcnt");

  static_assert(NB128 <= 4 && 128 % WN == 0, "B scales of a stage fit in 16 bytes");
  static_assert(LDS_BYTES + 4 * (3 * MAX_MASKED_GROUPS + 1) <= 160 * 1024, "LDS budget");
  static_assert(SPREAD >= 1 && SPREAD <= TN, "a stage's copies end before the next sync");
  static_assert(PF >= 1 && PF < TN, "B prefetch distance");
};

#ifndef LARGE_PBUF
#define LARGE_PBUF 1
#endif

// Copy issue: only the younger wave of each SIMD's pair copies (the SIMD
// favours the older wave's MFMAs, so the younger one has issue slots to
// spare), and a stage's copies are split over two slices so that no wave
// holds a long run of back-to-back copies.
#ifndef LARGE_SPREAD
#define LARGE_SPREAD 2
#endif
#ifndef MID_SPREAD
#define MID_SPREAD 2
#endif
#ifndef LARGE_COPY_WAVES
#define LARGE_COPY_WAVES 4
#endif
#ifndef MID_COPY_WAVES
#define MID_COPY_WAVES 4
#endif
#ifndef LARGE_PF
#define LARGE_PF 2
#endif
#ifndef MID_PF
#define MID_PF 2
#endif
#ifndef LARGE_GROUP_M
#define LARGE_GROUP_M 4
#endif
#ifndef LARGE_PRIO
#define LARGE_PRIO 1
#endif
#ifndef MID_PRIO
#define MID_PRIO 1
#endif
// dense / masked with large M: 8 waves of 64x128
using CfgLarge = Cfg<256, 256, 2, LARGE_GROUP_M, LARGE_PBUF, 64, 128, LARGE_SPREAD, LARGE_COPY_WAVES,
                     LARGE_PF, LARGE_PRIO>;
// 128-row blocks (contiguous experts, M <= 128): 8 waves of 64x64
using CfgMid = Cfg<128, 256, 3, 8, 2, 64, 64, MID_SPREAD, MID_COPY_WAVES, MID_PF, MID_PRIO>;


struct TileInfo {
  const uint8_t* a;      // first row of the tile's A rows
  const float* sa;       // scale of the tile's first row, K block 0
  const uint8_t* b;      // first row of the tile's B rows (expert applied)
  const float* sb;       // scale of the tile's first N block, K block 0
  uint16_t* d;           // first output row of the tile, column n0
  int mvalid;            // rows of the tile that exist (1..BM)
  int nvalid;            // columns of the tile that exist (multiple of 16, 16..BN)
  int kblocks;           // ceil(K / 128) (row length of the B scale array)
  int b_once;            // 1: no other tile reads this tile's B rows (an
                         // expert with one m-block), so its B copies stream
  int64_t row0, col0;    // the tile's first row and column in the output
};


// LDS swizzle of the 16-byte chunk index within a 128-byte row:
// chunk ^ (row & 7) ^ ((row >> 3) & 1). Any 8 consecutive rows then use 8
// distinct chunks (conflict-free for 8 lanes x 16 B on 32 banks), and so do
// the even rows and the odd rows of any 16 consecutive rows (conflict-free
// for 16 lanes x 16 B on 64 banks, where rows r and r+2 share banks).
FP8G_HD int swz(int row, int chunk) {
  return chunk ^ (row & 7) ^ ((row >> 3) & 1);
}

// Partial last K block (K mod 128 = kr bytes, a multiple of 16, exist): the
// chunks kr / 16 .. 7 of every row of a stage's A and B tiles (rows
// 0 .. BM + BN - 1, B after A; BM is a multiple of 16, so a B row's swizzle
// is the same counted from either tile's start) are zeroed before the step
// reads them. Item i of that list and its byte offset in the stage:
template <class C>
FP8G_HD int past_k_items(int kr) {
  return (C::BM + C::BN) * (8 - kr / 16);
}
template <class C>
FP8G_HD uint32_t past_k_offset(int i, int kr) {
  const int npast = 8 - kr / 16;
  const int row = i / npast, chunk = kr / 16 + i % npast;
  return (uint32_t)(row * BK + swz(row, chunk) * 16);
}

template <class C>
struct CopyPlan {
  uint32_t voff;       // per-lane offset of row0, chunk applied
  uint32_t sa_voff;    // per-lane offset of this lane's A row scale
  uint32_t sb_voff;    // per-lane offset of this lane's B block scale
  uint32_t dst0;       // LDS offset of this wave's first 8-row group
  uint32_t ch16;       // byte offset of this lane's source chunk
  int cw;              // copy wave index (negative: this wave issues no copies)
  int ragged;          // wave-uniform: clamp rows copy by copy
  int mvalid, nvalid;
};

template <class C>
FP8G_HD void make_plan_at(CopyPlan<C>& pl, const TileInfo& ti, int64_t K, int wave, int lane) {
  const int cw = wave - C::FIRST_COPY_WAVE;
  const int cwc = cw < 0 ? 0 : cw;   // (offsets of waves that copy nothing stay small)
  // swizzle: row & 7 = lane >> 3, and (row >> 3) & 1 = cw & 1 for every
  // group of this wave (COPY_WAVES is even)
  pl.ch16 = (uint32_t)((lane & 7) ^ (lane >> 3) ^ (cwc & 1)) * 16u;
  pl.voff = (uint32_t)(cwc * 8 + (lane >> 3)) * (uint32_t)K + pl.ch16;
  pl.ragged = (ti.mvalid < C::BM || ti.nvalid < C::BN) ? 1 : 0;
  pl.mvalid = ti.mvalid;
  pl.nvalid = ti.nvalid;
  const int ra = cwc * 64 + lane;
  pl.sa_voff = (uint32_t)(ra < ti.mvalid ? ra : ti.mvalid - 1) * 4u;
  const int nb = lane * 128 < ti.nvalid ? lane : (ti.nvalid + 127) / 128 - 1;
  pl.sb_voff = (uint32_t)nb * (uint32_t)ti.kblocks * 4u;
  pl.dst0 = (uint32_t)cwc * 8u * BK;
  pl.cw = cw;
}

// Source of copy i of a copy wave's share of one stage (K block kb): a
// wave-uniform base pointer and this lane's byte offset from it (what
// global_load_lds reads: 16 bytes at base + voff). A copies come first. On a
// full tile every copy uses the plan's one lane offset; on a ragged tile
// (pl.ragged) every row is clamped to the last row that exists. vsub as for
// issue_copies.
template <class C>
FP8G_HD void copy_source_full(const CopyPlan<C>& pl, const TileInfo& ti, int64_t K, int kb, int i,
                              uint32_t vsub, const uint8_t*& base, uint32_t& voff) {
  const int64_t step = (int64_t)C::COPY_WAVES * 8 * K;     // bytes between a wave's copies
  base = i < C::A_COPIES ? ti.a + (int64_t)kb * BK + i * step
                         : ti.b + (int64_t)kb * BK + (i - C::A_COPIES) * step;
  voff = pl.voff - vsub;
}
template <class C>
FP8G_HD void copy_source_ragged(const CopyPlan<C>& pl, const TileInfo& ti, int64_t K, int kb,
                                int i, int lane, uint32_t vsub, const uint8_t*& base,
                                uint32_t& voff) {
  const bool is_a = i < C::A_COPIES;
  const int r = pl.cw * 8 + (lane >> 3) + (is_a ? i : i - C::A_COPIES) * C::COPY_WAVES * 8;
  const int lim = (is_a ? pl.mvalid : pl.nvalid) - 1;
  base = (is_a ? ti.a : ti.b) + (int64_t)kb * BK;
  voff = (uint32_t)(r < lim ? r : lim) * (uint32_t)K + pl.ch16 - vsub;
}

// Tile order: slot -> (m-block, n-block) with group_m m-blocks per group.
FP8G_HD void swizzle_tile(int slot, int mblocks, int nblocks, int group_m,
                                             int& mb, int& nb) {
  const int per_group = group_m * nblocks;
  const int group = slot / per_group;
  const int first_m = group * group_m;
  const int gsize = imin(mblocks - first_m, group_m);
  const int in_group = slot - group * per_group;
  mb = first_m + in_group % gsize;
  nb = in_group / gsize;
}

// What the persistent loop needs to turn a tile slot into operand pointers.
struct Sched {
  int mblocks;        // m-blocks (masked: enumerated valid m-blocks of all experts)
  int nblocks;        // BN-wide column blocks
  int nblocks128;     // 128-wide column blocks (row length of the B scale layout)
  int tiles;
};

// m-blocks enumerated expert by expert (from device metadata in LDS): the
// masked layout, and the contiguous layout with 256-row tiles, whose
// expert boundaries (multiples of 128) need not fall on a 256-row grid.
template <class C, int MODE>
constexpr bool per_expert() {
  return MODE == MODE_MASKED || (MODE == MODE_CONTIGUOUS && C::BM > 128);
}

// Per-expert metadata in LDS, built once per workgroup: the clamped row
// count of each expert (masked: valid rows; contiguous: its padded rows),
// the experts in enumeration order (masked: decreasing count, ties by
// index; contiguous: expert order), and the m-blocks enumerated in that
// order (prefix[r] = m-blocks of the experts ranked before r).
struct MaskedMeta {
  int cnt[MAX_MASKED_GROUPS];
  int order[MAX_MASKED_GROUPS];
  int prefix[MAX_MASKED_GROUPS + 1];
};

// The tile slots of the workgroup whose first slot is `first`: one per round
// of `grid` slots. Dense and contiguous tiles all cost the same and take
// slot first + k * grid. Masked tiles are enumerated largest expert first,
// so their cost falls from round to round; odd rounds then run backwards
// (slot k * grid + grid - 1 - first), so that the workgroups that took the
// larger tiles of one round take the smaller ones of the next.
template <int MODE>
FP8G_HD int next_slot(int slot, int first, int grid) {
  if constexpr (MODE == MODE_MASKED) {
    const int k = slot / grid + 1;
    return k * grid + ((k & 1) ? grid - 1 - first : first);
  } else {
    return slot + grid;
  }
}
template <int MODE>
FP8G_HD int slot_count(int first, int grid, int tiles) {
  if constexpr (MODE == MODE_MASKED) {
    const int rounds = tiles / grid, rem = tiles - rounds * grid;
    const int x = (rounds & 1) ? grid - 1 - first : first;
    return rounds + (x < rem ? 1 : 0);
  } else {
    return first < tiles ? (tiles - first + grid - 1) / grid : 0;
  }
}

// Work slots: slot w < base is tile w over all of K; with splits > 1 the
// slots from base on are K pieces, slot base + t * splits + q covering K
// blocks [q * kpt, (q + 1) * kpt) of tile base + t.
struct SplitPlan {
  int base;
  int splits;
};
FP8G_HD bool is_piece(const SplitPlan& sp, int w) {
  return sp.splits > 1 && w >= sp.base;
}
FP8G_HD int work_tile(const SplitPlan& sp, int w) {
  return is_piece(sp, w) ? sp.base + (w - sp.base) / sp.splits : w;
}
FP8G_HD int work_k0(const SplitPlan& sp, int w, int kpt) {
  return is_piece(sp, w) ? ((w - sp.base) % sp.splits) * kpt : 0;
}
FP8G_HD int work_steps(const SplitPlan& sp, int w, int nkb, int kpt) {
  return is_piece(sp, w) ? kpt : nkb;
}

constexpr int MAX_SPLITS = 8;
// K pieces per leftover tile when the last round of `tiles` tiles on `grid`
// workgroups would be at most half full: the largest of 8, 4, 2 whose pieces
// fit that round and keep at least 4 K blocks each; 1 = no split.
FP8G_HD int choose_splits(int64_t tiles, int64_t grid, int64_t nkb) {
  const int64_t full = (tiles / grid) * grid, tail = tiles - full;
  if (full <= 0 || tail <= 0 || tail * 2 > grid) return 1;
  for (int sp = MAX_SPLITS; sp >= 2; sp >>= 1)
    if (tail * sp <= grid && nkb % sp == 0 && nkb / sp >= 4) return sp;
  return 1;
}

// slot -> tile: expert, first row, valid rows and columns, operand pointers.
// (N and K come from the kernel: compile-time constants in its
// shape-specialised instantiations)
template <class C, int MODE>
FP8G_HD void decode_tile(const GemmArgs& args, const MaskedMeta* meta,
                                            const Sched& sc, int slot, TileInfo& ti, int64_t N,
                                            int64_t K) {
  const int64_t kblocks = (K + BK - 1) / BK;     // (the last block may be partial)
  int mb, nb;
  // (masked: one expert's column blocks in a row, so that the workgroups of
  // an XCD running together share that expert's A rows in L2)
  swizzle_tile(slot, sc.mblocks, sc.nblocks, MODE == MODE_MASKED ? 1 : C::GROUP_M, mb, nb);
  int g = 0;
  int64_t row_start;
  // (metadata reads go through readfirstlane: every value here is
  // workgroup-uniform and belongs in scalar registers)
  ti.b_once = 0;
  if constexpr (MODE == MODE_DENSE || MODE == MODE_PERTENSOR) {
    row_start = (int64_t)mb * C::BM;
    ti.mvalid = (int)lmin((int64_t)C::BM, args.rows - row_start);
  } else if constexpr (MODE == MODE_CONTIGUOUS && !per_expert<C, MODE>()) {
    row_start = (int64_t)mb * C::BM;
    // expert g: the last g with offsets[g] <= row_start (binary search)
    int lo = 0, hi = args.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)uniform(args.group[mid]) <= row_start) lo = mid;
      else hi = mid - 1;
    }
    g = lo;
    ti.mvalid = (int)lmin((int64_t)C::BM, args.rows - row_start);
  } else {
    int lo = 0, hi = args.G - 1;       // the last rank r with prefix[r] <= mb
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uniform(meta->prefix[mid]) <= mb) lo = mid; else hi = mid - 1;
    }
    g = uniform(meta->order[lo]);
    const int local = mb - uniform(meta->prefix[lo]);
    const int m = uniform(meta->cnt[g]);
    int64_t base;                      // expert g's first row
    if constexpr (MODE == MODE_MASKED) {
      base = (int64_t)g * args.rows;
    } else {
      // (clamped into [0, rows] as when the counts were formed, so the
      // tile's rows stay inside [0, rows) whatever the offsets hold)
      const int64_t o = uniform(args.group[g]);
      base = o < 0 ? 0 : (o > args.rows ? args.rows : o);
    }
    row_start = base + (int64_t)local * C::BM;
    ti.mvalid = imin(C::BM, m - local * C::BM);
    ti.b_once = m <= C::BM ? 1 : 0;
  }
  const int64_t n0 = (int64_t)nb * C::BN;
  ti.nvalid = (int)lmin((int64_t)C::BN, N - n0);
  ti.a = args.a + row_start * K;
  ti.b = args.b + ((int64_t)g * N + n0) * K;
  if constexpr (MODE == MODE_PERTENSOR) {
    ti.sa = args.sa;                   // (one scale per operand: never copied per stage)
    ti.sb = args.sb;
  } else {
    ti.sa = args.sa + row_start;
    ti.sb = args.sb + ((int64_t)g * sc.nblocks128 + n0 / 128) * kblocks;
  }
  ti.kblocks = (int)kblocks;
  ti.row0 = row_start;
  ti.col0 = n0;
  ti.d = args.d + row_start * N + n0;
}

// MFMA row tiles of this wave that hold a row of the tile (wave-uniform):
// tile i covers rows (wm + i * WAVES_M) * 16 .. +15, so the tiles that hold
// rows are i < active_tiles, and a tile with u 16-row slices in use gives
// each row band ceil(u / 4) or floor(u / 4) of them.
template <class C>
FP8G_HD int active_tiles(const TileInfo& ti, int wm, int wn) {
  if (wn * C::WN >= ti.nvalid) return 0;
  const int u = (ti.mvalid + 15) >> 4;
  if (u <= wm) return 0;
  return imin(C::TM, (u - wm + C::WAVES_M - 1) / C::WAVES_M);
}

// ---------------------------------------------------------------------------
// Small-M (split-K) kernel: wave v of a workgroup takes K blocks
// [c0 + v kpw, c0 + (v + 1) kpw) of the chunk starting at block c0, and each
// lane loads, per block, two 16-byte halves of one A row and one B row at
// bytes kbyte = 32 (lane / 16) .. +31 of the block.
// Blocks of the chunk that belong to wave v (0..kpw).
FP8G_HD int smallm_count(int nkb, int c0, int wave, int kpw) {
  return imax(0, imin(kpw, nkb - (c0 + wave * kpw)));
}
struct SmallMSlot {
  int kb;          // K block loaded: the slot's, or the last one for a slot
                   // past the wave's blocks (loaded, not used)
  int64_t o0, o1;  // byte offsets from the operand row's start of the halves
  bool h0, h1;     // the half lies inside K; a half past K (ragged K only)
                   // reads the row's last 16 bytes, replaced by zeros
};
template <bool TAIL>
FP8G_HD SmallMSlot smallm_slot(int64_t K, int nkb, int kb0, int t, int kbyte) {
  SmallMSlot s;
  s.kb = imin(kb0 + t, nkb - 1);
  const int64_t ko = (int64_t)s.kb * BK + kbyte;
  s.h0 = !TAIL || ko < K;
  s.h1 = !TAIL || ko + 16 < K;
  s.o0 = s.h0 ? ko : K - 16;
  s.o1 = s.h1 ? ko + 16 : K - 16;
  return s;
}

// Workgroups of a persistent launch (one per CU, fewer if there are fewer
// tiles) and the most tiles the call can have (host side).
template <class C>
inline int64_t launch_grid(const GemmArgs& args, const DeviceInfo& dev, int64_t* tiles_out) {
  const int64_t nblocks = (args.N + C::BN - 1) / C::BN;
  // contiguous with 256-row tiles: each expert's rows (multiples of 128)
  // start a new block, so the count is at most rows / BM plus one per expert
  const bool expert_blocks = args.mode == MODE_CONTIGUOUS && C::BM > 128;
  int64_t mblocks_max;
  if (args.mode == MODE_MASKED)
    mblocks_max = (int64_t)args.G * ((args.rows + C::BM - 1) / C::BM);
  else if (expert_blocks)
    mblocks_max = args.rows / C::BM + args.G;
  else
    mblocks_max = (args.rows + C::BM - 1) / C::BM;
  *tiles_out = mblocks_max * nblocks;
  return *tiles_out < dev.cu_count ? *tiles_out : dev.cu_count;
}

}  // namespace gidx
}  // namespace fp8g
