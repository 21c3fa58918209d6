// Host build of the persistent GEMM's index arithmetic (debug check).
//
// Compiles moe_grouped_gemm_quantizer_amd/csrc/gemm_index.h -- the same
// functions the kernel runs: tile scheduling (launch_grid, slot_count,
// next_slot, swizzle_tile, the split-tail work slots), tile decoding
// (decode_tile, including the per-expert enumeration of the grouped
// layouts) and the copy plan (make_plan_at, copy_source_full,
// copy_source_ragged) -- with a host compiler, enumerates every workgroup,
// tile, K block, copy wave, lane and copy of a launch, and checks:
//   * every 16-byte copy source lies inside its operand (A or B), every
//     scale copy inside its scale array, for full and ragged tiles and for
//     the partial last K block; every copy's LDS destination (1 KB per
//     wave-wide copy, 4 bytes per lane for scales) inside its tile's or
//     scales' region of the ring stage the K step uses;
//   * every element the epilogue stores lies inside D (and, masked, inside
//     its expert's valid rows), and every element of the output region is
//     stored exactly once -- or, for split-tail tiles, every K block of the
//     tile is covered exactly once by its pieces;
//   * every workgroup's slot walk terminates within the slots of the launch.
// The operands are never touched: their base pointers are fake addresses,
// and only the offsets the index arithmetic produces are compared with the
// buffer sizes. Prints the number of cases and violations; exit status 0
// only when there are none.
//
// Build: g++ -std=c++17 -O2 -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include
//        -I<pkg>/csrc gemm_index_check.cpp -o gemm_index_check

#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <cstdint>
#include <numeric>
#include <string>
#include <vector>

#include "gemm_index.h"

using namespace fp8g;
using namespace fp8g::gidx;

namespace {

long g_violations = 0;
long g_checks = 0;
long g_split_cases = 0;   // cases whose launch has a split tail

void fail(const std::string& what) {
  if (g_violations < 20) fprintf(stderr, "violation: %s\n", what.c_str());
  ++g_violations;
}

// Fake device addresses, far apart, so that an offset that strays into a
// neighbouring buffer is caught too.
const uintptr_t kA = 0x100000000000ull, kB = 0x200000000000ull, kSA = 0x300000000000ull,
                kSB = 0x400000000000ull, kD = 0x500000000000ull;

struct Case {
  std::string name;
  int mode;                  // GemmMode
  int64_t rows, N, K;        // rows: M, M_total or max_m
  int G;
  std::vector<int32_t> group;  // contiguous offsets [G+1] / masked counts [G]
  int expected_m;
  bool workspace;            // contiguous: a split-tail workspace is given
  bool large;                // 256-row configuration (else 128x256)
  int cus;
  // device metadata outside its contract (offsets not increasing, not
  // multiples of 128, negative or past the rows): the kernel clamps it, so
  // every access must still stay in bounds, but which rows are stored is
  // then unspecified -- only the bounds are checked
  bool bounds_only = false;
};

template <class C, int MODE>
void run_case(const Case& c) {
  const int64_t N = c.N, K = c.K;
  const int64_t KB = (K + BK - 1) / BK;
  const int64_t NB = (N + 127) / 128;
  const int G = (MODE == MODE_DENSE || MODE == MODE_PERTENSOR) ? 1 : c.G;
  // operand sizes (bytes / floats / elements)
  const int64_t a_rows = MODE == MODE_MASKED ? (int64_t)G * c.rows : c.rows;
  const int64_t b_rows = (int64_t)G * N;
  const int64_t a_bytes = a_rows * K, b_bytes = b_rows * K;
  const int64_t sa_count = KB * a_rows, sb_count = (int64_t)G * NB * KB;
  const int64_t d_elems = a_rows * N;

  GemmArgs args{reinterpret_cast<const uint8_t*>(kA), reinterpret_cast<const float*>(kSA),
                reinterpret_cast<const uint8_t*>(kB), reinterpret_cast<const float*>(kSB),
                reinterpret_cast<uint16_t*>(kD), c.group.empty() ? nullptr : c.group.data(),
                c.rows, a_rows, N, K, G, MODE};
  DeviceInfo dev{1, c.cus};

  // per-expert metadata, as the kernel's prologue builds it in LDS
  static MaskedMeta meta;
  Sched sc;
  sc.nblocks128 = (int)NB;
  sc.nblocks = (int)((N + C::BN - 1) / C::BN);
  if constexpr (per_expert<C, MODE>()) {
    for (int g = 0; g < G; ++g) {
      if constexpr (MODE == MODE_MASKED) {
        const int m = c.group[g];
        meta.cnt[g] = m < 0 ? 0 : (m > c.rows ? (int)c.rows : m);
      } else {
        int64_t lo = c.group[g], hi = c.group[g + 1];
        lo = std::min<int64_t>(std::max<int64_t>(lo, 0), c.rows);
        hi = std::min<int64_t>(std::max<int64_t>(hi, 0), c.rows);
        meta.cnt[g] = hi > lo ? (int)(hi - lo) : 0;
      }
      meta.order[g] = g;
    }
    if constexpr (MODE == MODE_MASKED)   // decreasing count, ties by index
      std::stable_sort(meta.order, meta.order + G,
                       [](int x, int y) { return meta.cnt[x] > meta.cnt[y]; });
    meta.prefix[0] = 0;
    for (int r = 0; r < G; ++r) meta.prefix[r + 1] = meta.prefix[r] + (meta.cnt[meta.order[r]] + C::BM - 1) / C::BM;
    sc.mblocks = meta.prefix[G];
  } else {
    sc.mblocks = (int)((c.rows + C::BM - 1) / C::BM);
  }
  sc.tiles = sc.mblocks * sc.nblocks;

  int64_t tiles_max;
  const int64_t grid64 = launch_grid<C>(args, dev, &tiles_max);
  if (tiles_max <= 0) return;
  if (sc.tiles > tiles_max && !c.bounds_only) fail(c.name + ": more tiles than launch_grid allows for");
  const int grid = (int)grid64;
  const int remap = (grid % 8 == 0) ? 1 : 0;
  const int nkb = (int)KB;
  // the split plan, as launch_cfg (host) and the kernel (device) form it
  SplitPlan spl{0, 1};
  if (MODE == MODE_CONTIGUOUS && c.workspace) {
    if (per_expert<C, MODE>()) {
      spl.splits = choose_splits(sc.tiles, grid, nkb);
      spl.base = spl.splits > 1 ? (sc.tiles / grid) * grid : 0;
    } else {
      spl.splits = choose_splits(tiles_max, grid, nkb);
      spl.base = (int)((tiles_max / grid) * grid);
    }
  }
  if (spl.splits > 1) ++g_split_cases;
  const int nwork = spl.splits > 1 ? spl.base + (sc.tiles - spl.base) * spl.splits : sc.tiles;
  const int kpt = nkb / spl.splits;
  const int kr = (int)(K % BK);

  std::vector<uint8_t> written(d_elems, 0);
  std::vector<uint8_t> kcover((size_t)sc.tiles * nkb, 0);

  for (int w = 0; w < grid; ++w) {
    const int first = remap ? (w & 7) * (grid >> 3) + (w >> 3) : w;
    const int nslots = slot_count<MODE>(first, grid, nwork);
    int slot = first;
    int step = 0;                 // the workgroup's K step counter (ring position)
    for (int k = 0; k < nslots; ++k, slot = next_slot<MODE>(slot, first, grid)) {
      if (slot < 0 || slot >= nwork) {
        fail(c.name + ": slot walk leaves the work list");
        break;
      }
      const int tile = work_tile(spl, slot);
      TileInfo ti;
      decode_tile<C, MODE>(args, &meta, sc, tile, ti, N, K);
      const int k0 = work_k0(spl, slot, kpt), steps = work_steps(spl, slot, nkb, kpt);
      for (int kb = k0; kb < k0 + steps; ++kb) ++kcover[(size_t)tile * nkb + kb];
      if (ti.mvalid <= 0 || ti.nvalid <= 0 || ti.nvalid % 16 != 0) {
        fail(c.name + ": tile with no rows or columns, or columns not a multiple of 16");
        continue;
      }
      // copies of every K step of the slot
      for (int kb = k0; kb < k0 + steps; ++kb, ++step) {
        for (int wave = C::FIRST_COPY_WAVE; wave < C::WAVES; ++wave) {
          for (int lane = 0; lane < 64; ++lane) {
            CopyPlan<C> pl;
            make_plan_at<C>(pl, ti, K, wave, lane);
            const uint32_t vsub = (kr != 0 && kb == nkb - 1 && (int)pl.ch16 >= kr) ? pl.ch16 : 0u;
            for (int i = 0; i < C::COPIES_PER_WAVE; ++i) {
              const uint8_t* base;
              uint32_t voff;
              if (!pl.ragged) copy_source_full<C>(pl, ti, K, kb, i, vsub, base, voff);
              else copy_source_ragged<C>(pl, ti, K, kb, i, lane, vsub, base, voff);
              const uintptr_t addr = reinterpret_cast<uintptr_t>(base) + voff;
              const bool is_a = i < C::A_COPIES;
              const uintptr_t lo = is_a ? kA : kB;
              const int64_t size = is_a ? a_bytes : b_bytes;
              ++g_checks;
              if (addr < lo || addr + 16 > lo + (uintptr_t)size)
                fail(c.name + ": " + (is_a ? "A" : "B") + " copy out of bounds");
              // LDS destination of the whole 64-lane copy (1 KB at dst), as
              // issue_copies forms it, inside its tile's region of the ring
              if (lane == 0) {
                const int stage = (step % C::STAGES) * C::STAGE_BYTES;
                const int dst = stage + (int)pl.dst0 + i * C::COPY_WAVES * 8 * BK;
                const int r0 = stage + (is_a ? 0 : C::BM * BK);
                const int r1 = r0 + (is_a ? C::BM : C::BN) * BK;
                if (dst < r0 || dst + 1024 > r1 || dst + 1024 > C::LDS_BYTES)
                  fail(c.name + ": LDS destination outside its tile");
              }
            }
            if (MODE != MODE_PERTENSOR) {
              const int cw = wave - C::FIRST_COPY_WAVE;
              if (cw < C::SA_WAVES) {
                const uintptr_t addr = reinterpret_cast<uintptr_t>(ti.sa + (int64_t)kb * args.sa_ld) + pl.sa_voff;
                if (addr < kSA || addr + 4 > kSA + (uintptr_t)sa_count * 4) fail(c.name + ": A scale copy out of bounds");
                const int sa0 = (step % C::STAGES) * C::STAGE_BYTES + C::SA_OFFSET;
                const int dst = sa0 + cw * 256 + lane * 4;
                if (dst + 4 > sa0 + C::BM * 4) fail(c.name + ": A scale LDS destination");
              }
              if (cw == C::SB_WAVE && lane < C::NB128) {
                const uintptr_t addr = reinterpret_cast<uintptr_t>(ti.sb + kb) + pl.sb_voff;
                if (addr < kSB || addr + 4 > kSB + (uintptr_t)sb_count * 4) fail(c.name + ": B scale copy out of bounds");
                const int sb0 = (step % C::STAGES) * C::STAGE_BYTES + C::SB_OFFSET;
                const int dst = sb0 + lane * 4;
                if (dst + 4 > sb0 + 16 || dst + 4 > C::LDS_BYTES) fail(c.name + ": B scale LDS destination");
              }
            }
          }
        }
      }
      if (is_piece(spl, slot)) {
        // pieces store fp32 partial tiles (summed by the reduction): the
        // workspace holds one round of grid partial tiles and grid records
        const int piece = slot - spl.base;
        if (piece < 0 || piece >= grid) fail(c.name + ": partial tile past the workspace");
        continue;
      }
      // the epilogue's stores (store_tile's guards)
      const int64_t tile_off = (int64_t)(reinterpret_cast<uintptr_t>(ti.d) - kD) / 2;
      for (int wave = 0; wave < C::WAVES; ++wave) {
        const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
        if (active_tiles<C>(ti, wm, wn) <= 0) continue;
        for (int i = 0; i < C::TM; ++i)
          for (int r16 = 0; r16 < 16; ++r16) {
            const int r = wm * 16 + r16 + i * C::RSTEP;
            if (r >= ti.mvalid) continue;
            for (int j = 0; j < C::TN; ++j) {
              if (wn * C::WN + j * 16 >= ti.nvalid) continue;
              for (int cc = 0; cc < 16; ++cc) {
                const int64_t e = tile_off + (int64_t)r * N + wn * C::WN + j * 16 + cc;
                if (e < 0 || e >= d_elems) { fail(c.name + ": store out of bounds"); continue; }
                ++written[e];
              }
            }
            // the quantising epilogue's scale store (dense, 128-column waves):
            // sd [ceil(N / 128)][rows], one per row and wave
            if (MODE == MODE_DENSE && C::WN == 128) {
              const int64_t cb = ti.col0 / 128 + wn;
              const int64_t s = cb * c.rows + ti.row0 + r;
              if (s < 0 || s >= NB * c.rows) fail(c.name + ": quantised scale store out of bounds");
            }
          }
      }
    }
  }
  if (c.bounds_only) return;
  // split tail: the pieces of a tile together cover each K block once
  for (int t = spl.splits > 1 ? spl.base : sc.tiles; t < sc.tiles; ++t)
    for (int kb = 0; kb < nkb; ++kb)
      if (kcover[(size_t)t * nkb + kb] != 1) { fail(c.name + ": a split tile's K block is not covered once"); t = sc.tiles; break; }
  // every output element of the region stored exactly once (split tiles
  // are stored by the reduction, which covers the recorded tiles' valid
  // rows and columns: counted here from their decoded extents)
  for (int t = spl.splits > 1 ? spl.base : sc.tiles; t < sc.tiles; ++t) {
    TileInfo ti;
    decode_tile<C, MODE>(args, &meta, sc, t, ti, N, K);
    const int64_t tile_off = (int64_t)(reinterpret_cast<uintptr_t>(ti.d) - kD) / 2;
    for (int r = 0; r < ti.mvalid; ++r)
      for (int cc = 0; cc < ti.nvalid; ++cc) {
        const int64_t e = tile_off + (int64_t)r * N + cc;
        if (e < 0 || e >= d_elems) { fail(c.name + ": reduction store out of bounds"); continue; }
        ++written[e];
      }
  }
  for (int64_t row = 0; row < a_rows; ++row) {
    bool expect = true;
    if (MODE == MODE_MASKED) {
      const int g = (int)(row / c.rows);
      expect = (row % c.rows) < meta.cnt[g];
    } else if (MODE == MODE_CONTIGUOUS) {
      expect = false;       // rows inside some expert's [offset, next offset)
      for (int g = 0; g < G; ++g)
        if (row >= std::max<int64_t>(0, c.group[g]) && row < std::min<int64_t>(c.rows, c.group[g + 1])) expect = true;
    }
    for (int64_t col = 0; col < N; ++col) {
      const uint8_t n = written[row * N + col];
      if (n != (expect ? 1 : 0)) {
        fail(c.name + ": output element stored " + std::to_string(n) + " times (row " +
             std::to_string(row) + ", col " + std::to_string(col) + ")");
        row = a_rows;
        break;
      }
    }
  }
}

template <int MODE>
void run_mode(const Case& c) {
  if (c.large) run_case<CfgLarge, MODE>(c);
  else run_case<CfgMid, MODE>(c);
}

void run(const Case& c) {
  switch (c.mode) {
    case MODE_DENSE: run_mode<MODE_DENSE>(c); break;
    case MODE_PERTENSOR: run_mode<MODE_PERTENSOR>(c); break;
    case MODE_CONTIGUOUS: run_mode<MODE_CONTIGUOUS>(c); break;
    default: run_mode<MODE_MASKED>(c); break;
  }
}

// Small-M (split-K) kernel, M <= 32: for every workgroup, chunk, wave, slot
// and lane, the two 16-byte halves it loads lie inside their A and B rows
// (rows inside the operands), the scale reads inside the scale arrays, and
// -- over the slots a wave uses -- every byte of K is loaded exactly once by
// a half kept as loaded, while every half replaced by zeros lies wholly
// past K. Where the kernel takes the wave's block count as the constant kpw
// (K fixed at compile time, a whole number of chunks), that count must be
// kpw for every wave.
long g_smallm_cases = 0;
template <bool TAIL>
void run_smallm_t(int64_t M, int64_t N, int64_t K, int mt_count, int kpw) {
  const std::string name = "small-M " + std::to_string(M) + "x" + std::to_string(N) + "x" +
                           std::to_string(K) + " MT" + std::to_string(mt_count) + " kpw" +
                           std::to_string(kpw);
  ++g_smallm_cases;
  const int nkb = (int)((K + BK - 1) / BK);
  const int64_t sa_len = (int64_t)nkb * M, sb_len = ((N + 127) / 128) * nkb;
  const bool whole = K % BK == 0 && nkb % (8 * kpw) == 0;
  for (int64_t wg = 0; wg < N / 16; ++wg) {
    const int64_t n0 = wg * 16;
    for (int g = 0; g < 4; ++g) {            // lanes 16 g .. 16 g + 15 share kbyte
      const int kbyte = 32 * g;
      std::vector<int> cover(wg == 0 ? K : 0, 0);
      for (int c0 = 0; c0 < nkb; c0 += 8 * kpw)
        for (int wave = 0; wave < 8; ++wave) {
          const int cnt = smallm_count(nkb, c0, wave, kpw);
          if (whole && cnt != kpw) fail(name + ": constant block count is wrong");
          if (cnt <= 0) continue;              // the wave loads nothing
          const int kb0 = c0 + wave * kpw;
          for (int t = 0; t < kpw; ++t) {
            const SmallMSlot sl = smallm_slot<TAIL>(K, nkb, kb0, t, kbyte);
            ++g_checks;
            if (sl.kb < 0 || sl.kb >= nkb) fail(name + ": K block out of range");
            for (int64_t o : {sl.o0, sl.o1})
              if (o < 0 || o + 16 > K) fail(name + ": fragment half outside its row");
            for (int r = 0; r < 16; ++r) {
              if (n0 + r >= N) fail(name + ": B row outside B");
              if ((n0 / 128) * nkb + sl.kb >= sb_len) fail(name + ": B scale outside sb");
              for (int mt = 0; mt < mt_count; ++mt) {
                const int64_t srow = std::min<int64_t>(mt * 16 + r, M - 1);
                if (srow < 0 || srow >= M) fail(name + ": A row outside A");
                if ((int64_t)sl.kb * M + srow >= sa_len) fail(name + ": A scale outside sa");
              }
            }
            if (wg != 0 || t >= cnt) continue;
            const int64_t nominal = (int64_t)sl.kb * BK + kbyte;
            const int64_t pos[2] = {nominal, nominal + 16};
            const bool kept[2] = {sl.h0, sl.h1};
            const int64_t off[2] = {sl.o0, sl.o1};
            for (int h = 0; h < 2; ++h) {
              if (kept[h]) {
                if (off[h] != pos[h]) fail(name + ": kept half not at its K position");
                for (int64_t k = off[h]; k < off[h] + 16 && k < K; ++k) ++cover[k];
              } else if (pos[h] < K) {
                fail(name + ": a half inside K replaced by zeros");
              }
            }
          }
        }
      if (wg == 0) {
        // the lanes of group g load bytes 32 g .. 32 g + 31 of each block
        for (int64_t k = 0; k < K; ++k) {
          const bool mine = (k % BK) / 32 == g;
          if (cover[k] != (mine ? 1 : 0)) {
            fail(name + ": K byte " + std::to_string(k) + " loaded " + std::to_string(cover[k]) +
                 " times");
            break;
          }
        }
      }
    }
  }
}
void run_smallm(int64_t M, int64_t N, int64_t K, int mt_count, int kpw) {
  if (K % BK != 0) run_smallm_t<true>(M, N, K, mt_count, kpw);
  else run_smallm_t<false>(M, N, K, mt_count, kpw);
}

// LDS layout of a stage (rows 0 .. BM + BN - 1, A then B, 128 bytes each):
//   * every copy lands the 16-byte chunk ch of its source row at slot
//     swz(row, ch) of that row of the stage -- where the fragment reads
//     (chunk c of row r at r * 128 + swz(r, c) * 16) look for it -- and the
//     row it lands in is the row it reads;
//   * the partial last K block's zeroing (kr = K mod 128 valid bytes)
//     writes each past-K chunk's slot of every row once, inside the A and B
//     tiles, and no slot of a chunk inside K.
template <class C>
void run_lds_layout(const char* cname) {
  TileInfo ti{};
  ti.mvalid = C::BM;
  ti.nvalid = C::BN;
  ti.kblocks = 8;
  for (int wave = C::FIRST_COPY_WAVE; wave < C::WAVES; ++wave)
    for (int lane = 0; lane < 64; ++lane) {
      CopyPlan<C> pl;
      make_plan_at<C>(pl, ti, 1024, wave, lane);
      for (int i = 0; i < C::COPIES_PER_WAVE; ++i) {
        ++g_checks;
        const uint32_t dst = pl.dst0 + (uint32_t)(i * C::COPY_WAVES * 8 * BK) + (uint32_t)lane * 16u;
        const int row = (int)(dst / BK), slot = (int)(dst % BK) / 16;
        const bool is_a = i < C::A_COPIES;
        const int src_row = pl.cw * 8 + (lane >> 3) + (is_a ? i : i - C::A_COPIES) * C::COPY_WAVES * 8;
        if ((is_a ? row : row - C::BM) != src_row)
          fail(std::string(cname) + ": a copy lands in another row than it reads");
        if (swz(row, (int)(pl.ch16 / 16)) != slot)
          fail(std::string(cname) + ": a copied chunk lands off its swizzled slot");
      }
    }
  for (int kr = 16; kr < BK; kr += 16) {
    std::vector<int> hits((C::BM + C::BN) * BK / 16, 0);
    for (int i = 0; i < past_k_items<C>(kr); ++i) {
      ++g_checks;
      const uint32_t off = past_k_offset<C>(i, kr);
      if (off % 16 != 0 || off >= (uint32_t)((C::BM + C::BN) * BK)) {
        fail(std::string(cname) + ": past-K zeroing outside the A and B tiles");
        continue;
      }
      ++hits[off / 16];
    }
    for (int row = 0; row < C::BM + C::BN; ++row)
      for (int c = 0; c < 8; ++c) {
        const int h = hits[(row * BK + swz(row, c) * 16) / 16];
        if (h != (c * 16 >= kr ? 1 : 0))
          fail(std::string(cname) + ": kr " + std::to_string(kr) + " row " + std::to_string(row) +
               " chunk " + std::to_string(c) + " zeroed " + std::to_string(h) + " times");
      }
  }
}

std::vector<int32_t> offsets_of(const std::vector<int>& counts) {
  std::vector<int32_t> off(1, 0);
  for (int cnt : counts) off.push_back(off.back() + (cnt + 127) / 128 * 128);
  return off;
}

}  // namespace

int main() {
  std::vector<Case> cases;
  // dense: the configuration the library picks (rows > 128: 256-row tiles),
  // aligned and ragged N and K, a grid smaller than the CU count
  const int64_t dense[][3] = {{4096, 8192, 8192}, {300, 144, 176}, {129, 400, 1040}, {513, 1040, 2064},
                              {257, 272, 16}, {100, 48, 400}, {64, 656, 8208}, {33, 128, 256},
                              {1, 16, 144}, {4096, 4096, 7168}};
  for (auto& s : dense)
    for (int mode : {MODE_DENSE, MODE_PERTENSOR})
      for (bool large : {true, false})
        cases.push_back({"dense " + std::to_string(s[0]) + "x" + std::to_string(s[1]) + "x" +
                             std::to_string(s[2]) + (large ? " L" : " M") +
                             (mode == MODE_PERTENSOR ? " pt" : ""),
                         mode, s[0], s[1], s[2], 1, {}, 0, false, large, 256});
  // contiguous: skewed counts, empty experts, a split tail, ragged shapes,
  // more experts than CUs
  const std::vector<std::vector<int>> cont = {{1796, 753, 466, 321, 255, 211, 161, 133},
                                              {9000, 4500, 2600, 2200}, {130, 0, 7, 256},
                                              {8, 8}, {0, 0, 300}, {1}, {500, 1, 0},
                                              {12000, 6000, 3000, 3000}};
  const int64_t cshapes[][2] = {{4096, 7168}, {1024, 2048}, {640, 1024}, {144, 400}, {48, 16}};
  for (size_t ci = 0; ci < cont.size(); ++ci)
    for (auto& s : cshapes)
      for (bool ws : {false, true})
        for (bool large : {true, false}) {
          auto off = offsets_of(cont[ci]);
          cases.push_back({"contiguous #" + std::to_string(ci) + " N" + std::to_string(s[0]) + " K" +
                               std::to_string(s[1]) + (ws ? " ws" : "") + (large ? " L" : " M"),
                           MODE_CONTIGUOUS, off.back(), s[0], s[1], (int)cont[ci].size(), off, 0,
                           ws, large, 256});
        }
  // masked: counts incl. 0, full, above max_m and negative (clamped)
  std::vector<int> mcounts(32);
  for (int g = 0; g < 32; ++g) mcounts[g] = (g * 97 + 13) % 257;
  mcounts[5] = 0;
  const std::vector<std::vector<int>> masked = {mcounts, {0, 1, 255, 256}, {3, 0, 77},
                                                {129, 128, 0, 200, 5}, {600, 0, 257, 513, 1, 16, 17, 255},
                                                {-5, 300, 40}};
  const int64_t mshapes[][3] = {{256, 7168, 2048}, {256, 256, 384}, {100, 144, 400}, {200, 48, 16},
                                {600, 512, 256}};
  for (size_t mi = 0; mi < masked.size(); ++mi)
    for (auto& s : mshapes)
      for (bool large : {true, false})
        cases.push_back({"masked #" + std::to_string(mi) + " max_m" + std::to_string(s[0]) + " N" +
                             std::to_string(s[1]) + " K" + std::to_string(s[2]) + (large ? " L" : " M"),
                         MODE_MASKED, s[0], s[1], s[2], (int)masked[mi].size(),
                         std::vector<int32_t>(masked[mi].begin(), masked[mi].end()), 0, false, large,
                         256});
  // contiguous offsets that break the layout's contract
  const std::vector<std::vector<int32_t>> bad = {{0, 4096, 0, 4096}, {300, 100, 5000, -7, 4096},
                                                 {-500, 77, 77, 9000}, {4096, 0}, {0, 129, 385, 4000}};
  for (size_t bi = 0; bi < bad.size(); ++bi)
    for (bool ws : {false, true})
      for (bool large : {true, false}) {
        Case c{"contiguous bad offsets #" + std::to_string(bi) + (ws ? " ws" : "") + (large ? " L" : " M"),
               MODE_CONTIGUOUS, 4096, 1024, 2048, (int)bad[bi].size() - 1, bad[bi], 0, ws, large, 256};
        c.bounds_only = true;
        cases.push_back(c);
      }
  // a GPU with fewer compute units (grids not a multiple of 8 included)
  cases.push_back({"dense 1000x1040x2064 on 100 CUs", MODE_DENSE, 1000, 1040, 2064, 1, {}, 0, false, true, 100});
  {
    auto off = offsets_of({9000, 4500, 2600, 2200});
    cases.push_back({"contiguous on 60 CUs ws", MODE_CONTIGUOUS, off.back(), 1024, 2048, 4, off, 0, true, true, 60});
  }
  cases.push_back({"masked on 36 CUs", MODE_MASKED, 256, 7168, 2048, 32,
                   std::vector<int32_t>(mcounts.begin(), mcounts.end()), 0, false, true, 36});

  for (auto& c : cases) run(c);
  run_lds_layout<CfgLarge>("256x256 stage");
  run_lds_layout<CfgMid>("128x256 stage");
  // small-M: the decode shapes, ragged K (multiples of 16), chunks that end
  // mid-wave and waves without blocks, for every instantiated (MT, kpw)
  const int64_t sm[][3] = {{16, 4096, 7168}, {32, 4096, 7168}, {1, 16, 16}, {5, 48, 7104},
                           {17, 144, 2064}, {32, 7168, 2048}, {16, 4096, 7168 - 64},
                           {3, 16, 128 * 57 + 48}, {8, 32, 4096}, {31, 64, 1040}};
  for (auto& s : sm)
    for (int mt_count : {1, 2})
      for (int kpw : {4, 7, 8})
        if (mt_count * 16 >= s[0]) run_smallm(s[0], s[1], s[2], mt_count, kpw);
  printf("cases %zu (split tail: %ld), small-M cases %ld, copy-lane checks %ld, violations %ld\n",
         cases.size(), g_split_cases, g_smallm_cases, g_checks, g_violations);
  return g_violations == 0 ? 0 : 1;
}
