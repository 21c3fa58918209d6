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
//  * Workgroup tile 128x128, 4 waves in a 2x2 arrangement of 64x64 wave tiles
//    (4x4 MFMA tiles each, 64 fp32 accumulators per lane).
//  * Operand tiles are copied global -> LDS directly (no staging registers),
//    two LDS stages, the next K block's copies in flight while the current
//    one is multiplied.
//    LDS rows are 128 bytes (one K block of one row); the 16-byte chunk index
//    is XOR-swizzled with (row & 7) so that both the 16-byte writes and the
//    MFMA fragment reads of 8 consecutive lanes touch 8 distinct chunks.
//  * Persistent grid (about two workgroups per CU). Tile indices are first
//    remapped so that each XCD (workgroups are dealt round-robin to the 8
//    XCDs) walks a contiguous run of tiles, then grouped GROUP_M m-blocks at
//    a time (the tile swizzle of the gtnt Triton kernel) so that the tiles an
//    XCD runs together share A rows and B columns in its L2.
//  * Grouped layouts decode the tile index on the device from the group
//    metadata (offsets or valid counts), so the host never synchronises
//    (nxmr §3.2: each expert's work goes to its own workgroups, one launch).

#include "internal.h"

namespace fp8g {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 128;            // one scale block
constexpr int WAVES = 4;
constexpr int THREADS = WAVES * 64;
constexpr int WM = 64;             // wave tile rows
constexpr int WN = 64;             // wave tile columns
constexpr int TM = WM / 16;        // MFMA tiles per wave, M
constexpr int TN = WN / 16;        // MFMA tiles per wave, N
constexpr int GROUP_M = 8;
constexpr int SA_OFFSET = (BM + BN) * BK;          // A row scales of the K block
constexpr int STAGE_BYTES = SA_OFFSET + BM * 4;
constexpr int MAX_MASKED_GROUPS = 1024;

struct TileInfo {
  const uint8_t* a;      // first row of the tile's A rows
  const float* sa;       // scale of the tile's first row, K block 0
  const uint8_t* b;      // first row of the tile's B rows (expert applied)
  const float* sb;       // scale of the tile's N block, K block 0
  uint16_t* d;           // first output row of the tile, column n0
  int mvalid;            // rows of the tile that exist (1..BM)
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// float -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Global -> LDS copy of one K block of the A and B tiles and of the A row
// scales, straight into LDS (global_load_lds: each lane's 16 (or 4) bytes land
// at the wave-uniform LDS base + lane * size, no staging registers, and the
// copies are tracked by the vector-memory counter only, never mixed with
// register loads). One 16-byte instruction moves 8 rows x 128 bytes; lane l
// takes row base + (l >> 3) and, because its destination chunk is fixed to
// (l & 7), reads the logical chunk (l & 7) ^ (l >> 3), so that the LDS image
// is the XOR-swizzled layout. Wave w copies rows 32w .. 32w+31 of both tiles;
// wave 0 also copies the 128 row scales. Rows of A past mvalid are clamped to
// the last valid row: they are read (in bounds) but never stored.
__device__ __forceinline__ void issue_stage(const TileInfo& ti, int64_t K, int64_t sa_ld,
                                            int kb, uint8_t* stage) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunk = (lane & 7) ^ (lane >> 3);
  const int64_t koff = (int64_t)kb * BK + chunk * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rbase = wave * 32 + i * 8;
    const int r = rbase + (lane >> 3);
    const int ra = r < ti.mvalid ? r : ti.mvalid - 1;
    __builtin_amdgcn_global_load_lds(ti.a + (int64_t)ra * K + koff,
                                     (lds_ptr_t)(stage + rbase * BK), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(ti.b + (int64_t)r * K + koff,
                                     (lds_ptr_t)(stage + BM * BK + rbase * BK), 16, 0, 0);
  }
  if (wave == 0) {
    const float* sak = ti.sa + (int64_t)kb * sa_ld;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = h * 64 + lane;
      __builtin_amdgcn_global_load_lds(sak + (r < ti.mvalid ? r : ti.mvalid - 1),
                                       (lds_ptr_t)(stage + SA_OFFSET + h * 256), 4, 0, 0);
    }
  }
}

// MFMA operand fragment: lane l holds row (l & 15) of the 16-row slice
// starting at `row0`, bytes [(l >> 4) * 32, +32) of the K block. A and B use
// the same lane -> K assignment, so the product sums over the full block
// whatever order the hardware takes the K elements in.
__device__ __forceinline__ v8i load_frag(const uint8_t* tile, int row0, int lane) {
  const int r = row0 + (lane & 15);
  const int c0 = (lane >> 4) * 2;
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + r * BK + swz(r, c0) * 16);
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + r * BK + swz(r, c0 + 1) * 16);
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

__device__ void run_tile(const TileInfo& ti, int64_t N, int64_t K, int64_t sa_ld,
                         uint8_t* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1;          // 0..1
  const int wn = wave & 1;           // 0..1
  const int nkb = (int)(K / BK);
  const int rlane = wm * WM + (lane >> 4) * 4;   // first accumulator row of this lane

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  issue_stage(ti, K, sa_ld, 0, lds);

  for (int kb = 0; kb < nkb; ++kb) {
    uint8_t* cur = lds + (kb & 1) * STAGE_BYTES;
    // this K block's tile copies are the only loads in flight: wait for them
    // and make every wave's copies visible to every wave
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the other stage was last read before the barrier: refill it
    if (kb + 1 < nkb) issue_stage(ti, K, sa_ld, kb + 1, lds + ((kb + 1) & 1) * STAGE_BYTES);

    // block scales: one B scale per (tile, kb) (scalar load); the A row
    // scales of this K block sit in the stage next to the tiles
    const float sbv = ti.sb[kb];
    const float* sas = reinterpret_cast<const float*>(cur + SA_OFFSET);

    v8i bf[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = load_frag(cur + BM * BK, wn * WN + j * 16, lane);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const float4 sa4 = *reinterpret_cast<const float4*>(sas + rlane + i * 16);
      const float cs[4] = {sa4.x * sbv, sa4.y * sbv, sa4.z * sbv, sa4.w * sbv};
      const v8i af = load_frag(cur, wm * WM + i * 16, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(p[e], cs[e], acc[i][j][e]);
      }
    }
  }
  // all waves are done reading the last stage before the next tile reuses LDS
  __syncthreads();

  // epilogue: bf16 RNE, rows past mvalid are not written
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rlane + i * 16 + e;
      if (r < ti.mvalid) {
        uint16_t* drow = ti.d + (int64_t)r * N + wn * WN + (lane & 15);
#pragma unroll
        for (int j = 0; j < TN; ++j) drow[j * 16] = (uint16_t)bf16_rne(acc[i][j][e]);
      }
    }
  }
}

// Tile order: slot -> (m-block, n-block) with GROUP_M m-blocks per group.
__device__ __forceinline__ void swizzle_tile(int slot, int mblocks, int nblocks, int& mb,
                                             int& nb) {
  const int per_group = GROUP_M * nblocks;
  const int group = slot / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(mblocks - first_m, GROUP_M);
  const int in_group = slot - group * per_group;
  mb = first_m + in_group % gsize;
  nb = in_group / gsize;
}

__global__ void __launch_bounds__(THREADS, 2)
gemm_fp8_bs_kernel(GemmArgs args, int xcd_remap) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int prefix[MAX_MASKED_GROUPS + 1];

  const int64_t N = args.N;
  const int64_t K = args.K;
  const int nblocks = (int)(N / BN);
  const int64_t kblocks = K / BK;
  int mblocks;

  if (args.mode == MODE_MASKED) {
    // per-expert m-block counts -> prefix sums, computed by thread 0
    if (threadIdx.x == 0) {
      int acc = 0;
      prefix[0] = 0;
      for (int g = 0; g < args.G; ++g) {
        int m = args.group[g];
        m = m < 0 ? 0 : (m > args.rows ? (int)args.rows : m);
        acc += (m + BM - 1) / BM;
        prefix[g + 1] = acc;
      }
    }
    __syncthreads();
    mblocks = prefix[args.G];
  } else {
    mblocks = (int)((args.rows + BM - 1) / BM);
  }
  const int tiles = mblocks * nblocks;
  const int grid = gridDim.x;
  const int w = blockIdx.x;
  const int lane_slot = xcd_remap ? (w & 7) * (grid >> 3) + (w >> 3) : w;

  for (int base = 0;; base += grid) {
    const int slot = base + lane_slot;
    if (slot >= tiles) break;
    int mb, nb;
    swizzle_tile(slot, mblocks, nblocks, mb, nb);

    TileInfo ti;
    int g = 0;
    int64_t row_start;
    if (args.mode == MODE_DENSE) {
      row_start = (int64_t)mb * BM;
      ti.mvalid = (int)min((int64_t)BM, args.rows - row_start);
    } else if (args.mode == MODE_CONTIGUOUS) {
      row_start = (int64_t)mb * BM;
      // expert g: the last g with offsets[g] <= row_start (binary search)
      int lo = 0, hi = args.G - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if ((int64_t)args.group[mid] <= row_start) lo = mid; else hi = mid - 1;
      }
      g = lo;
      ti.mvalid = BM;
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
      row_start = (int64_t)g * args.rows + (int64_t)local * BM;
      ti.mvalid = min(BM, m - local * BM);
    }
    const int64_t n0 = (int64_t)nb * BN;
    ti.a = args.a + row_start * K;
    ti.sa = args.sa + row_start;
    ti.b = args.b + ((int64_t)g * N + n0) * K;
    ti.sb = args.sb + ((int64_t)g * nblocks + nb) * kblocks;
    ti.d = args.d + row_start * N + n0;
    run_tile(ti, N, K, args.sa_ld, lds);
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& args, const DeviceInfo& dev, int expected_m,
                       hipStream_t stream) {
  (void)expected_m;
  const int64_t nblocks = args.N / BN;
  int64_t mblocks_max;
  if (args.mode == MODE_MASKED)
    mblocks_max = (int64_t)args.G * ((args.rows + BM - 1) / BM);
  else
    mblocks_max = (args.rows + BM - 1) / BM;
  const int64_t tiles_max = mblocks_max * nblocks;
  if (tiles_max <= 0) return hipSuccess;
  int64_t grid = (int64_t)dev.cu_count * 2;
  if (grid > tiles_max) grid = tiles_max;
  const int remap = (grid % 8 == 0) ? 1 : 0;
  const size_t lds_bytes = 2 * STAGE_BYTES;
  hipLaunchKernelGGL(gemm_fp8_bs_kernel, dim3((unsigned)grid), dim3(THREADS), lds_bytes, stream,
                     args, remap);
  return hipGetLastError();
}

}  // namespace fp8g
