// Grouped block-scaled FP8 (E4M3FN) GEMM for gfx950, BF16 output.
//
// What is computed (flashinfer#7877 page, "Intro" and "Code analysis 1"):
// rows of A are routed to experts by m_indices; row i of C is
//   C[i, n] = sum_kb a_scale[i, kb] * b_scale[g, n/128, kb] * sum_{k in kb} A[i,k] B[g,n,k]
// with FP32 scales per 128-wide K block, FP32 accumulation and BF16 output;
// padding rows (m_indices = -1) are written as zeros.
//
// Design (gfx950-first; the page's TMA/warp-specialised design is prior art):
//  * Work tile = (row window of BM rows, column tile of BN columns).  A window
//    may hold several expert runs (a run can start or end inside it, the case
//    the page's window-segment program targets).  The workgroup finds the
//    experts present in its window on device -- m_indices is read on every
//    launch, never on the host -- and runs one pass of the K loop per
//    expert, storing only that expert's rows.  Padding rows are zero-filled.
//  * K step = 128 = one scale block.  Each step stages a BM x 128 A tile and
//    a BN x 128 B tile in LDS (two stages: the next step's global loads are
//    in flight while the current step computes), 16-byte coalesced loads, an
//    XOR swizzle of 16-byte chunks by row so fragment reads hit distinct
//    banks.
//  * One v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, unit E8M0 scales)
//    per 16x16 output tile per K step covers exactly one 128-K scale block,
//    giving a fresh FP32 partial that is promoted into the FP32 accumulator
//    with a_scale * b_scale (one FMA per output element per K block).
//  * The MFMA's first operand is the B tile (output columns) and its second
//    the A tile (output rows), so each lane ends up holding four consecutive
//    columns of one row: one 8-byte BF16 store per lane per 16x16 tile.
//  * Tiles are mapped to workgroups XCD-aware (see map_tile).  The grid is
//    min(tiles, cap); a workgroup loops over tiles with stride gridDim.x and
//    re-initialises all pipeline state (LDS stages, accumulators, expert
//    cursor) per tile and per pass.
#include "common.h"

#include <climits>

namespace fgg {
namespace fp8_detail {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct Fp8Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WM = BM / WAVES_M;  // rows per wave
  static constexpr int WN = BN / WAVES_N;  // columns per wave
  static constexpr int TM = WM / 16;       // 16-row subtiles per wave
  static constexpr int TN = WN / 16;       // 16-column subtiles per wave
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_BYTES = BN * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  // Direct global->LDS loads: one instruction moves 64 lanes x 16 bytes =
  // 8 tile rows; each wave issues A_LOADS + B_LOADS of them per K step.
  static constexpr int A_LOADS = BM / 8 / WAVES;
  static constexpr int B_LOADS = BN / 8 / WAVES;
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must share one b_scale block");
  static_assert(BM % (16 * WAVES_M) == 0 && BN % (16 * WAVES_N) == 0, "tile shape");
  static_assert(BM % (8 * WAVES) == 0 && BN % (8 * WAVES) == 0, "load split");
};

typedef __attribute__((address_space(3))) void* lds_ptr;

// LDS byte offset of 16-byte chunk `c` (0..7) of tile row `r`.
__device__ __forceinline__ int swz(int r, int c) { return (r << 7) | ((c ^ (r & 7)) << 4); }

// Fragment of 16 rows x 128 K bytes for v_mfma_*_16x16x128 with 8-bit
// operands: lane l holds row (l % 16) and K bytes [32 q, 32 q + 32), q = l / 16.
// The A and B operands use the same lane/K assignment, so the product sums
// over every k exactly once whatever order the hardware uses inside a lane.
__device__ __forceinline__ i32x8 read_frag(const uint8_t* tile, int row0, int lane) {
  const int r = row0 + (lane & 15);
  const int q = lane >> 4;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(tile + swz(r, 2 * q));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(tile + swz(r, 2 * q + 1));
  return (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Wait for this wave's outstanding vector-memory operations (including the
// direct-to-LDS loads), so that a following barrier publishes their data.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Stage the A and B tiles of K step `kb` into LDS stage `st` with direct
// global->LDS loads (no VGPR staging).
template <class T>
__device__ __forceinline__ void stage_in(uint8_t* st, const uint8_t* a_base, const uint8_t* b_base,
                                         const uint32_t (&a_off)[T::A_LOADS],
                                         const uint32_t (&b_off)[T::B_LOADS], int kb, int wave) {
  const uint8_t* ga = a_base + (kb << 7);
  const uint8_t* gb = b_base + (kb << 7);
#pragma unroll
  for (int s = 0; s < T::A_LOADS; ++s)
    __builtin_amdgcn_global_load_lds(ga + a_off[s], (lds_ptr)(st + (s * T::WAVES + wave) * 1024),
                                     16, 0, 0);
#pragma unroll
  for (int s = 0; s < T::B_LOADS; ++s)
    __builtin_amdgcn_global_load_lds(gb + b_off[s],
                                     (lds_ptr)(st + T::A_BYTES + (s * T::WAVES + wave) * 1024), 16,
                                     0, 0);
}

template <class T>
__global__ __launch_bounds__(T::THREADS) void fp8_grouped_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
    const float* __restrict__ a_scale, const float* __restrict__ b_scale,
    const int32_t* __restrict__ m_indices, uint16_t* __restrict__ C, int M, int N, int K, int G,
    int num_windows, int num_ntiles, int total_tiles, int group_w) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * T::STAGE];
  __shared__ int ids[T::BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / T::WAVES_N;
  const int wn = wave % T::WAVES_N;
  const int nkb = K >> 7;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  for (int tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    int window, ntile;
    map_tile(tile, total_tiles, num_windows, num_ntiles, group_w, window, ntile);
    const int row0 = window * T::BM;
    const int col0 = ntile * T::BN;

    __syncthreads();  // the previous tile is done with ids[] and smem
    for (int r = tid; r < T::BM; r += T::THREADS) {
      const int gr = row0 + r;
      int e = -2;  // past the end of A: never stored
      if (gr < M) {
        e = m_indices ? m_indices[gr] : 0;
        if (e < -1 || e >= G) e = -1;
      }
      ids[r] = e;
    }
    __syncthreads();

    // Padding rows of this window: zeros in this column tile.
    for (int c = tid; c < T::BM * (T::BN / 8); c += T::THREADS) {
      const int r = c / (T::BN / 8);
      const int cc = c % (T::BN / 8);
      const int col = col0 + cc * 8;
      if (ids[r] == -1 && col < N)
        *reinterpret_cast<uint4*>(C + (size_t)(row0 + r) * N + col) = make_uint4(0, 0, 0, 0);
    }

    // Per-lane byte offsets of the staged chunks inside the window / column
    // tile (rows past the end are clamped to the last row: they are loaded
    // but never stored).  Lane l of a load writes LDS bytes [16 l, 16 l + 16)
    // of its 1 KB block = tile row 8 b + l / 8, physical chunk l % 8, so it
    // fetches logical chunk (l % 8) ^ (row % 8) of that row.
    uint32_t a_off[T::A_LOADS], b_off[T::B_LOADS];
    const int last_a = M - 1 - row0, last_b = N - 1 - col0;
#pragma unroll
    for (int s = 0; s < T::A_LOADS; ++s) {
      const int r = (s * T::WAVES + wave) * 8 + (lane >> 3);
      a_off[s] = (uint32_t)min(r, last_a) * (uint32_t)K + (uint32_t)(((lane & 7) ^ (r & 7)) << 4);
    }
#pragma unroll
    for (int s = 0; s < T::B_LOADS; ++s) {
      const int r = (s * T::WAVES + wave) * 8 + (lane >> 3);
      b_off[s] = (uint32_t)min(r, last_b) * (uint32_t)K + (uint32_t)(((lane & 7) ^ (r & 7)) << 4);
    }

    // One pass per distinct expert present in the window, in increasing id.
    int cur = -1;
    while (true) {
      int e = INT_MAX;
      for (int r = lane; r < T::BM; r += 64) {
        const int v = ids[r];
        if (v > cur && v < e) e = v;
      }
      e = wave_min(e);  // identical in every wave: all take the same passes
      if (e == INT_MAX) break;
      cur = e;

      const uint8_t* a_base = A + (size_t)row0 * K;
      const uint8_t* b_base = B + ((size_t)e * N + col0) * K;
      // b_scale row of this wave's 128-column block (wave-uniform).
      const int wcol0 = col0 + wn * T::WN;
      const float* bs_row =
          b_scale + ((size_t)e * (N >> 7) + (min(wcol0, N - 1) >> 7)) * nkb;
      // a_scale rows of this lane (one per 16-row subtile).
      uint32_t as_off[T::TM];
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
        as_off[i] = (uint32_t)min(wm * T::WM + i * 16 + (lane & 15), last_a) * (uint32_t)nkb;
      const float* as_base = a_scale + (size_t)row0 * nkb;

      f32x4 acc[T::TM][T::TN];
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = zero;

      stage_in<T>(smem, a_base, b_base, a_off, b_off, 0, wave);
      float sa_next[T::TM];
#pragma unroll
      for (int i = 0; i < T::TM; ++i) sa_next[i] = as_base[as_off[i]];
      float sb_next = bs_row[0];
      wait_vmem();
      __syncthreads();

      for (int kb = 0; kb < nkb; ++kb) {
        const bool more = kb + 1 < nkb;
        float s[T::TM];
#pragma unroll
        for (int i = 0; i < T::TM; ++i) s[i] = sa_next[i] * sb_next;
        if (more) {
          stage_in<T>(smem + ((kb + 1) & 1) * T::STAGE, a_base, b_base, a_off, b_off, kb + 1, wave);
#pragma unroll
          for (int i = 0; i < T::TM; ++i) sa_next[i] = as_base[as_off[i] + kb + 1];
          sb_next = bs_row[kb + 1];
        }
        const uint8_t* sA = smem + (kb & 1) * T::STAGE;
        const uint8_t* sB = sA + T::A_BYTES;
        i32x8 af[T::TM];
#pragma unroll
        for (int i = 0; i < T::TM; ++i) af[i] = read_frag(sA, wm * T::WM + i * 16, lane);
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
          const i32x8 bf = read_frag(sB, wn * T::WN + j * 16, lane);
#pragma unroll
          for (int i = 0; i < T::TM; ++i) {
            const f32x4 p =
                __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], zero, 0, 0, 0, 127, 0, 127);
            acc[i][j] += p * s[i];
          }
        }
        wait_vmem();
        __syncthreads();
      }

      // Epilogue: this expert's rows only.  Lane holds C[m][n .. n+3].
#pragma unroll
      for (int i = 0; i < T::TM; ++i) {
        const int rl = wm * T::WM + i * 16 + (lane & 15);
        const int gr = row0 + rl;
        if (gr >= M || ids[rl] != e) continue;
        uint16_t* crow = C + (size_t)gr * N;
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
          const int n = wcol0 + j * 16 + 4 * (lane >> 4);
          if (n < N)
            *reinterpret_cast<uint2*>(crow + n) =
                pack_bf16x4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    }
  }
}

// Compiled tile shapes.  tput is the relative per-CU efficiency the ranker
// uses; wg_per_cu follows from LDS use (2 stages x (BM + BN) x 128 bytes).
using Cfg0 = Fp8Cfg<256, 256, 4, 2>;  // 8 waves, 64x128 per wave, 128 KB LDS
using Cfg1 = Fp8Cfg<256, 128, 4, 1>;  // 4 waves, 64x128 per wave,  96 KB LDS
using Cfg2 = Fp8Cfg<128, 256, 2, 2>;  // 4 waves, 64x128 per wave,  96 KB LDS
using Cfg3 = Fp8Cfg<128, 128, 2, 2>;  // 4 waves, 64x64 per wave,   64 KB LDS

const TileCfg kFp8Tiles[] = {
    {0, 256, 256, 8, 1, 1.00f},
    {1, 256, 128, 4, 1, 0.90f},
    {2, 128, 256, 4, 1, 0.90f},
    {3, 128, 128, 4, 2, 0.80f},
};

template <class T>
hipError_t launch_cfg(const Fp8Args& a, int max_wg, int num_cus, hipStream_t s) {
  const int num_windows = (a.M + T::BM - 1) / T::BM;
  const int num_ntiles = (a.N + T::BN - 1) / T::BN;
  const long long total = (long long)num_windows * num_ntiles;
  if (total <= 0) return hipSuccess;
  if (total > INT_MAX) return hipErrorInvalidValue;
  int grid = (int)total;
  if (max_wg > 0 && max_wg < grid) grid = max_wg;
  // Row windows per tile group: enough that one XCD's resident workgroups
  // cover a compact block of windows x column tiles.
  const int per_xcd = (num_cus > 0 ? num_cus : 256) / kXcds;
  int group_w = per_xcd / (num_ntiles < 8 ? num_ntiles : 8);
  if (group_w < 1) group_w = 1;
  hipLaunchKernelGGL(fp8_grouped_kernel<T>, dim3(grid), dim3(T::THREADS), 0, s, a.A, a.B,
                     a.a_scale, a.b_scale, a.m_indices, a.C, a.M, a.N, a.K, a.G, num_windows,
                     num_ntiles, (int)total, group_w);
  return hipGetLastError();
}

}  // namespace fp8_detail

using namespace fp8_detail;

int fp8_num_tiles() { return (int)(sizeof(kFp8Tiles) / sizeof(kFp8Tiles[0])); }
const TileCfg& fp8_tile(int id) { return kFp8Tiles[id]; }

hipError_t launch_fp8(const Fp8Args& a, int tile_id, int max_wg, int num_cus, hipStream_t s) {
  switch (tile_id) {
    case 0: return launch_cfg<Cfg0>(a, max_wg, num_cus, s);
    case 1: return launch_cfg<Cfg1>(a, max_wg, num_cus, s);
    case 2: return launch_cfg<Cfg2>(a, max_wg, num_cus, s);
    case 3: return launch_cfg<Cfg3>(a, max_wg, num_cus, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fgg
