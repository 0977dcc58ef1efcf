// Shared declarations of the gfx950 block-scaled GEMM library: tile configs,
// launcher signatures and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgg {

// ---------------------------------------------------------------- configs
struct TileCfg {
  int id;
  int block_m, block_n;
  int waves;
  int wg_per_cu;
  float tput;  // relative per-CU throughput of the shape (1.0 = best)
};

struct Fp8Args {
  const uint8_t* A;
  const uint8_t* B;
  const float* a_scale;
  const float* b_scale;
  const int32_t* m_indices;  // nullptr = every row is expert 0 (dense)
  uint16_t* C;
  int M, N, K, G;
};

struct Fp4Args {
  const uint8_t* A;        // [M, K/2]
  const uint8_t* B;        // [G, N, K/2]
  const uint8_t* a_scale;  // [M, K/16] E4M3
  const uint8_t* b_scale;  // [G, N, K/16] E4M3
  const int32_t* m_indices;  // nullptr = dense
  float alpha;
  const float* alphas;       // device [G] per-expert alpha, or nullptr (use alpha)
  uint16_t* C;
  int M, N, K, G;
};

// A batch of dense NVFP4 problems, passed to the kernel by value (kernel
// arguments: no device allocation, capturable in a graph).
constexpr int kMaxProblems = 32;
struct Fp4Problem {
  const uint8_t* A;        // [M, K/2]
  const uint8_t* B;        // [N, K/2]
  const uint8_t* a_scale;  // [M, K/16]
  const uint8_t* b_scale;  // [N, K/16]
  uint16_t* C;             // [M, N]
  int M, N, K;
  float alpha;
};
struct Fp4ProblemSet {
  Fp4Problem p[kMaxProblems];
  int tile_start[kMaxProblems + 1];  // filled by the launcher
  int count;
};

// A batch of dense block-scaled FP8 problems, passed by value likewise.
struct Fp8Problem {
  const uint8_t* A;        // [M, K] E4M3FN
  const uint8_t* B;        // [N, K] E4M3FN
  const float* a_scale;    // [M, K/128]
  const float* b_scale;    // [N/128, K/128]
  uint16_t* C;             // [M, N]
  int M, N, K;
};
struct Fp8ProblemSet {
  Fp8Problem p[kMaxProblems];
  int tile_start[kMaxProblems + 1];  // filled by the launcher
  int count;
};

// Number of compiled configs and their descriptions.
int fp8_num_tiles();
const TileCfg& fp8_tile(int id);
int fp4_num_tiles();
const TileCfg& fp4_tile(int id);

struct W4A16Args {
  const uint16_t* A;         // [M, K] BF16
  const uint8_t* B;          // [G, N, K/2] packed E2M1
  const uint8_t* b_scale;    // [G, N, K/16] E4M3
  const int32_t* m_indices;  // [M]
  float b_global;            // global scale of B
  uint16_t* C;               // [M, N] BF16
  int M, N, K, G;
};

// Launch choices made on the host.
struct LaunchOpts {
  int max_wg;     // > 0: cap on the persistent grid
  int num_cus;    // compute units of the device
  int run_split;  // 0 automatic, < 0 never, > 0 whenever possible (see split_items)
};

// Work items per tile.  A row window holding several experts' rows takes one
// K-loop pass per expert.  Normally one workgroup runs them one after the
// other; in split mode each pass is its own work item, so the passes of a
// window run side by side (the window-segment program of the flashinfer#7877
// page, "Code analysis 2": one CTA per expert run of a 128-row window, used
// when all of them fit in a single wave of the GPU).  The host cannot read
// m_indices, so a tile gets one item per expert: item r runs expert r's pass
// if the window holds a row of it and ends at once otherwise.  Knowing its
// expert from its index, an item can fetch that expert's B before the
// routing arrives.  Automatic mode splits only when every item of the
// launch runs at once on the device (tiles * G workgroups fit the CUs);
// then the launch lasts about one pass.
inline int split_items(int mode, bool grouped, int G, int BM, long long tiles, int slots) {
  (void)BM;
  if (!grouped || G < 2 || mode < 0) return 1;
  const long long s = G;
  if (tiles * s > 0x7FFFFFFFLL) return 1;
  if (mode == 0 && tiles * s > slots) return 1;
  return (int)s;
}

// Launchers: enqueue on `stream`, return hipSuccess or the launch error.
hipError_t launch_fp8(const Fp8Args& a, int tile_id, const LaunchOpts& o, hipStream_t s);
hipError_t launch_fp4(const Fp4Args& a, int tile_id, const LaunchOpts& o, hipStream_t s);
hipError_t launch_fp4_problems(const Fp4ProblemSet& set, int tile_id, const LaunchOpts& o,
                               hipStream_t s);
hipError_t launch_fp8_problems(const Fp8ProblemSet& set, int tile_id, const LaunchOpts& o,
                               hipStream_t s);
hipError_t launch_w4a16(const W4A16Args& a, hipStream_t s);
// rows (may be null): output row r quantises input row rows[r] of X's T
// rows, zeros when rows[r] is outside [0, T) (the MoE row expansion).
hipError_t launch_quant_fp8(const uint16_t* X, uint8_t* Q, float* scale, int M, int K,
                            int num_cus, hipStream_t s, const int32_t* rows = nullptr, int T = 0);
hipError_t launch_quant_nvfp4(const uint16_t* X, uint8_t* Q, uint8_t* S, float* g, int M, int K,
                              int num_cus, hipStream_t s);
hipError_t launch_quant_nvfp4_static(const uint16_t* X, uint8_t* Q, uint8_t* S, float g, int M,
                                     int K, int num_cus, hipStream_t s,
                                     const int32_t* rows = nullptr, int T = 0);

// --------------------------------------------------------- device helpers
#ifdef __HIPCC__
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Number of XCDs (each with its own L2) that the dispatcher deals
// workgroups to round-robin on MI355X.
constexpr int kXcds = 8;

// Work-tile order.  Workgroup ids are dealt to XCDs round-robin, so tile
// `slot * 8 + x` runs on XCD x.  Remap ids so that each XCD owns one
// contiguous range of logical tiles; inside a range, tiles go in groups of
// `group_w` row windows x all column tiles (row window fastest), so that
// workgroups resident on one XCD share A windows and B column tiles in
// that XCD's L2.  A bijection on [0, total).
__device__ __forceinline__ void map_tile(int id, int total, int num_windows, int num_ntiles,
                                         int group_w, int& window, int& ntile) {
  const int q = total / kXcds, r = total % kXcds;
  const int xcd = id % kXcds, slot = id / kXcds;
  const int logical = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
  const int per_group = group_w * num_ntiles;
  const int grp = logical / per_group;
  const int in = logical % per_group;
  const int first_w = grp * group_w;
  const int gw = min(group_w, num_windows - first_w);
  window = first_w + in % gw;
  ntile = in / gw;
}

// Heavy-first tile order.  A row window whose first and last rows hold two
// different valid experts needs (at least) two passes of the K loop, so its
// tiles cost up to twice as much.  With a static stride assignment of tiles
// to workgroups, a workgroup can draw two such tiles while others draw none,
// and the launch lasts as long as that workgroup.  Each workgroup therefore
// marks these windows (two reads of m_indices per window, into an LDS
// bitmask) and orders their tiles first: with at most gridDim.x of them,
// no workgroup gets two.  Each class keeps the XCD-aware order of map_tile;
// the heavy windows lie far apart in M (often under different experts), so
// their class goes one window at a time: the tiles an XCD runs together
// then share an A window instead of touching several windows and experts.
// Windows beyond kPlanWindows (large M: many tiles per workgroup, where the
// order matters little) are not planned.  Only the order depends on this
// estimate; which experts a tile processes is decided from all its rows.
constexpr int kPlanWindows = 4096;
constexpr int kPlanWords = kPlanWindows / 32;

// All threads of the workgroup call this; `bits` (kPlanWords words) and
// `count` are in LDS.  Ends with a barrier.
template <int BM, int THREADS>
__device__ __forceinline__ void build_plan(uint32_t* bits, int* count, const int32_t* m_indices,
                                           int M, int G, int num_windows) {
  const int tid = threadIdx.x;
  for (int w = tid; w < kPlanWords; w += THREADS) bits[w] = 0u;
  if (tid == 0) *count = 0;
  __syncthreads();
  if (m_indices != nullptr && num_windows <= kPlanWindows) {
    for (int w = tid; w < num_windows; w += THREADS) {
      const int r0 = w * BM;
      const int r1 = min(r0 + BM, M) - 1;
      const int a = m_indices[r0], b = m_indices[r1];
      if (a != b && a >= 0 && a < G && b >= 0 && b < G) {
        atomicOr(&bits[w >> 5], 1u << (w & 31));
        atomicAdd(count, 1);
      }
    }
  }
  __syncthreads();
}

// Index of the k-th window (from 0) whose bit equals `set`; k must be below
// the number of such windows.
__device__ __forceinline__ int nth_window(const uint32_t* bits, int num_windows, int k, bool set) {
  const int words = (num_windows + 31) >> 5;
  for (int wd = 0; wd < words; ++wd) {
    uint32_t v = set ? bits[wd] : ~bits[wd];
    const int left = num_windows - wd * 32;
    if (left < 32) v &= (1u << left) - 1u;
    const int c = __popc(v);
    if (k < c) {
      for (int i = 0; i < k; ++i) v &= v - 1u;
      return wd * 32 + __ffs(v) - 1;
    }
    k -= c;
  }
  return num_windows - 1;  // not reached for k below the count
}

// Tile `id` of the heavy-first order -> (row window, column tile).  A
// bijection on [0, num_windows * num_ntiles).
__device__ __forceinline__ void plan_tile(const uint32_t* bits, int heavy, int id, int num_windows,
                                          int num_ntiles, int group_w, int& window, int& ntile) {
  const int total = num_windows * num_ntiles;
  if (heavy <= 0) {
    map_tile(id, total, num_windows, num_ntiles, group_w, window, ntile);
    return;
  }
  const int th = heavy * num_ntiles;
  int cw;
  if (id < th) {
    map_tile(id, th, heavy, num_ntiles, 1, cw, ntile);
    window = nth_window(bits, num_windows, cw, true);
  } else {
    map_tile(id - th, total - th, num_windows - heavy, num_ntiles, group_w, cw, ntile);
    window = nth_window(bits, num_windows, cw, false);
  }
}

// Round four FP32 values to BF16 (round to nearest even) and pack them.
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  bf16x2 lo = __builtin_convertvector((f32x2){a, b}, bf16x2);
  bf16x2 hi = __builtin_convertvector((f32x2){c, d}, bf16x2);
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// ------------------------------------------------- direct-to-LDS staging
// Shared by the kernels that stage tiles with buffer loads straight into
// LDS and order them with explicit waits and barriers.
namespace lds_dma {

typedef __attribute__((address_space(3))) void* lds_ptr;

// Wait until at most N of this wave's vector-memory operations (including
// the loads into LDS) are outstanding; they complete in issue order, so a
// following barrier publishes the data of every earlier load.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier after this wave's LDS reads have completed.  Unlike
// __syncthreads() it does not also wait for every global load in flight
// (the look-ahead stages must stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A buffer offset past every buffer's end (buffers are below 2^31 bytes):
// a load there returns zeros without touching memory.
constexpr uint32_t kSkip = 0x80000000u;

// Raw buffer resource over [base, base + bytes), as its four descriptor
// words (base address, stride 0, size, raw-access flags).  The range check
// compares the instruction's VGPR offset (plus its immediate offset) with
// the size; the SGPR offset is added to the address after the check.  So a
// load whose VGPR offset lies past the end returns zeros without touching
// memory -- the out-of-range fill the tail tiles rely on -- and every caller
// keeps its SGPR offset to a displacement that cannot leave the row or
// block that an in-range VGPR offset points into.
__device__ __forceinline__ i32x4 rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return (i32x4){(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr)(const_cast<void*>(p));
}

// Direct global->LDS loads of 16 (or 4) bytes per lane at buffer offset
// voff + soff; lane l's bytes land at LDS address lds + 16 l (or 4 l).
// Inline assembly, so that the compiler does not track these LDS writes and
// add waits of its own for them: the pipeline orders them with its explicit
// vmcnt waits and barriers.
__device__ __forceinline__ void dma16(i32x4 rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds),
               "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(i32x4 rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(lds), "v"(voff),
               "s"(rs), "s"(soff)
               : "memory", "m0");
}

}  // namespace lds_dma

// Wave-wide minimum (64 lanes).
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  return v;
}
#endif

}  // namespace fgg
