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
  uint16_t* C;
  int M, N, K, G;
};

// Number of compiled configs and their descriptions.
int fp8_num_tiles();
const TileCfg& fp8_tile(int id);
int fp4_num_tiles();
const TileCfg& fp4_tile(int id);

// Launchers: enqueue on `stream`, return hipSuccess or the launch error.
hipError_t launch_fp8(const Fp8Args& a, int tile_id, int max_wg, int num_cus, hipStream_t s);
hipError_t launch_fp4(const Fp4Args& a, int tile_id, int max_wg, int num_cus, hipStream_t s);

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

// Round four FP32 values to BF16 (round to nearest even) and pack them.
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  bf16x2 lo = __builtin_convertvector((f32x2){a, b}, bf16x2);
  bf16x2 hi = __builtin_convertvector((f32x2){c, d}, bf16x2);
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Wave-wide minimum (64 lanes).
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  return v;
}
#endif

}  // namespace fgg
