// Activation quantisers for gfx950: BF16 -> FP8 E4M3FN with one FP32 scale
// per row and 128-wide K block, and BF16 -> NVFP4 (E2M1 codes, one E4M3
// scale per 16 elements, one FP32 global scale).  The step before the GEMM.
//
// What is computed (sglang#27745 page, "Code analysis 1: FP8 quantisation":
// clamp to +-448, the gfx950 E4M3FN maximum, then encode; the per-128 FP32
// block scales of the flashinfer#7877 page; the W4A4 layout of the
// onnxruntime#29824 page):
//   FP8    scale = amax(block) / 448 (1.0 for an all-zero block),
//          code  = E4M3FN_RNE(clamp(x / scale, +-448))
//   NVFP4  g = amax(X) / 2688 (1.0 for all-zero X),
//          s = E4M3FN_RNE(min(amax(block16) / (6 g), 448)), d = value(s) g,
//          code = E2M1_RNE(clamp(x / d, +-6)) (0 where d = 0),
//          element 2j in the low nibble of byte j.
// Every step that decides a code is an FP32 operation rounded to nearest
// even (IEEE division, not a reciprocal), so a code is a function of the
// input alone.  Codes come from the hardware pack converts (round to
// nearest even; the inputs are clamped first, so saturation never applies).
//
// Both kernels treat X as a flat array of M * K values: K is a multiple of
// 128, so no block crosses a row, and the scale arrays are the blocks in
// flat order.  They are HBM-bound: 2 bytes read and 1 (FP8) or 0.5 (NVFP4)
// written per value, 16-byte loads per lane.
#include "common.h"

#include <climits>

namespace fgg {
namespace quant_detail {

// 8 BF16 values (16 bytes) -> FP32 (exact: BF16 is the top half of FP32).
__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Maximum over the lanes of aligned groups of `width` lanes (width <= 64).
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = 1; off < width; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ------------------------------------------------------------- FP8 1x128
// One wave per 512 values (four 128-value blocks); lane l holds values
// [8 l, 8 l + 8) of the segment, block l / 16.
constexpr int kQThreads = 256;

__global__ __launch_bounds__(kQThreads) void quant_fp8_kernel(const uint16_t* __restrict__ X,
                                                              uint8_t* __restrict__ Q,
                                                              float* __restrict__ scale,
                                                              long long nblocks) {
  const int lane = threadIdx.x & 63;
  const long long waves = (long long)gridDim.x * (kQThreads / 64);
  for (long long seg = (long long)blockIdx.x * (kQThreads / 64) + (threadIdx.x >> 6);
       seg * 4 < nblocks; seg += waves) {
    const long long blk = seg * 4 + (lane >> 4);
    const bool valid = blk < nblocks;  // the last segment may hold fewer blocks
    const long long base = seg * 512 + lane * 8;
    float v[8];
    if (valid) {
      load8(X + base, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
    const float amax = group_max<16>(a);
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(v[i] / s, -448.0f), 448.0f);
    // bytes 0,1 then 2,3 of each word, in value order
    uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)lo, true);
    uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)hi, true);
    if (valid) {
      *reinterpret_cast<uint2*>(Q + base) = make_uint2(lo, hi);
      if ((lane & 15) == 0) scale[blk] = s;
    }
  }
}

// ------------------------------------------------------------------ NVFP4
// Global amax: max over |x| of the flat array, as the bit pattern of a
// non-negative float (ordered like the value) in amax_bits[0], which the
// first kernel clears.
__global__ void clear_kernel(uint32_t* p) { p[0] = 0u; }

__global__ __launch_bounds__(kQThreads) void amax_kernel(const uint16_t* __restrict__ X,
                                                         long long n8, uint32_t* amax_bits) {
  float a = 0.f;
  const long long stride = (long long)gridDim.x * kQThreads;
  for (long long i = (long long)blockIdx.x * kQThreads + threadIdx.x; i < n8; i += stride) {
    float v[8];
    load8(X + i * 8, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(v[k]));
  }
  a = group_max<64>(a);
  __shared__ float wmax[kQThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = wmax[0];
#pragma unroll
    for (int w = 1; w < kQThreads / 64; ++w) m = fmaxf(m, wmax[w]);
    atomicMax(amax_bits, __float_as_uint(m));
  }
}

__device__ __forceinline__ float global_scale(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits);
  return amax > 0.f ? amax / 2688.0f : 1.0f;
}

// One wave per 512 values (32 blocks of 16); lane l holds values
// [8 l, 8 l + 8), block l / 2.
__global__ __launch_bounds__(kQThreads) void quant_nvfp4_kernel(const uint16_t* __restrict__ X,
                                                                uint8_t* __restrict__ Q,
                                                                uint8_t* __restrict__ S,
                                                                const uint32_t* amax_bits,
                                                                long long nblocks) {
  const int lane = threadIdx.x & 63;
  const float g = global_scale(amax_bits[0]);
  const float g6 = 6.0f * g;
  const long long waves = (long long)gridDim.x * (kQThreads / 64);
  for (long long seg = (long long)blockIdx.x * (kQThreads / 64) + (threadIdx.x >> 6);
       seg * 32 < nblocks; seg += waves) {
    const long long blk = seg * 32 + (lane >> 1);
    const bool valid = blk < nblocks;
    const long long base = seg * 512 + lane * 8;
    float v[8];
    if (valid) {
      load8(X + base, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
    const float bamax = group_max<2>(a);
    const float s_in = fminf(bamax / g6, 448.0f);
    const uint32_t s_code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s_in, 0.f, 0, false) & 0xFFu;
    const float d = __builtin_amdgcn_cvt_f32_fp8((int)s_code, 0) * g;
    uint32_t packed = 0;
    if (d > 0.f) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float y0 = fminf(fmaxf(v[i] / d, -6.0f), 6.0f);
        const float y1 = fminf(fmaxf(v[i + 1] / d, -6.0f), 6.0f);
        const uint32_t two =
            (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0, y0, y1, 1.0f, 0) & 0xFFu;
        packed |= two << (4 * i);
      }
    }
    if (valid) {
      *reinterpret_cast<uint32_t*>(Q + base / 2) = packed;
      if ((lane & 1) == 0) S[blk] = (uint8_t)s_code;
    }
  }
}

__global__ void finalize_kernel(uint32_t* g) {
  g[0] = __float_as_uint(global_scale(g[0]));
}

int grid_for(long long waves, int num_cus) {
  const long long wgs = (waves + kQThreads / 64 - 1) / (kQThreads / 64);
  const long long cap = (long long)num_cus * 16;
  return (int)(wgs < cap ? (wgs > 0 ? wgs : 1) : cap);
}

}  // namespace quant_detail

using namespace quant_detail;

hipError_t launch_quant_fp8(const uint16_t* X, uint8_t* Q, float* scale, int M, int K,
                            int num_cus, hipStream_t s) {
  const long long nblocks = (long long)M * (K / 128);
  if (nblocks <= 0) return hipSuccess;
  const long long segs = (nblocks + 3) / 4;
  hipLaunchKernelGGL(quant_fp8_kernel, dim3(grid_for(segs, num_cus)), dim3(kQThreads), 0, s, X, Q,
                     scale, nblocks);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const uint16_t* X, uint8_t* Q, uint8_t* S, float* g, int M, int K,
                              int num_cus, hipStream_t s) {
  const long long n = (long long)M * K;
  if (n <= 0) return hipSuccess;
  uint32_t* gb = reinterpret_cast<uint32_t*>(g);
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(1), 0, s, gb);
  const long long n8 = n / 8;
  hipLaunchKernelGGL(amax_kernel, dim3(grid_for(n8 / 64 + 1, num_cus)), dim3(kQThreads), 0, s, X,
                     n8, gb);
  const long long nblocks = n / 16;
  const long long segs = (nblocks + 31) / 32;
  hipLaunchKernelGGL(quant_nvfp4_kernel, dim3(grid_for(segs, num_cus)), dim3(kQThreads), 0, s, X,
                     Q, S, (const uint32_t*)gb, nblocks);
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1), 0, s, gb);
  return hipGetLastError();
}

}  // namespace fgg
