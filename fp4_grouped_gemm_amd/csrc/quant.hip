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
// written per value.
#include "common.h"

#include <climits>

namespace fgg {
namespace quant_detail {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 8 BF16 values (16 bytes) -> FP32 (exact: BF16 is the top half of FP32).
__device__ __forceinline__ void bf16x8(u32x4 w, float v[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// 32 consecutive BF16 values (64 bytes) at p -> FP32: four 16-byte loads,
// all issued before any is used.
__device__ __forceinline__ void load32(const uint16_t* p, float v[4][8]) {
  u32x4 w[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) w[u] = *reinterpret_cast<const u32x4*>(p + 8 * u);
#pragma unroll
  for (int u = 0; u < 4; ++u) bf16x8(w[u], v[u]);
}

// Maximum over the lanes of aligned groups of `width` lanes (width <= 64).
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = 1; off < width; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// x / d rounded to nearest even -- the IEEE quotient -- from r = 1 / d (an
// IEEE division, once per block): q = x r, then two residual corrections
// q += fma(-d, q, x) r.  The first brings q within one ulp of x / d; from
// there, with r the correctly rounded reciprocal and no underflow or
// overflow, one correction gives the correctly rounded quotient (Markstein's
// theorem).  Callers take this path only when 2^-64 <= d <= 2^64 and every
// quotient is at most 2^64: the residuals of quotients above 2^-40 are then
// normal numbers; smaller quotients may come out a little off, but every
// value below 2^-11 encodes to zero in both formats, and the sign is taken
// from x (so -0 stays -0).  A multiply, four multiply-adds and a sign copy
// per value instead of the eleven-instruction division sequence, which had
// made these encoders ALU-bound.
__device__ __forceinline__ float div_rn(float x, float d, float r) {
  float q = x * r;
  q = fmaf(fmaf(-d, q, x), r, q);
  q = fmaf(fmaf(-d, q, x), r, q);
  return __builtin_copysignf(q, x);
}
// d and the block maximum a allow div_rn for every value of the block
__device__ __forceinline__ bool div_rn_ok(float d, float a) {
  return d >= 0x1p-64f && d <= 0x1p64f && a <= d * 0x1p64f;
}

// Both encoders give each lane 32 consecutive values (four 16-byte loads in
// flight per lane, whole 16-byte code stores) and a wave 2048; the 32-value
// pieces are independent of the rows, as blocks never cross a row.  Lanes
// past the end load the last piece instead and store nothing: a block is
// valid or not as a whole, so their values reach no valid block.
constexpr int kQThreads = 256;

// Where the values of an output row come from.  rows == nullptr: output row
// r is input row r (X read as a flat array).  Otherwise output row r is
// input row rows[r] of the T rows of X, and an entry outside [0, T) gives a
// row of zeros: the row expansion of an MoE layer, which copies each
// token's activations to the rows of the experts it is routed to (in expert
// order, with padding rows), fused with the quantisation of those rows
// (the onnxruntime#29824 page, "Code analysis 1": expandInputRowsKernel
// quantises while it expands).  Pieces are indexed in 32 bits (the host
// checks R * K / 32 < 2^31).
struct RowMap {
  const int32_t* rows;
  uint32_t ppr;  // 32-value pieces per row, K / 32
  int T;
};

__device__ __forceinline__ void load_piece(const uint16_t* X, long long q, const RowMap& m,
                                           float v[4][8]) {
  if (m.rows == nullptr) {
    load32(X + q * 32, v);
    return;
  }
  const uint32_t qq = (uint32_t)q;
  const uint32_t r = qq / m.ppr, c = qq - r * m.ppr;
  const int src = m.rows[r];
  if (src >= 0 && src < m.T) {
    load32(X + ((long long)src * m.ppr + c) * 32, v);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[u][i] = 0.f;
  }
}

// ------------------------------------------------------------- FP8 1x128
// A 128-value block is 4 lanes.
__global__ __launch_bounds__(kQThreads) void quant_fp8_kernel(const uint16_t* __restrict__ X,
                                                              uint8_t* __restrict__ Q,
                                                              float* __restrict__ scale,
                                                              long long nblocks, RowMap map) {
  const int lane = threadIdx.x & 63;
  const long long waves = (long long)gridDim.x * (kQThreads / 64);
  const long long pieces = nblocks * 4;
  for (long long w = (long long)blockIdx.x * (kQThreads / 64) + (threadIdx.x >> 6);
       w * 64 < pieces; w += waves) {
    const long long q = min(w * 64 + lane, pieces - 1);
    float v[4][8];
    load_piece(X, q, map, v);
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[u][i]));
    const float amax = group_max<4>(a);
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    float(&y)[4][8] = v;  // the quotients replace the values
    if (__builtin_expect(div_rn_ok(s, amax), 1)) {
      const float r = 1.0f / s;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) y[u][i] = div_rn(v[u][i], s, r);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) y[u][i] = v[u][i] / s;
    }
    u32x4 out[2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[u][i] = fminf(fmaxf(y[u][i], -448.0f), 448.0f);
      // bytes 0,1 then 2,3 of each word, in value order
      uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[u][0], y[u][1], 0, false);
      lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[u][2], y[u][3], (int)lo, true);
      uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[u][4], y[u][5], 0, false);
      hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[u][6], y[u][7], (int)hi, true);
      out[u >> 1][2 * (u & 1)] = lo;
      out[u >> 1][2 * (u & 1) + 1] = hi;
    }
    if (w * 64 + lane < pieces) {
      u32x4* o = reinterpret_cast<u32x4*>(Q + q * 32);
      o[0] = out[0];
      o[1] = out[1];
      if ((lane & 3) == 0) scale[q >> 2] = s;
    }
  }
}

// ------------------------------------------------------------------ NVFP4
// Global amax: max over |x| of the flat array, as the bit pattern of a
// non-negative float (ordered like the value) in amax_bits[0], which the
// first kernel clears.  X is read once here and once by the encoder, far
// apart, so these loads are non-temporal.
__global__ void clear_kernel(uint32_t* p) { p[0] = 0u; }

__global__ __launch_bounds__(kQThreads) void amax_kernel(const uint16_t* __restrict__ X,
                                                         long long n8, uint32_t* amax_bits) {
  constexpr int kLoads = 4;  // 16-byte loads in flight per lane
  float a = 0.f;
  const long long stride = (long long)gridDim.x * kQThreads * kLoads;
  for (long long i0 = (long long)blockIdx.x * kQThreads * kLoads + threadIdx.x; i0 < n8;
       i0 += stride) {
    // past the end: the last chunk again (a repeat cannot change the maximum)
    u32x4 w[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
      w[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(X + min(i0 + (long long)u * kQThreads, n8 - 1) * 8));
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      float v[8];
      bf16x8(w[u], v);
#pragma unroll
      for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(v[k]));
    }
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

// 8 quotients x / d -> 8 E2M1 codes (element 2j in the low nibble of byte j).
__device__ __forceinline__ uint32_t e2m1x8(const float y[8]) {
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const float y0 = fminf(fmaxf(y[i], -6.0f), 6.0f);
    const float y1 = fminf(fmaxf(y[i + 1], -6.0f), 6.0f);
    const uint32_t two =
        (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0, y0, y1, 1.0f, 0) & 0xFFu;
    packed |= two << (4 * i);
  }
  return packed;
}

// The 16 codes of a block (two words) from its values and decode scale d:
// all zero when d is 0.
__device__ __forceinline__ void e2m1_block(const float v0[8], const float v1[8], float d,
                                           float a, uint32_t& c0, uint32_t& c1) {
  c0 = c1 = 0;
  if (d > 0.f) {
    float y0[8], y1[8];
    if (__builtin_expect(div_rn_ok(d, a), 1)) {
      const float r = 1.0f / d;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        y0[i] = div_rn(v0[i], d, r);
        y1[i] = div_rn(v1[i], d, r);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        y0[i] = v0[i] / d;
        y1[i] = v1[i] / d;
      }
    }
    c0 = e2m1x8(y0);
    c1 = e2m1x8(y1);
  }
}

// A lane holds two whole 16-value blocks: no cross-lane reduction.
__global__ __launch_bounds__(kQThreads) void quant_nvfp4_kernel(const uint16_t* __restrict__ X,
                                                                uint8_t* __restrict__ Q,
                                                                uint8_t* __restrict__ S,
                                                                const uint32_t* amax_bits,
                                                                float g_given, long long nblocks,
                                                                RowMap map) {
  const int lane = threadIdx.x & 63;
  // the global scale: from the amax pass, or given by the caller (static)
  const float g = amax_bits ? global_scale(amax_bits[0]) : g_given;
  const float g6 = 6.0f * g;
  const long long waves = (long long)gridDim.x * (kQThreads / 64);
  const long long pieces = nblocks / 2;  // nblocks is even (K % 128 == 0)
  for (long long w = (long long)blockIdx.x * (kQThreads / 64) + (threadIdx.x >> 6);
       w * 64 < pieces; w += waves) {
    const long long q = min(w * 64 + lane, pieces - 1);
    float v[4][8];
    load_piece(X, q, map, v);
    u32x4 codes;
    uint32_t sc = 0;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float a = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[2 * b + h][i]));
      const float s_in = fminf(a / g6, 448.0f);
      const uint32_t s_code =
          (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s_in, 0.f, 0, false) & 0xFFu;
      const float d = __builtin_amdgcn_cvt_f32_fp8((int)s_code, 0) * g;
      uint32_t c0, c1;
      e2m1_block(v[2 * b], v[2 * b + 1], d, a, c0, c1);
      codes[2 * b] = c0;
      codes[2 * b + 1] = c1;
      sc |= s_code << (8 * b);
    }
    if (w * 64 + lane < pieces) {
      *reinterpret_cast<u32x4*>(Q + q * 16) = codes;
      S[q * 2] = (uint8_t)sc;  // byte stores: the scale array may have any alignment
      S[q * 2 + 1] = (uint8_t)(sc >> 8);
    }
  }
}

__global__ void finalize_kernel(uint32_t* g) {
  g[0] = __float_as_uint(global_scale(g[0]));
}

// Workgroups for `waves` waves of work, at most per_cu per compute unit
// (the rest loop); measured best: 8 per CU for the streaming loops here.
int grid_for(long long waves, int num_cus, int per_cu) {
  const long long wgs = (waves + kQThreads / 64 - 1) / (kQThreads / 64);
  const long long cap = (long long)num_cus * per_cu;
  return (int)(wgs < cap ? (wgs > 0 ? wgs : 1) : cap);
}

}  // namespace quant_detail

using namespace quant_detail;

hipError_t launch_quant_fp8(const uint16_t* X, uint8_t* Q, float* scale, int M, int K,
                            int num_cus, hipStream_t s, const int32_t* rows, int T) {
  const long long nblocks = (long long)M * (K / 128);
  if (nblocks <= 0) return hipSuccess;
  if (rows && nblocks * 4 > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const RowMap map{rows, (uint32_t)(K / 32), T};
  hipLaunchKernelGGL(quant_fp8_kernel, dim3(grid_for((nblocks * 4 + 63) / 64, num_cus, 8)),
                     dim3(kQThreads), 0, s, X, Q, scale, nblocks, map);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const uint16_t* X, uint8_t* Q, uint8_t* S, float* g, int M, int K,
                              int num_cus, hipStream_t s) {
  const long long n = (long long)M * K;
  if (n <= 0) return hipSuccess;
  uint32_t* gb = reinterpret_cast<uint32_t*>(g);
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(1), 0, s, gb);
  const long long n8 = n / 8;
  hipLaunchKernelGGL(amax_kernel, dim3(grid_for((n8 + 255) / 256, num_cus, 8)), dim3(kQThreads), 0,
                     s, X, n8, gb);
  const long long nblocks = n / 16;
  hipLaunchKernelGGL(quant_nvfp4_kernel, dim3(grid_for((nblocks / 2 + 63) / 64, num_cus, 16)),
                     dim3(kQThreads), 0, s, X, Q, S, (const uint32_t*)gb, 0.0f, nblocks,
                     RowMap{nullptr, (uint32_t)(K / 32), 0});
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1), 0, s, gb);
  return hipGetLastError();
}

// With a global scale given by the caller: the encode pass only (one read of X).
hipError_t launch_quant_nvfp4_static(const uint16_t* X, uint8_t* Q, uint8_t* S, float g, int M,
                                     int K, int num_cus, hipStream_t s, const int32_t* rows,
                                     int T) {
  const long long n = (long long)M * K;
  if (n <= 0) return hipSuccess;
  const long long nblocks = n / 16;
  if (rows && nblocks / 2 > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const RowMap map{rows, (uint32_t)(K / 32), T};
  hipLaunchKernelGGL(quant_nvfp4_kernel, dim3(grid_for((nblocks / 2 + 63) / 64, num_cus, 16)),
                     dim3(kQThreads), 0, s, X, Q, S, (const uint32_t*)nullptr, g, nblocks, map);
  return hipGetLastError();
}

}  // namespace fgg
