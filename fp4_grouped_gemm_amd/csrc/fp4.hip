// NVFP4 (E2M1 values, E4M3 scale per 16 elements, FP32 global scales) dense
// and grouped GEMM for gfx950, BF16 output.
//
// What is computed (onnxruntime#29824 page, "Code analysis 1": W4A4 grouped
// GEMM for MoE prefill; flashinfer#3948 page: dense mm_fp4):
//   C[i, n] = alpha * sum_k (qA[i,k] sA[i,k/16]) (qB[g,n,k] sB[g,n,k/16]),
//   g = m_indices[i] (dense: g = 0), alpha = product of the global scales.
//
// Why FP16 MFMA and not the FP4 MFMA: gfx950's block-scaled MFMAs take one
// power-of-two (E8M0) scale per 32 elements, while NVFP4 carries a general
// E4M3 scale per 16 elements, and every FP4 MFMA spans at least 64 K
// elements, so the per-16 scales can neither ride in the instruction nor be
// applied to its output.  The product q * s of an E2M1 value and an E4M3
// scale has at most 6 significant bits and lies in [2^-10, 2688], so it is
// exact in FP16.  The kernel dequantises each element exactly once per
// workgroup while staging it into LDS (the dequantise-to-16-bit idea of the
// page's fallback runner, done here inside the GEMM), then runs
// v_mfma_f32_16x16x32_f16 with FP32 accumulation and multiplies by alpha in
// the epilogue.  Results match the exact NVFP4 product up to FP32 rounding.
//
// Work tiles, the in-window expert passes, padding rows and the XCD-aware
// order are as in the grouped FP8 kernel.  K step = 64 elements (32 packed
// bytes, 4 scale bytes per row); a tile row of 64 FP16 values is 128 bytes,
// stored as eight 16-byte chunks XOR-swizzled by row.
#include "common.h"

#include <climits>

namespace fgg {
namespace fp4_detail {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct Fp4Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int TM = WM / 16;
  static constexpr int TN = WN / 16;
  static constexpr int BK = 64;                 // K elements per step
  static constexpr int A_BYTES = BM * BK * 2;   // FP16 tile
  static constexpr int B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  // Each staging unit is 16 packed bytes = 32 elements = half a tile row.
  static constexpr int A_UNITS = BM * 2 / THREADS;
  static constexpr int B_UNITS = BN * 2 / THREADS;
  static_assert((BM * 2) % THREADS == 0 && (BN * 2) % THREADS == 0, "staging split");
  static_assert(BM % (16 * WAVES_M) == 0 && BN % (16 * WAVES_N) == 0, "tile shape");
};

__device__ __forceinline__ int swz(int r, int c) { return (r << 7) | ((c ^ (r & 7)) << 4); }

// E4M3FN code -> its value as FP16 (exact: 4 significant bits, 2^-9..448).
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t c) {
  const uint32_t E = (c >> 3) & 15u, M = c & 7u;
  float f = E ? __uint_as_float(((E + 120u) << 23) | (M << 20)) : (float)M * 0.001953125f;
  if (c & 0x80u) f = -f;
  return (_Float16)f;
}

// 16 packed bytes (32 E2M1 codes) and the two E4M3 scale codes of their
// 16-element blocks (bytes 0-7 -> scale0, bytes 8-15 -> scale1) -> 32 FP16
// values q * s in 4 x 16 bytes.  The hardware convert decodes two E2M1
// codes of one byte (scale 1.0, so it is exact whatever the convert does with
// a scale's mantissa); the multiply by the block scale is exact in FP16.
__device__ __forceinline__ void dequant32(const i32x4 packed, uint32_t sc, i32x4 out[4]) {
  const _Float16 s0 = e4m3_to_f16(sc & 0xFFu), s1 = e4m3_to_f16((sc >> 8) & 0xFFu);
  const f16x2 ss0 = {s0, s0}, ss1 = {s1, s1};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t word = (uint32_t)packed[w];
    const f16x2 ss = w < 2 ? ss0 : ss1;
    f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * ss;
    f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * ss;
    f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * ss;
    f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * ss;
    out[w] = (i32x4){__builtin_bit_cast(int, v0), __builtin_bit_cast(int, v1),
                     __builtin_bit_cast(int, v2), __builtin_bit_cast(int, v3)};
  }
}

// Fragment for v_mfma_f32_16x16x32_f16: lane l holds row (l % 16) and the
// 8 FP16 values of 16-byte chunk `kk * 4 + l / 16` of that row.  A and B use
// the same assignment, so every k is paired with itself.
__device__ __forceinline__ f16x8 read_frag(const uint8_t* tile, int row0, int lane, int kk) {
  const int r = row0 + (lane & 15);
  return *reinterpret_cast<const f16x8*>(tile + swz(r, kk * 4 + (lane >> 4)));
}

template <class T>
__global__ __launch_bounds__(T::THREADS) void fp4_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ a_scale, const uint8_t* __restrict__ b_scale,
    const int32_t* __restrict__ m_indices, float alpha, uint16_t* __restrict__ C, int M, int N,
    int K, int G, int num_windows, int num_ntiles, int total_tiles, int group_w) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * T::STAGE];
  __shared__ int ids[T::BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / T::WAVES_N;
  const int wn = wave % T::WAVES_N;
  const int nks = K / T::BK;
  const int Kp = K >> 1;   // packed bytes per row
  const int Ks = K >> 4;   // scale bytes per row
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  for (int tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    int window, ntile;
    map_tile(tile, total_tiles, num_windows, num_ntiles, group_w, window, ntile);
    const int row0 = window * T::BM;
    const int col0 = ntile * T::BN;

    __syncthreads();
    for (int r = tid; r < T::BM; r += T::THREADS) {
      const int gr = row0 + r;
      int e = -2;
      if (gr < M) {
        e = m_indices ? m_indices[gr] : 0;
        if (e < -1 || e >= G) e = -1;
      }
      ids[r] = e;
    }
    __syncthreads();

    for (int c = tid; c < T::BM * (T::BN / 8); c += T::THREADS) {
      const int r = c / (T::BN / 8);
      const int cc = c % (T::BN / 8);
      const int col = col0 + cc * 8;
      if (ids[r] == -1 && col < N)
        *reinterpret_cast<uint4*>(C + (size_t)(row0 + r) * N + col) = make_uint4(0, 0, 0, 0);
    }

    // Staging units of this thread: tile row and half (0: elements 0-31 of
    // the step, 1: 32-63).  Rows past the end are clamped (never stored).
    int a_row[T::A_UNITS], b_row[T::B_UNITS], a_half[T::A_UNITS], b_half[T::B_UNITS];
#pragma unroll
    for (int s = 0; s < T::A_UNITS; ++s) {
      const int u = tid + s * T::THREADS;
      a_row[s] = u >> 1;
      a_half[s] = u & 1;
    }
#pragma unroll
    for (int s = 0; s < T::B_UNITS; ++s) {
      const int u = tid + s * T::THREADS;
      b_row[s] = u >> 1;
      b_half[s] = u & 1;
    }
    const int last_a = M - 1 - row0, last_b = N - 1 - col0;

    int cur = -1;
    while (true) {
      int e = INT_MAX;
      for (int r = lane; r < T::BM; r += 64) {
        const int v = ids[r];
        if (v > cur && v < e) e = v;
      }
      e = wave_min(e);
      if (e == INT_MAX) break;
      cur = e;

      const uint8_t* Bg = B + (size_t)e * N * Kp;
      const uint8_t* Sg = b_scale + (size_t)e * N * Ks;
      const uint8_t* a_src[T::A_UNITS];
      const uint8_t* as_src[T::A_UNITS];
      const uint8_t* b_src[T::B_UNITS];
      const uint8_t* bs_src[T::B_UNITS];
#pragma unroll
      for (int s = 0; s < T::A_UNITS; ++s) {
        const size_t gr = (size_t)(row0 + min(a_row[s], last_a));
        a_src[s] = A + gr * Kp + a_half[s] * 16;
        as_src[s] = a_scale + gr * Ks + a_half[s] * 2;
      }
#pragma unroll
      for (int s = 0; s < T::B_UNITS; ++s) {
        const size_t gn = (size_t)(col0 + min(b_row[s], last_b));
        b_src[s] = Bg + gn * Kp + b_half[s] * 16;
        bs_src[s] = Sg + gn * Ks + b_half[s] * 2;
      }

      f32x4 acc[T::TM][T::TN];
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = zero;

      i32x4 ra[T::A_UNITS], rb[T::B_UNITS];
      uint32_t rsa[T::A_UNITS], rsb[T::B_UNITS];
#pragma unroll
      for (int s = 0; s < T::A_UNITS; ++s) {
        ra[s] = *reinterpret_cast<const i32x4*>(a_src[s]);
        rsa[s] = *reinterpret_cast<const uint16_t*>(as_src[s]);
      }
#pragma unroll
      for (int s = 0; s < T::B_UNITS; ++s) {
        rb[s] = *reinterpret_cast<const i32x4*>(b_src[s]);
        rsb[s] = *reinterpret_cast<const uint16_t*>(bs_src[s]);
      }
      // dequantise step 0 into stage 0
#pragma unroll
      for (int s = 0; s < T::A_UNITS; ++s) {
        i32x4 o[4];
        dequant32(ra[s], rsa[s], o);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<i32x4*>(smem + swz(a_row[s], a_half[s] * 4 + c)) = o[c];
      }
#pragma unroll
      for (int s = 0; s < T::B_UNITS; ++s) {
        i32x4 o[4];
        dequant32(rb[s], rsb[s], o);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<i32x4*>(smem + T::A_BYTES + swz(b_row[s], b_half[s] * 4 + c)) = o[c];
      }
      __syncthreads();

      for (int ks = 0; ks < nks; ++ks) {
        const bool more = ks + 1 < nks;
        if (more) {
          const int po = (ks + 1) * (T::BK / 2), so = (ks + 1) * (T::BK / 16);
#pragma unroll
          for (int s = 0; s < T::A_UNITS; ++s) {
            ra[s] = *reinterpret_cast<const i32x4*>(a_src[s] + po);
            rsa[s] = *reinterpret_cast<const uint16_t*>(as_src[s] + so);
          }
#pragma unroll
          for (int s = 0; s < T::B_UNITS; ++s) {
            rb[s] = *reinterpret_cast<const i32x4*>(b_src[s] + po);
            rsb[s] = *reinterpret_cast<const uint16_t*>(bs_src[s] + so);
          }
        }
        const uint8_t* sA = smem + (ks & 1) * T::STAGE;
        const uint8_t* sB = sA + T::A_BYTES;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          f16x8 af[T::TM];
#pragma unroll
          for (int i = 0; i < T::TM; ++i) af[i] = read_frag(sA, wm * T::WM + i * 16, lane, kk);
#pragma unroll
          for (int j = 0; j < T::TN; ++j) {
            const f16x8 bf = read_frag(sB, wn * T::WN + j * 16, lane, kk);
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[i], acc[i][j], 0, 0, 0);
          }
        }
        if (more) {
          uint8_t* nxt = smem + ((ks + 1) & 1) * T::STAGE;
#pragma unroll
          for (int s = 0; s < T::A_UNITS; ++s) {
            i32x4 o[4];
            dequant32(ra[s], rsa[s], o);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              *reinterpret_cast<i32x4*>(nxt + swz(a_row[s], a_half[s] * 4 + c)) = o[c];
          }
#pragma unroll
          for (int s = 0; s < T::B_UNITS; ++s) {
            i32x4 o[4];
            dequant32(rb[s], rsb[s], o);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              *reinterpret_cast<i32x4*>(nxt + T::A_BYTES + swz(b_row[s], b_half[s] * 4 + c)) = o[c];
          }
        }
        __syncthreads();
      }

      const int wcol0 = col0 + wn * T::WN;
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
                pack_bf16x4(alpha * acc[i][j][0], alpha * acc[i][j][1], alpha * acc[i][j][2],
                            alpha * acc[i][j][3]);
        }
      }
    }
  }
}

using Cfg0 = Fp4Cfg<256, 256, 4, 2>;  // 8 waves, 64x128 per wave, 128 KB LDS
using Cfg1 = Fp4Cfg<256, 128, 4, 1>;  // 4 waves, 64x128 per wave,  96 KB LDS
using Cfg2 = Fp4Cfg<128, 256, 2, 2>;  // 4 waves, 64x128 per wave,  96 KB LDS
using Cfg3 = Fp4Cfg<128, 128, 2, 2>;  // 4 waves, 64x64 per wave,   64 KB LDS

const TileCfg kFp4Tiles[] = {
    {0, 256, 256, 8, 1, 1.00f},
    {1, 256, 128, 4, 1, 0.90f},
    {2, 128, 256, 4, 1, 0.90f},
    {3, 128, 128, 4, 2, 0.80f},
};

template <class T>
hipError_t launch_cfg(const Fp4Args& a, int max_wg, int num_cus, hipStream_t s) {
  const int num_windows = (a.M + T::BM - 1) / T::BM;
  const int num_ntiles = (a.N + T::BN - 1) / T::BN;
  const long long total = (long long)num_windows * num_ntiles;
  if (total <= 0) return hipSuccess;
  if (total > INT_MAX) return hipErrorInvalidValue;
  int grid = (int)total;
  if (max_wg > 0 && max_wg < grid) grid = max_wg;
  const int per_xcd = (num_cus > 0 ? num_cus : 256) / kXcds;
  int group_w = per_xcd / (num_ntiles < 8 ? num_ntiles : 8);
  if (group_w < 1) group_w = 1;
  hipLaunchKernelGGL(fp4_gemm_kernel<T>, dim3(grid), dim3(T::THREADS), 0, s, a.A, a.B, a.a_scale,
                     a.b_scale, a.m_indices, a.alpha, a.C, a.M, a.N, a.K, a.G, num_windows,
                     num_ntiles, (int)total, group_w);
  return hipGetLastError();
}

}  // namespace fp4_detail

using namespace fp4_detail;

int fp4_num_tiles() { return (int)(sizeof(kFp4Tiles) / sizeof(kFp4Tiles[0])); }
const TileCfg& fp4_tile(int id) { return kFp4Tiles[id]; }

hipError_t launch_fp4(const Fp4Args& a, int tile_id, int max_wg, int num_cus, hipStream_t s) {
  switch (tile_id) {
    case 0: return launch_cfg<Cfg0>(a, max_wg, num_cus, s);
    case 1: return launch_cfg<Cfg1>(a, max_wg, num_cus, s);
    case 2: return launch_cfg<Cfg2>(a, max_wg, num_cus, s);
    case 3: return launch_cfg<Cfg3>(a, max_wg, num_cus, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fgg
