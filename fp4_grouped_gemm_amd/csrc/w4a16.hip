// Grouped W4A16 GEMM for gfx950: BF16 activations times NVFP4 weights, BF16
// output -- the decode / small-M path.
//
// What is computed (onnxruntime#29824 page, "Code analysis 1": FP4 weights
// with 16-bit activations, dequantised, for decode and small-M shapes):
//   C[i, n] = gB * sum_k A[i, k] * qB[g, n, k] * sB[g, n, k / 16],
//   g = m_indices[i]; rows with g outside [0, G) are written as zeros.
//
// Design: with a few rows per expert the weights dominate the traffic (each
// weight byte is used by those few rows only), so the kernel streams B once
// from HBM at full width and keeps everything else on the side.
//  * One workgroup per (expert, 128-column block).  A workgroup first compacts the rows
//    routed to its expert into LDS (one wave, ballot + popcount, in row
//    order); a workgroup whose expert has no rows ends there and never reads
//    that expert's weights.  Rows are processed 32 at a time (two MFMA row
//    blocks sharing each dequantised weight fragment), each chunk streaming
//    the 64 columns' weights again.
//  * The four waves split K (128-wide groups, round robin).  Per group a lane
//    loads, for each of the 8 column blocks, 16 packed bytes (32 weights of
//    one column) and their two E4M3 scale codes, and 64 bytes of each of its
//    two activation rows (from L2: every workgroup of the expert reads the same
//    rows).  The next group's loads are in flight during this group's
//    dequantisation and MFMAs.
//  * Weights are dequantised exactly to BF16 in registers (q * s has at most
//    6 significant bits and lies in [2^-10, 2688]): the E2M1 pair convert with
//    scale 1.0, an FP32 multiply by the block scale, a pack to BF16.  Then
//    v_mfma_f32_16x16x32_bf16 with FP32 accumulation: lane (r, q) of the
//    activation operand and lane (c, q) of the weight operand hold the same
//    eight k, so every k pairs with itself.
//  * The four waves' partial sums meet in LDS and are added in wave order
//    (deterministic), times gB, rounded to BF16 and stored for the chunk's
//    rows.  The workgroups of expert 0 also write the zero rows (found in
//    the same scan).
#include "common.h"

#include <climits>

namespace fgg {
namespace w4a16_detail {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = 128;      // columns per workgroup: 8 MFMA column blocks
constexpr int kBlocks = kCols / 16;
static_assert(kCols == 2 * 64, "a zero row is one 4-byte store per lane");
constexpr int kRB = 2;          // MFMA row blocks per chunk
constexpr int kRows = 16 * kRB; // rows per chunk
constexpr int kGroup = 128;     // K per group: 4 MFMAs of K = 32
constexpr int kScan = 1024;     // m_indices entries compacted per scan

// One group's operands in registers.
struct Group {
  i32x4 a[kRB][4];           // activation rows of this lane: 32 BF16 at k0 + 32 q
  i32x4 b[kBlocks];          // packed weights: 32 E2M1 of column c at k0 + 32 q
  uint32_t s[kBlocks];       // two E4M3 scale codes of those 32 weights
};

__device__ __forceinline__ void load_group(Group& gr, const uint16_t* const arow[kRB],
                                           const uint8_t* bcol, const uint8_t* scol, int k0, int q,
                                           uint32_t Kp, uint32_t Ks) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const i32x4* ap = reinterpret_cast<const i32x4*>(arow[rb] + k0 + 32 * q);
#pragma unroll
    for (int u = 0; u < 4; ++u) gr.a[rb][u] = ap[u];
  }
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) {
    gr.b[b] = *reinterpret_cast<const i32x4*>(bcol + (size_t)b * 16 * Kp + (k0 + 32 * q) / 2);
    gr.s[b] = *reinterpret_cast<const uint16_t*>(scol + (size_t)b * 16 * Ks + (k0 + 32 * q) / 16);
  }
}

// Eight E2M1 codes (one 32-bit word, low nibble first) times the block
// scale s -> eight BF16 values.  Exact: at most 6 significant bits.
template <int H>
__device__ __forceinline__ void dequant2(uint32_t word, float s, bf16x8& r) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, H);  // byte H
  const bf16x2 p = __builtin_convertvector((f32x2){v[0] * s, v[1] * s}, bf16x2);
  r[2 * H] = p[0];
  r[2 * H + 1] = p[1];
}

__device__ __forceinline__ bf16x8 dequant8(uint32_t word, float s) {
  bf16x8 r;
  dequant2<0>(word, s, r);
  dequant2<1>(word, s, r);
  dequant2<2>(word, s, r);
  dequant2<3>(word, s, r);
  return r;
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

__device__ __forceinline__ void mma_group(const Group& gr, f32x4 acc[kRB][kBlocks], bool valid) {
  // MFMA j takes k0 + 32 q + 8 j .. + 8: 16-byte chunk j of the lane's 64
  // activation bytes and 32-bit word j of its 16 weight bytes; each
  // dequantised weight fragment serves every row block.
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) {
    const uint32_t sc = valid ? gr.s[b] : 0u;  // code 0 = scale 0
    const float s0 = e4m3_value(sc & 0xFFu), s1 = e4m3_value((sc >> 8) & 0xFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 bf = dequant8((uint32_t)gr.b[b][j], j < 2 ? s0 : s1);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        acc[rb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            bf, __builtin_bit_cast(bf16x8, gr.a[rb][j]), acc[rb][b], 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(kThreads) void w4a16_kernel(const uint16_t* __restrict__ A,
                                                         const uint8_t* __restrict__ B,
                                                         const uint8_t* __restrict__ b_scale,
                                                         const int32_t* __restrict__ m_indices,
                                                         float gb, uint16_t* __restrict__ C,
                                                         int M, int N, int K, int G) {
  __shared__ int rows[kScan];
  __shared__ int nrows;
  __shared__ f32x4 red[kWaves][kRB][kBlocks][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nblk = N / kCols;
  const int n0 = (blockIdx.x % nblk) * kCols;
  const int g = blockIdx.x / nblk;
  const uint32_t Kp = (uint32_t)K / 2, Ks = (uint32_t)K / 16;
  const int r = lane & 15, q = lane >> 4;

  // Weights of this workgroup: column n0 + 16 b + (lane % 16), from byte
  // (k0 + 32 q) / 2 of its row.
  const uint8_t* bcol = B + ((size_t)g * N + n0 + r) * Kp;
  const uint8_t* scol = b_scale + ((size_t)g * N + n0 + r) * Ks;
  const int ngroups = K / kGroup;

  for (int scan0 = 0; scan0 < M; scan0 += kScan) {
    // Compact the rows of this expert among m_indices[scan0, scan0 + kScan).
    __syncthreads();  // the previous chunks are done with rows[]
    if (wave == 0) {
      int count = 0;
      const int end = min(M, scan0 + kScan);
      for (int i0 = scan0; i0 < end; i0 += 64) {
        const int i = i0 + lane;
        const int e = i < end ? m_indices[i] : g;
        const bool hit = i < end && e == g;
        const uint64_t mask = __ballot(hit);
        if (hit) rows[count + __popcll(mask & ((1ull << lane) - 1ull))] = i;
        count += __popcll(mask);
        // Zero rows (padding or out-of-range ids): written by expert 0's
        // workgroups for their columns, one 256-byte row store per row.
        uint64_t bad = __ballot(g == 0 && (e < 0 || e >= G));
        while (bad) {
          const int b = __builtin_ctzll(bad);
          bad &= bad - 1;
          *reinterpret_cast<uint32_t*>(C + (size_t)(i0 + b) * N + n0 + 2 * lane) = 0u;
        }
      }
      if (lane == 0) nrows = count;
    }
    __syncthreads();
    const int count = nrows;

    for (int c0 = 0; c0 < count; c0 += kRows) {
      // Rows of this lane in the activation operands (row block rb: chunk
      // row 16 rb + l % 16); rows past the chunk read a valid row and are
      // never stored.
      const uint16_t* arow[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) arow[rb] = A + (size_t)rows[min(c0 + 16 * rb + r, count - 1)] * K;
      f32x4 acc[kRB][kBlocks];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) acc[rb][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

      // This wave's groups wave, wave + 4, ...: two register sets used in
      // turn, the next group's loads issued before this group's MFMAs.
      // Loads are unconditional (a group index past the end is clamped to
      // the last group and its data unused), so the waits count a fixed
      // number of loads; the fences keep each batch of loads ahead of the
      // MFMAs it overlaps.
      // Groups are taken in pairs with no early exit (an exit between a
      // load and its use lets the compiler sink the load past it): the
      // second group of the last pair may lie past the end, and then its
      // block scales are taken as 0, so it adds exact zeros (A is finite).
      Group g0, g1;
      const int last = ngroups - 1;
      load_group(g0, arow, bcol, scol, min(wave, last) * kGroup, q, Kp, Ks);
      for (int kg = wave; kg < ngroups; kg += 2 * kWaves) {
        load_group(g1, arow, bcol, scol, min(kg + kWaves, last) * kGroup, q, Kp, Ks);
        __builtin_amdgcn_sched_barrier(0);
        mma_group(g0, acc, true);
        load_group(g0, arow, bcol, scol, min(kg + 2 * kWaves, last) * kGroup, q, Kp, Ks);
        __builtin_amdgcn_sched_barrier(0);
        mma_group(g1, acc, kg + kWaves < ngroups);
      }

      // Sum the waves' partials in wave order; lane holds C[row c0 + 16 rb
      // + l % 16][n0 + 16 b + 4 (l / 16) + t].
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) red[wave][rb][b][lane] = acc[rb][b];
      __syncthreads();
      for (int b = wave; b < kBlocks; b += kWaves) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          f32x4 s = red[0][rb][b][lane];
#pragma unroll
          for (int w = 1; w < kWaves; ++w) s += red[w][rb][b][lane];
          const int m = c0 + 16 * rb + (lane & 15);
          if (m < count) {
            const int n = n0 + 16 * b + 4 * (lane >> 4);
            *reinterpret_cast<uint2*>(C + (size_t)rows[m] * N + n) =
                pack_bf16x4(gb * s[0], gb * s[1], gb * s[2], gb * s[3]);
          }
        }
      }
      __syncthreads();  // red[] is reused by the next chunk
    }
  }
}

}  // namespace w4a16_detail

using namespace w4a16_detail;

hipError_t launch_w4a16(const W4A16Args& a, hipStream_t s) {
  if (a.N % kCols || a.K % kGroup) return hipErrorInvalidValue;
  const long long grid = (long long)(a.N / kCols) * a.G;
  if (grid <= 0 || grid > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(w4a16_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a.A, a.B,
                     a.b_scale, a.m_indices, a.b_global, a.C, a.M, a.N, a.K, a.G);
  return hipGetLastError();
}

}  // namespace fgg
