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
// from HBM with many loads in flight and keeps the dequantisation VALU work
// of one wave overlapped with the load waits of the others.
//  * One workgroup (4 waves) per (expert, 128-column block); wave w owns
//    columns 32 w .. 32 w + 31 (two MFMA column blocks) over all of K, so
//    no partial sums cross waves.  Wave 0 first compacts the rows routed to
//    the expert into LDS (ballot + popcount, in row order; expert 0's
//    workgroups also zero the padding rows found); a workgroup whose expert
//    has no rows stops there and never reads that expert's weights.
//  * Rows run 32 at a time (two MFMA row blocks sharing each dequantised
//    weight fragment).  Their activations, 32 rows x 256 K per group, go
//    through a 4-stage LDS ring with direct-to-LDS loads (no registers),
//    shared by the four waves; 16-byte chunks are XOR-swizzled by row so a
//    fragment read hits 16 distinct chunk positions.
//  * Weights stream through a 4-slot register ring, 3 groups ahead: per
//    group a lane loads 32 packed bytes (64 weights of one column) and their
//    four E4M3 scale codes per column block.  Every group issues the same
//    loads (past the last group they reload it and add exact zeros through
//    a zero scale), so one explicit count waits for the oldest group.
//  * Weights are dequantised exactly to BF16 in registers (q * s has at most
//    6 significant bits and lies in [2^-10, 2688]): the E2M1 pair convert with
//    scale 1.0, an FP32 multiply by the block scale, and the upper halves of
//    two exact products packed as a BF16 pair (no rounding needed).  Then
//    v_mfma_f32_16x16x32_bf16 with FP32 accumulation: lane (r, q) of the
//    activation operand and lane (c, q) of the weight operand hold the same
//    eight k, so every k pairs with itself.
#include "common.h"

#include <climits>
#include <utility>

namespace fgg {
namespace w4a16_detail {

using namespace lds_dma;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kCB = 2;                 // MFMA column blocks per wave
constexpr int kCols = 16 * kCB * kWaves;  // columns per workgroup
constexpr int kRB = 2;                 // MFMA row blocks per chunk
constexpr int kRows = 16 * kRB;        // rows per chunk
constexpr int kGroup = 256;            // K per group: 8 MFMAs of K = 32
constexpr int kWords = kGroup / 32;    // 32-bit words of packed weights per lane per group
constexpr int kChunks = kGroup / 8;    // 16-byte activation chunks per row per group
constexpr int kScan = 1024;            // m_indices entries compacted per scan
constexpr int kAStages = 4;            // LDS ring of activation groups
constexpr int kBSlots = 4;             // register ring of weight groups
constexpr int kAhead = kBSlots - 1;    // weight groups issued ahead
constexpr int kAStage = kRows * kGroup * 2;         // bytes per activation stage
constexpr int kADma = kAStage / 16 / kThreads;      // 16-byte loads per thread
static_assert(kCols == 2 * 64, "a zero row is one 4-byte store per lane");
static_assert(kBSlots % kAStages == 0, "an unrolled block of kBSlots groups starts at stage 0");
static_assert(kADma * 16 * kThreads == kAStage, "activation staging split");
// Loads per group per wave: activation DMAs, then per column block the
// weight bytes (16 bytes per load) and the scale codes.
constexpr int kLoadsPerGroup = kADma + kCB * (kWords / 4 + 1);
// Step i issues the activations of group i + kAStages - 1, then the weights
// of group i + kAhead.  So group i's weights go out kLead steps before its
// activations (or right after them, kLead = 0), and when step i waits, the
// later of the two is followed by the weights of its own step (kLead > 0)
// and by the kAStages - 2 steps in between.
constexpr int kLead = kAhead - kAStages + 1;
static_assert(kLead >= 0, "weights must not trail their activations");
constexpr int kWaitAfter =
    (kLead > 0 ? kCB * (kWords / 4 + 1) : 0) + (kAStages - 2) * kLoadsPerGroup;

struct Weights {
  i32x4 b[kCB][kWords / 4];  // 64 E2M1 codes of column c at k0 + 64 q
  uint32_t s[kCB];           // their four E4M3 scale codes
};

// The two codes of byte H times s, as a BF16 pair.  q * s has at most 6
// significant bits, so its FP32 value carries no bits below the top 16 and
// BF16 is that upper half exactly: a byte permute takes the upper halves of
// the two products (no rounding convert, which issues at a quarter of the
// multiply rate).  A NaN scale code gives the quiet NaN 0x7FC00000, whose
// upper half is a BF16 NaN.
template <int H>
__device__ __forceinline__ void dequant2(uint32_t word, float s, bf16x8& r) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, H);  // byte H
  const uint32_t lo = __builtin_bit_cast(uint32_t, v[0] * s);
  const uint32_t hi = __builtin_bit_cast(uint32_t, v[1] * s);
  const bf16x2 p = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(hi, lo, 0x07060302u));
  r[2 * H] = p[0];
  r[2 * H + 1] = p[1];
}

// Eight E2M1 codes (one 32-bit word, low nibble first) times the block
// scale s -> eight BF16 values.  Exact: at most 6 significant bits.
__device__ __forceinline__ bf16x8 dequant8(uint32_t word, float s) {
  bf16x8 r;
  dequant2<0>(word, s, r);
  dequant2<1>(word, s, r);
  dequant2<2>(word, s, r);
  dequant2<3>(word, s, r);
  return r;
}

// LDS byte offset of 16-byte chunk c (0..31) of activation row r (0..31).
__device__ __forceinline__ int a_swz(int r, int c) { return r * (kGroup * 2) + ((c ^ r) << 4); }
static_assert(kChunks == kRows, "the chunk swizzle uses the row's 5 bits");

struct Ctx {
  const uint8_t* bcol[kCB];   // weight row of this lane's column, per column block
  const uint8_t* scol[kCB];   // its scale codes
  i32x4 ra;                   // activation buffer resource (whole A)
  uint32_t a_off[kADma];      // this lane's activation chunks: row offset + chunk
  uint32_t lds_a[kADma];      // their LDS destinations (stage 0)
  int ngroups;
  int K;
  int q;
};

// Issue group g's activation chunks into LDS stage g % kAStages (group index
// clamped to the last one past the end).
__device__ __forceinline__ void load_a(const Ctx& c, uint8_t* ring, int g) {
  const int gc = min(g, c.ngroups - 1);
  const uint32_t st = (uint32_t)((g % kAStages) * kAStage);
#pragma unroll
  for (int u = 0; u < kADma; ++u) dma16(c.ra, c.lds_a[u] + st, c.a_off[u], gc * kGroup * 2);
  (void)ring;
}

// Group g's weights of this lane: K = k0 + 64 q .. + 63.  When K is an odd
// multiple of 128 the last group is half full; lanes past K load the
// group's first valid piece instead (never past the row) and are zeroed by
// lane_valid.
__device__ __forceinline__ void load_b(const Ctx& c, Weights& w, int g) {
  const int k0 = min(g, c.ngroups - 1) * kGroup;
  const int kq = k0 + 64 * c.q < c.K ? k0 + 64 * c.q : k0;
#pragma unroll
  for (int b = 0; b < kCB; ++b) {
#pragma unroll
    for (int h = 0; h < kWords / 4; ++h)
      w.b[b][h] = *reinterpret_cast<const i32x4*>(c.bcol[b] + kq / 2 + 16 * h);
    w.s[b] = *reinterpret_cast<const uint32_t*>(c.scol[b] + kq / 16);
  }
}

__device__ __forceinline__ bool lane_valid(const Ctx& c, int g) {
  return g < c.ngroups && g * kGroup + 64 * c.q < c.K;
}

// MFMAs of one group: activations from LDS stage `a`, weights from `w`;
// RB row blocks (the second is skipped when the chunk has at most 16 rows).
// Each activation fragment is read once per k slice and serves both column
// blocks.
template <int RB>
__device__ __forceinline__ void mma_group(const uint8_t* a, const Weights& w, bool valid, int lane,
                                          f32x4 acc[kRB][kCB]) {
  const int r = lane & 15, q = lane >> 4;
  uint32_t sc[kCB];
#pragma unroll
  for (int b = 0; b < kCB; ++b) sc[b] = valid ? w.s[b] : 0u;  // code 0 = scale 0: exact zeros
#pragma unroll
  for (int t = 0; t < kWords; ++t) {
    // k0 + 64 q + 8 t .. + 8: chunk 8 q + t of the lane's activation rows and
    // word t of its 32 weight bytes (block scale t / 2)
    bf16x8 af[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      af[rb] = *reinterpret_cast<const bf16x8*>(a + a_swz(16 * rb + r, 8 * q + t));
#pragma unroll
    for (int b = 0; b < kCB; ++b) {
      const float s = __builtin_amdgcn_cvt_f32_fp8((int)((sc[b] >> (8 * (t / 2))) & 0xFFu), 0);
      const bf16x8 bf = dequant8((uint32_t)w.b[b][t / 4][t % 4], s);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, af[rb], acc[rb][b], 0, 0, 0);
    }
  }
}

// One group i = g0 + I of the ring: wait until group i's activations and
// weights have landed, publish the stage, refill the rings (activations of
// group i + kAStages - 1 into the stage group i - 1 used, weights of group
// i + kAhead into the slot group i - 1 used), then compute group i.
template <int RB, int I>
__device__ __forceinline__ void group_step(const Ctx& c, uint8_t* ring, Weights (&w)[kBSlots],
                                           int g0, int lane, f32x4 acc[kRB][kCB]) {
  const int i = g0 + I;
  wait_vmem<kWaitAfter>();
  lds_barrier();
  load_a(c, ring, i + kAStages - 1);
  load_b(c, w[(I + kAhead) % kBSlots], i + kAhead);
  __builtin_amdgcn_sched_barrier(0);
  mma_group<RB>(ring + (I % kAStages) * kAStage, w[I % kBSlots], lane_valid(c, i), lane, acc);
  __builtin_amdgcn_sched_barrier(0);
}

template <int RB, int... I>
__device__ __forceinline__ void group_steps(const Ctx& c, uint8_t* ring, Weights (&w)[kBSlots],
                                            int g0, int lane, f32x4 acc[kRB][kCB],
                                            std::integer_sequence<int, I...>) {
  (group_step<RB, I>(c, ring, w, g0, lane, acc), ...);
}

// Two waves per SIMD at least (one wave's dequantisation overlaps another's
// load waits): at most 256 registers per lane.
__global__ __launch_bounds__(kThreads, 2) void w4a16_kernel(const uint16_t* __restrict__ A,
                                                         const uint8_t* __restrict__ B,
                                                         const uint8_t* __restrict__ b_scale,
                                                         const int32_t* __restrict__ m_indices,
                                                         float gb, uint16_t* __restrict__ C,
                                                         int M, int N, int K, int G) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kAStages * kAStage];
  __shared__ int rows[kScan];
  __shared__ int nrows;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nblk = N / kCols;
  const int n0 = (blockIdx.x % nblk) * kCols;
  const int g = blockIdx.x / nblk;
  const uint32_t Kp = (uint32_t)K / 2, Ks = (uint32_t)K / 16;

  Ctx c;
  c.q = lane >> 4;
  c.ngroups = (K + kGroup - 1) / kGroup;
  c.K = K;
  c.ra = rsrc(A, (uint32_t)((size_t)M * K * 2));
#pragma unroll
  for (int b = 0; b < kCB; ++b) {
    const size_t col = (size_t)g * N + n0 + 32 * wave + 16 * b + (lane & 15);
    c.bcol[b] = B + col * Kp;
    c.scol[b] = b_scale + col * Ks;
  }

  for (int scan0 = 0; scan0 < M; scan0 += kScan) {
    // Compact the rows of this expert among m_indices[scan0, scan0 + kScan).
    __syncthreads();  // the previous chunks are done with rows[] and the ring
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
      // This thread's activation chunks: LDS chunk p = u * 256 + tid of a
      // stage is row p / kChunks, physical chunk p % kChunks, which holds
      // logical chunk (p % kChunks) ^ row; rows past the chunk read a valid
      // row and are never stored.
#pragma unroll
      for (int u = 0; u < kADma; ++u) {
        const int p = u * kThreads + tid;
        const int row = p / kChunks, lc = (p % kChunks) ^ row;
        c.a_off[u] = (uint32_t)rows[min(c0 + row, count - 1)] * (uint32_t)K * 2u + (uint32_t)lc * 16u;
        c.lds_a[u] = lds_addr(ring) + (uint32_t)(u * kThreads + wave * 64) * 16u;
      }
      f32x4 acc[kRB][kCB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int b = 0; b < kCB; ++b) acc[rb][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

      // Prologue in the steady-state order: the weights of the first kLead
      // groups, then (activations j, weights j + kLead).
      Weights w[kBSlots];
#pragma unroll
      for (int j = 0; j < kLead; ++j) load_b(c, w[j], j);
#pragma unroll
      for (int j = 0; j < kAStages - 1; ++j) {
        load_a(c, ring, j);
        load_b(c, w[j + kLead], j + kLead);
      }
      if (count - c0 > 16) {
        for (int g0 = 0; g0 < c.ngroups; g0 += kBSlots)
          group_steps<2>(c, ring, w, g0, lane, acc, std::make_integer_sequence<int, kBSlots>{});
      } else {
        for (int g0 = 0; g0 < c.ngroups; g0 += kBSlots)
          group_steps<1>(c, ring, w, g0, lane, acc, std::make_integer_sequence<int, kBSlots>{});
      }
      wait_vmem<0>();  // no load into the ring may outlive the chunk
      lds_barrier();

      // Lane holds C[row c0 + 16 rb + l % 16][n0 + 32 w + 16 b + 4 (l / 16) + t].
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const int m = c0 + 16 * rb + (lane & 15);
        if (m >= count) continue;
        uint16_t* crow = C + (size_t)rows[m] * N + n0 + 32 * wave + 4 * (lane >> 4);
#pragma unroll
        for (int b = 0; b < kCB; ++b)
          *reinterpret_cast<uint2*>(crow + 16 * b) =
              pack_bf16x4(gb * acc[rb][b][0], gb * acc[rb][b][1], gb * acc[rb][b][2],
                          gb * acc[rb][b][3]);
      }
    }
  }
}

}  // namespace w4a16_detail

using namespace w4a16_detail;

hipError_t launch_w4a16(const W4A16Args& a, hipStream_t s) {
  if (a.N % kCols || a.K % 128) return hipErrorInvalidValue;
  const long long grid = (long long)(a.N / kCols) * a.G;
  if (grid <= 0 || grid > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(w4a16_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a.A, a.B,
                     a.b_scale, a.m_indices, a.b_global, a.C, a.M, a.N, a.K, a.G);
  return hipGetLastError();
}

}  // namespace fgg
