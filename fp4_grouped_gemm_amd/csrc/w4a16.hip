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
// from HBM with direct-to-LDS loads of whole 128-byte lines, which stream
// faster than loads into registers, and overlaps the dequantisation of one
// group with the loads of the next.
//  * One workgroup (4 waves) per (expert, 128-column block); wave w owns
//    columns 32 w .. 32 w + 31 (two MFMA column blocks) over all of K, so
//    no partial sums cross waves.  Wave 0 first compacts the rows routed to
//    the expert into LDS (ballot + popcount, in row order; expert 0's
//    workgroups also zero the padding rows found); a workgroup whose expert
//    has no rows stops there and never reads that expert's weights.
//  * K runs in groups of 256.  Rows run 32 at a time (two MFMA row blocks
//    sharing each dequantised weight fragment).  Their activations, 32 rows
//    x 256 K per group, go through a 2-stage LDS ring shared by the four
//    waves; each wave's weights, 32 rows of 128 packed bytes plus their 16
//    scale bytes per group, through a 2-slot LDS ring of its own.  Both are
//    filled by direct-to-LDS loads (no registers): a weight load moves 8
//    whole lines.  16-byte chunks are XOR-swizzled by row so that fragment
//    reads hit 16 distinct bank groups per cycle.  Group i + 1 is issued as
//    group i starts, so one group's loads are in flight while the previous
//    one is computed (about 70 KB per CU with two workgroups per CU).
//  * Weights are dequantised exactly to BF16 in registers (q * s has at most
//    6 significant bits and lies in [2^-10, 2688]): the E2M1 pair convert with
//    scale 1.0, an FP32 multiply by the block scale, and the upper halves of
//    two exact products packed as a BF16 pair (no rounding needed).  Then
//    v_mfma_f32_16x16x32_bf16 with FP32 accumulation: lane (r, q) of the
//    activation operand and lane (c, q) of the weight operand hold the same
//    eight k, so every k pairs with itself.
#include "common.h"
#include "offsets.h"

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
constexpr int kStages = 2;             // depth of both LDS rings
constexpr int kAStage = kRows * kGroup * 2;         // bytes per activation stage
constexpr int kADma = kAStage / 16 / kThreads;      // 16-byte loads per thread
constexpr int kWRows = 16 * kCB;                    // weight rows (columns) per wave
constexpr int kWCode = kWRows * kGroup / 2;         // packed bytes per wave per group
constexpr int kWDma = kWCode / 1024;                // whole-line loads per wave per group
constexpr int kWSlot = kWCode + 1024;               // + the scale bytes' load (64 lanes x 16 B)
static_assert(kCols == 2 * 64, "a zero row is one 4-byte store per lane");
static_assert(kADma * 16 * kThreads == kAStage, "activation staging split");
static_assert(kWRows * 16 <= 1024, "a wave's scale bytes fit one load");

// The two codes of byte H times s, as a BF16 pair.  q * s has at most 6
// significant bits, so its FP32 value carries no bits below the top 16 and
// BF16 is that upper half exactly: a byte permute takes the upper halves of
// the two products (one instruction per pair, as a rounding convert would
// be; no rounding is needed).  A NaN scale code gives the quiet NaN
// 0x7FC00000, whose upper half is a BF16 NaN.
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

// LDS byte offset of 16-byte chunk c (0..31) of activation row r (0..31):
// an XOR swizzle whose key (offsets.h) keeps every cycle of a fragment read
// free of bank conflicts.
__device__ __forceinline__ int a_swz(int r, int c) { return off::w4a16_lds_off(r, c); }
static_assert(kChunks == kRows && kGroup * 2 == 512, "the chunk swizzle uses the row's 5 bits");
static_assert(kGroup == 256, "off::w4a16_act_voff assumes groups of 256 values");

struct Ctx {
  i32x4 ra;                   // activation buffer resource (whole A)
  i32x4 rw, rs;               // this wave's 32 weight rows and their scale rows
  uint32_t a_row[kADma];      // this lane's activation chunks: their rows
  int a_lc[kADma];            // and logical chunks (8 values) within a group
  uint32_t lds_a[kADma];      // their LDS destinations (stage 0)
  int w_lc[kWDma];            // this lane's weight chunk per whole-line load
  uint32_t Kp, Ks;
  int ngroups;
  int K;
  int q;
};

// Issue group g's activation chunks into LDS stage g % kStages.  The whole
// offset is a VGPR offset, which the buffer range check sees; a chunk at or
// past K (the half-full last group when K is an odd multiple of 128) loads
// zeros from past the buffer end instead of the next row's values, so no
// value outside the row's K ever meets a weight (0 x Inf would be NaN).
__device__ __forceinline__ void load_a(const Ctx& c, int g) {
  const uint32_t st = (uint32_t)((g % kStages) * kAStage);
#pragma unroll
  for (int u = 0; u < kADma; ++u)
    dma16(c.ra, c.lds_a[u] + st, off::w4a16_act_voff(c.a_row[u], c.a_lc[u], g, c.K), 0);
}

// Issue group g's weights of this wave into its slot `slot`: load j moves
// rows 8 j .. 8 j + 7, lane l fetching 16 bytes of row 8 j + l / 8 into
// physical chunk l % 8; then the rows' 16 scale bytes, lanes 0..31 one row
// each (the other lanes load zeros into the slot's spare half).
__device__ __forceinline__ void load_w(const Ctx& c, uint32_t slot, int g, int lane) {
#pragma unroll
  for (int j = 0; j < kWDma; ++j)
    dma16(c.rw, slot + 1024u * j, off::w4a16_w_voff((uint32_t)(8 * j + lane / 8), c.w_lc[j], g, c.Kp), 0);
  dma16(c.rs, slot + kWCode, lane < kWRows ? off::w4a16_s_voff((uint32_t)lane, g, c.Ks) : kSkip, 0);
}

__device__ __forceinline__ bool lane_valid(const Ctx& c, int g) {
  return g * kGroup + 64 * c.q < c.K;
}

// MFMAs of one group: activations from LDS stage `a`, this wave's weights
// from its slot `w`; RB row blocks (the second is skipped when the chunk has
// at most 16 rows).  Lane (c, q) takes the 64 codes k0 + 64 q .. + 63 of
// weight row 16 b + c (chunks 2 q and 2 q + 1) and their four scale codes;
// each activation fragment is read once per k slice and serves both column
// blocks.
template <int RB>
__device__ __forceinline__ void mma_group(const uint8_t* a, const uint8_t* w, bool valid, int lane,
                                          f32x4 acc[kRB][kCB]) {
  const int r = lane & 15, q = lane >> 4;
  i32x4 wb[kCB][2];
  uint32_t sc[kCB];
#pragma unroll
  for (int b = 0; b < kCB; ++b) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      wb[b][h] = *reinterpret_cast<const i32x4*>(w + off::w4a16_w_lds_off(16 * b + r, 2 * q + h));
    const uint32_t s = *reinterpret_cast<const uint32_t*>(w + kWCode + (16 * b + r) * 16 + 4 * q);
    sc[b] = valid ? s : 0u;  // code 0 = scale 0: exact zeros past K
  }
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
      const bf16x8 bf = dequant8((uint32_t)wb[b][t / 4][t % 4], s);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, af[rb], acc[rb][b], 0, 0, 0);
    }
  }
}

// The K loop of one chunk of rows: group 0 was issued by the caller; each
// group waits for its loads (this wave's; the barrier then publishes every
// wave's activation chunks), issues the next group into the other stage and
// slot (their readers finished with the previous group before the
// barrier), then computes.
template <int RB>
__device__ __forceinline__ void k_loop(const Ctx& c, uint8_t* ring, uint8_t* wslots, int wave,
                                       int lane, f32x4 acc[kRB][kCB]) {
  const uint32_t wbase = lds_addr(wslots);
  for (int i = 0; i < c.ngroups; ++i) {
    wait_vmem<0>();
    lds_barrier();
    if (i + 1 < c.ngroups) {
      load_a(c, i + 1);
      load_w(c, wbase + (uint32_t)(((i + 1) % kStages) * kWSlot), i + 1, lane);
    }
    mma_group<RB>(ring + (i % kStages) * kAStage, wslots + (i % kStages) * kWSlot,
                  lane_valid(c, i), lane, acc);
  }
  (void)wave;
}

// Two workgroups per CU (76 KB of LDS each): two waves per SIMD, at most
// 256 registers per lane.
__global__ __launch_bounds__(kThreads, 2) void w4a16_kernel(const uint16_t* __restrict__ A,
                                                         const uint8_t* __restrict__ B,
                                                         const uint8_t* __restrict__ b_scale,
                                                         const int32_t* __restrict__ m_indices,
                                                         float gb, uint16_t* __restrict__ C,
                                                         int M, int N, int K, int G) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages * kAStage];
  __shared__ __attribute__((aligned(1024))) uint8_t wring[kWaves][kStages * kWSlot];
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
  c.Kp = Kp;
  c.Ks = Ks;
  c.ra = rsrc(A, (uint32_t)((size_t)M * K * 2));
  // this wave's weight rows (output columns n0 + 32 w ..) of expert g
  const size_t wrow0 = (size_t)g * N + n0 + kWRows * wave;
  c.rw = rsrc(B + wrow0 * Kp, (uint32_t)kWRows * Kp);
  c.rs = rsrc(b_scale + wrow0 * Ks, (uint32_t)kWRows * Ks);
#pragma unroll
  for (int j = 0; j < kWDma; ++j) c.w_lc[j] = (lane % 8) ^ off::w4a16_wkey(8 * j + lane / 8);
  uint8_t* wslots = wring[wave];

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
      // logical chunk (p % kChunks) ^ key(row); rows past the chunk read a
      // valid row and are never stored.
#pragma unroll
      for (int u = 0; u < kADma; ++u) {
        const int p = u * kThreads + tid;
        const int row = p / kChunks, lc = (p % kChunks) ^ off::w4a16_swz_key(row);
        c.a_row[u] = (uint32_t)rows[min(c0 + row, count - 1)];
        c.a_lc[u] = lc;
        c.lds_a[u] = lds_addr(ring) + (uint32_t)(u * kThreads + wave * 64) * 16u;
      }
      f32x4 acc[kRB][kCB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int b = 0; b < kCB; ++b) acc[rb][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

      load_a(c, 0);
      load_w(c, lds_addr(wslots), 0, lane);
      if (count - c0 > 16)
        k_loop<2>(c, ring, wslots, wave, lane, acc);
      else
        k_loop<1>(c, ring, wslots, wave, lane, acc);
      lds_barrier();  // every wave is done with the rings before the next chunk

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
