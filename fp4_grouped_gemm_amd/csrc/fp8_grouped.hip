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
//    a BN x 128 B tile in LDS through a ring of 2 or 3 stages: the loads of
//    step k + STAGES - 1 are issued at the start of step k, so with 3 stages
//    every load has two steps to arrive and the latency of the next batch
//    overlaps the transfer of the previous one (the 256x256 shape only fits
//    2 stages in LDS).  Direct global->LDS 16-byte loads, an XOR swizzle of
//    16-byte chunks by row so fragment reads hit distinct banks.
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
#include "offsets.h"

#include <algorithm>
#include <climits>

namespace fgg {
namespace fp8_detail {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, int SA_BLK_, int SA_ROW_>
struct Fp8Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int STAGES = STAGES_;  // LDS stages of the A/B ring (2 or 3)
  // a_scale is staged in chunks of SA_BLK K blocks, SA_ROW floats per row in
  // LDS (SA_ROW >= SA_BLK, a power of two; the extra values are unused).
  static constexpr int SA_BLK = SA_BLK_, SA_ROW = SA_ROW_;
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
  // a_scale chunk: BM rows x SA_ROW floats, 64 floats per load instruction
  static constexpr int SA_LOADS = BM * SA_ROW / 64 / WAVES;
  static_assert((BM * SA_ROW) % (64 * WAVES) == 0, "a_scale chunk split");
  static_assert(SA_BLK <= SA_ROW && (SA_ROW & (SA_ROW - 1)) == 0, "a_scale chunk layout");
  static_assert(STAGES == 2 || (STAGES == 3 && SA_BLK == 3), "the 3-stage loop pairs chunks with stages");
  static constexpr int VM_TILE = A_LOADS + B_LOADS;  // loads per step into the A/B ring
  static_assert(WAVES % 2 == 0, "the staging swizzle assumes an even wave count");
  static_assert(WM == 64 && BM <= 512, "one row per lane in the pass masks");
};

// LDS byte offset of 16-byte chunk `c` (0..7) of tile row `r`: an XOR
// swizzle whose key (offsets.h) keeps every cycle of a fragment read free of
// bank conflicts.
__device__ __forceinline__ int swz(int r, int c) { return off::fp8_lds_off(r, c); }

// Fragment of 16 rows x 128 K bytes for v_mfma_*_16x16x128 with 8-bit
// operands: lane l holds row (l % 16) and K bytes [32 q, 32 q + 32), q = l / 16.
// The A and B operands use the same lane/K assignment, so the product sums
// over every k exactly once whatever order the hardware uses inside a lane.
// row0 is a multiple of 16 and the swizzle key reads row bits 1..3 only, so
// the lane's part of the offset does not depend on row0.
__device__ __forceinline__ i32x8 read_frag(const uint8_t* tile, int row0, int lane) {
  const uint8_t* p = tile + row0 * 128;
  const int r = lane & 15;
  const int q = lane >> 4;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(p + swz(r, 2 * q));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(p + swz(r, 2 * q + 1));
  return (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

using namespace lds_dma;

// Per-pass state: buffer resources, offsets, the b_scale row, accumulators.
//  * A/B staging: a tile row is K bytes for both operands; lane l of a
//    1 KB load writes LDS bytes [16 l, 16 l + 16) = tile row 8 b + l / 8,
//    physical chunk l % 8, so it fetches logical chunk (l % 8) ^ key(row).
//    Load s of wave w covers rows 8 (s W + w) .. + 7: the lane's offset
//    (row and chunk) goes in the instruction's VGPR offset, which the buffer
//    range check covers, so rows past the tile's last row return zeros
//    without touching memory; only the step's in-row kb * 128 goes in the
//    SGPR offset, which the range check leaves out (a chunk of a row inside
//    the buffer then stays inside that row).
template <class T>
struct Pass {
  i32x4 ra, rb;  // A window rows, B[e] column-tile rows
  i32x4 rsa;     // a_scale rows of the window
  uint32_t lane_off;              // (8 w + l / 8) K + 16 chunk
  uint32_t K;
  int nkb;
  // b_scale row of this wave's 128-column block: lane l holds block
  // 64 c + l of the current chunk c of 64 K blocks (read with readlane, so
  // the K loop issues no scalar loads, whose out-of-order return would make
  // every LDS wait a full drain).
  const float* bs_row;
  float bs_vec;
  uint64_t a_groups;              // 8-row groups of A holding a row of this pass
  bool active;                    // this wave's 64 rows hold a row of this pass
  f32x4 acc[T::TM][T::TN];

  // Step kb's A tile into stage `st`.  Groups of rows of other experts are
  // not needed.  With 3 stages their loads go past the buffer end (zeros, no
  // memory traffic), so that every step issues the same number of loads,
  // which the waits count; with 2 stages (the wait is for all loads) they
  // are skipped.
  __device__ __forceinline__ void stage_a(uint8_t* st, int kb, int wave) const {
#pragma unroll
    for (int s = 0; s < T::A_LOADS; ++s) {
      const bool need = (a_groups >> (s * T::WAVES + wave)) & 1;
      if (T::STAGES == 2 && !need) continue;
      dma16(ra, lds_addr(st + (s * T::WAVES + wave) * 1024),
            off::fp8_tile_voff(lane_off, s, T::WAVES, K, need), off::fp8_step_soff(kb));
    }
  }
  __device__ __forceinline__ void stage_b(uint8_t* st, int kb, int wave) const {
#pragma unroll
    for (int s = 0; s < T::B_LOADS; ++s)
      dma16(rb, lds_addr(st + T::A_BYTES + (s * T::WAVES + wave) * 1024),
            off::fp8_tile_voff(lane_off, s, T::WAVES, K, true), off::fp8_step_soff(kb));
  }
  __device__ __forceinline__ void stage_in(uint8_t* st, int kb, int wave) const {
    stage_a(st, kb, wave);
    stage_b(st, kb, wave);
  }

  // a_scale values of K blocks [c SA_BLK, c SA_BLK + SA_ROW) of every window
  // row, as [row][SA_ROW] floats: one 4-byte direct-to-LDS load per lane,
  // SA_ROW lanes per row (one short piece per row instead of one cache line
  // per row per step).  Blocks past the row's last one load from past the
  // buffer end (zeros, no access); rows past the window's last row fail the
  // range check likewise.  Values past the chunk are unused.
  __device__ __forceinline__ void stage_scales(float* buf, int c, int wave, int lane) const {
#pragma unroll
    for (int s = 0; s < T::SA_LOADS; ++s) {
      const int g = (s * T::WAVES + wave) * 64 + lane;  // row g / SA_ROW, block g % SA_ROW
      dma4(rsa, lds_addr(buf + (s * T::WAVES + wave) * 64),
           off::fp8_scale_voff(g, c, T::SA_BLK, T::SA_ROW, nkb), 0);
    }
  }

  // Blocks [kb, kb + 64) of the b_scale row into bs_vec (kb a multiple of
  // 64).  The value is used at once (the empty asm reads it), so the compiler
  // waits for this load here and nowhere else: its own waits do not see the
  // staging loads (inline assembly), and a wait for this load placed inside
  // the K loop would drain them.
  __device__ __forceinline__ void issue_b_scales(int kb, int lane) {
    bs_vec = kb + lane < nkb ? bs_row[kb + lane] : 0.f;
  }
  __device__ __forceinline__ void load_b_scales(int kb, int lane) {
    issue_b_scales(kb, lane);
    asm volatile("" ::"v"(bs_vec));
  }
  // B[e]'s rows of this column tile and the b_scale row of this wave's
  // 128-column block.
  __device__ __forceinline__ void set_expert(const uint8_t* B, const float* b_scale, int e, int N,
                                             int col0, int wcol0, int rows_b) {
    rb = rsrc(B + ((size_t)e * N + col0) * K, (uint32_t)rows_b * K);
    bs_row = b_scale + ((size_t)e * (N >> 7) + (min(wcol0, N - 1) >> 7)) * nkb;
  }
  __device__ __forceinline__ float b_scale_of(int kb) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bs_vec), kb & 63));
  }
};

// MFMA slot t of a K step (t = j TM + i: column subtile j, row subtile i,
// j-major) and the promotion of slot t - LAG: the partial of an MFMA is
// promoted LAG MFMAs later, from a small ring, so the FMAs overlap the
// following MFMAs and few partials are live at once; the next column
// subtile's B fragment is read TM MFMAs before its first use.
constexpr int kLag = 3;
template <class T>
__device__ __forceinline__ void mfma_slot(Pass<T>& ps, int t, i32x8& bf, i32x8& bnext,
                                          const i32x8* af, f32x4* ring, float* s, const float* sa,
                                          float sb, const uint8_t* rb, int wn, int lane) {
  constexpr int NT = T::TM * T::TN;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  if (t < NT) {
    const int j = t / T::TM, i = t % T::TM;
    if (i == 0) {
      if (j > 0) bf = bnext;
      if (j + 1 < T::TN) bnext = read_frag(rb, wn * T::WN + (j + 1) * 16, lane);
    }
    ring[t % (kLag + 1)] =
        __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], zero, 0, 0, 0, 127, 0, 127);
  }
  if (t >= kLag) {
    const int u = t - kLag;
    const int j = u / T::TM, i = u % T::TM;
    // the combined scale of row subtile i at its first use, so that the
    // wait for its a_scale read comes after the first MFMAs
    if (j == 0) s[i] = sa[i] * sb;
    ps.acc[i][j] += ring[u % (kLag + 1)] * s[i];
  }
  // Keep this order: left to itself the scheduler moves the FMAs next to
  // the MFMA whose result they read and the fragment reads next to their
  // use, which stalls on both latencies.
  __builtin_amdgcn_sched_barrier(0);
}

// One K step: start staging step kb + STAGES - 1 into `wr` (if any), then
// compute step kb from `rd`, then wait for step kb + 1's tiles and barrier.
// `rd` and `wr` are distinct __shared__ arrays (likewise the a_scale chunk
// buffers), which lets the compiler see that the LDS reads of `rd` do not
// depend on the loads still filling `wr`.
template <class T>
__device__ __forceinline__ void kstep(Pass<T>& ps, const uint8_t* rd, uint8_t* wr,
                                      const float* sa_rd, float* sa_wr, int kb, int lane, int wave,
                                      int wm, int wn) {
  const float sb = ps.b_scale_of(kb);
  const int kl = kb + T::STAGES - 1;  // the step whose tiles this step loads
  const bool load = kl < ps.nkb;
  // the next a_scale chunk, at the first step of a chunk (implies `load`)
  const bool sload = (unsigned)kb % T::SA_BLK == 0 && kb + T::SA_BLK < ps.nkb;
  if (load) {
    ps.stage_in(wr, kl, wave);
    if (sload) ps.stage_scales(sa_wr, (unsigned)kb / T::SA_BLK + 1, wave, lane);
  }
  if (ps.active) {
    constexpr int NT = T::TM * T::TN;
    const uint8_t* rb = rd + T::A_BYTES;
    i32x8 bf, bnext, af[T::TM];
    f32x4 ring[kLag + 1];
    float sa[T::TM], s[T::TM];
    // B fragment first: the first MFMA then waits for it and A fragment 0
    // only; the a_scale values of the lane's rows after the fragments
    bf = read_frag(rb, wn * T::WN, lane);
#pragma unroll
    for (int i = 0; i < T::TM; ++i) af[i] = read_frag(rd, wm * T::WM + i * 16, lane);
    bnext = bf;
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
      sa[i] = sa_rd[(wm * T::WM + i * 16 + (lane & 15)) * T::SA_ROW + (unsigned)kb % T::SA_BLK];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT + kLag; ++t) mfma_slot<T>(ps, t, bf, bnext, af, ring, s, sa, sb, rb, wn, lane);
  }
  if constexpr (T::STAGES == 2) {
    // step kb + 1's tiles were issued in this step
    wait_vmem<0>();
    lds_barrier();
  } else {
    // Step kb + 1's tiles were issued one step ago: only this step's loads
    // may stay in flight.
    if (!load) wait_vmem<0>();
    else if (sload) wait_vmem<T::VM_TILE + T::SA_LOADS>();
    else wait_vmem<T::VM_TILE>();
    lds_barrier();
  }
  // next chunk of 64 b_scale blocks (K above 8192; its wait drains the
  // loads in flight, once every 64 steps)
  if ((kb & 63) == 63 && kb + 1 < ps.nkb) ps.load_b_scales(kb + 1, lane);
}

// The K loop of one pass (buffer resources, offsets and the b_scale row
// set, accumulators zeroed).  Step 0's tiles and the b_scale row travel
// together, unless their A tiles (a_pre) or B tiles and b_scale row (b_pre)
// were issued early, with the steps the ring holds; the b_scale row is
// waited for at once (load_b_scales), which also waits for step 0.  With 3
// stages, step 1 is issued after that wait.
template <class T>
__device__ __forceinline__ void k_loop(Pass<T>& ps, uint8_t* lds0, uint8_t* lds1, uint8_t* lds2,
                                       float* sa0, float* sa1, bool a_pre, bool b_pre, int lane,
                                       int wave, int wm, int wn) {
  const int nkb = ps.nkb;
  if (!a_pre) {
    ps.stage_a(lds0, 0, wave);
    ps.stage_scales(sa0, 0, wave, lane);
  }
  if (!b_pre) {
    ps.stage_b(lds0, 0, wave);
    ps.load_b_scales(0, lane);
  }
  wait_vmem<0>();
  asm volatile("" ::"v"(ps.bs_vec));
  if constexpr (T::STAGES == 2) {
    lds_barrier();
    // K steps two at a time (LDS stage parity), scale chunks of SA_BLK
    // steps alternate between sa0 and sa1.
    for (int kb = 0; kb < nkb; kb += 2) {
      const bool odd_chunk = ((unsigned)kb / T::SA_BLK) & 1;
      float* sa_rd = odd_chunk ? sa1 : sa0;
      float* sa_wr = odd_chunk ? sa0 : sa1;
      kstep<T>(ps, lds0, lds1, sa_rd, sa_wr, kb, lane, wave, wm, wn);
      if (kb + 1 < nkb) kstep<T>(ps, lds1, lds0, sa_rd, sa_wr, kb + 1, lane, wave, wm, wn);
    }
  } else {
    if (nkb > 1) {
      if (!a_pre) ps.stage_a(lds1, 1, wave);
      if (!b_pre) ps.stage_b(lds1, 1, wave);
    }
    lds_barrier();
    // Six steps per iteration: stage = kb % 3 and scale chunk kb / 3
    // (alternating sa0 / sa1) are then known at compile time.
    for (int kb = 0; kb < nkb; kb += 6) {
      kstep<T>(ps, lds0, lds2, sa0, sa1, kb, lane, wave, wm, wn);
      if (kb + 1 < nkb) kstep<T>(ps, lds1, lds0, sa0, sa1, kb + 1, lane, wave, wm, wn);
      if (kb + 2 < nkb) kstep<T>(ps, lds2, lds1, sa0, sa1, kb + 2, lane, wave, wm, wn);
      if (kb + 3 < nkb) kstep<T>(ps, lds0, lds2, sa1, sa0, kb + 3, lane, wave, wm, wn);
      if (kb + 4 < nkb) kstep<T>(ps, lds1, lds0, sa1, sa0, kb + 4, lane, wave, wm, wn);
      if (kb + 5 < nkb) kstep<T>(ps, lds2, lds1, sa1, sa0, kb + 5, lane, wave, wm, wn);
    }
  }
}

// Store the pass's rows of the accumulators as BF16: row r of the tile
// (global row row0 + r) when store_row(r) holds, columns below N.  Lane
// holds C[m][n .. n + 3].
template <class T, class RowOk>
__device__ __forceinline__ void epilogue(const Pass<T>& ps, uint16_t* C, int row0, int wcol0, int N,
                                         int wm, int lane, RowOk store_row) {
#pragma unroll
  for (int i = 0; i < T::TM; ++i) {
    const int rl = wm * T::WM + i * 16 + (lane & 15);
    if (!store_row(rl)) continue;
    uint16_t* crow = C + (size_t)(row0 + rl) * N;
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const int n = wcol0 + j * 16 + 4 * (lane >> 4);
      if (n < N)
        *reinterpret_cast<uint2*>(crow + n) =
            pack_bf16x4(ps.acc[i][j][0], ps.acc[i][j][1], ps.acc[i][j][2], ps.acc[i][j][3]);
    }
  }
}

template <class T>
__global__ __launch_bounds__(T::THREADS) void fp8_grouped_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
    const float* __restrict__ a_scale, const float* __restrict__ b_scale,
    const int32_t* __restrict__ m_indices, uint16_t* __restrict__ C, int M, int N, int K, int G,
    int num_windows, int num_ntiles, int total_tiles, int group_w, int split) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[T::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[T::STAGES > 2 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(256))) float sa0[T::BM * T::SA_ROW];
  __shared__ __attribute__((aligned(256))) float sa1[T::BM * T::SA_ROW];
  __shared__ int ids[T::BM];
  __shared__ uint32_t plan_bits[kPlanWords];
  __shared__ int plan_heavy;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WAVES_N;
  const int wn = wave % T::WAVES_N;
  const int nkb = K >> 7;

  Pass<T> ps;
  ps.K = (uint32_t)K;
  ps.nkb = nkb;
  // row of this lane inside its load's 8-row group, and its swizzled chunk;
  // the group's first row 8 (s W + w) has bits 1..3 equal to 4 (w % 2)
  // because W is even, so the swizzle does not depend on s.
  ps.lane_off = off::fp8_lane_off(wave, lane, (uint32_t)K);

  // With split > 1 every pass of a tile is its own work item (the tile
  // order then needs no plan: no item costs more than one pass).
  build_plan<T::BM, T::THREADS>(plan_bits, &plan_heavy, split > 1 ? nullptr : m_indices, M, G,
                                num_windows);
  const int heavy = plan_heavy;
  const int items = total_tiles * split;

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int tile = split > 1 ? item / split : item;
    const int run_sel = split > 1 ? item % split : 0;  // split mode: this item's expert
    int window, ntile;
    plan_tile(plan_bits, heavy, tile, num_windows, num_ntiles, group_w, window, ntile);
    const int row0 = window * T::BM;
    const int col0 = ntile * T::BN;

    __syncthreads();  // the previous tile is done with ids[] and the stages

    // Rows (A) and columns (B) of this tile that exist; loads past them
    // read zeros and those rows / columns are never stored.
    const int rows_a = min(T::BM, M - row0);
    const int rows_b = min(T::BN, N - col0);
    ps.ra = rsrc(A + (size_t)row0 * K, (uint32_t)rows_a * (uint32_t)K);
    ps.rsa = rsrc(a_scale + (size_t)row0 * nkb, (uint32_t)rows_a * (uint32_t)nkb * 4u);
    const int wcol0 = col0 + wn * T::WN;

    // The A tiles of the first two K steps and the first a_scale chunk
    // depend on the window only, not on the routing: the 3-stage shapes
    // issue them now, every row group, so that they travel with the
    // m_indices reads instead of after them, and the first pass that runs
    // uses them (rows of other experts are computed and never stored).  The
    // 2-stage 256x256 shape, which holds all 256 VGPRs in its K loop, does
    // not: there the early offsets spill.
    // In split mode the item's expert is known before the routing is read
    // (item r of a tile runs expert r), so its B tiles of those steps and its
    // b_scale row go out now as well.
    bool a_pre = false, b_pre = false;
    if constexpr (T::STAGES > 2) {
      ps.a_groups = ~0ull;
      ps.stage_a(lds0, 0, wave);
      ps.stage_scales(sa0, 0, wave, lane);
      if (nkb > 1) ps.stage_a(lds1, 1, wave);
      a_pre = true;
      if (split > 1) {
        ps.set_expert(B, b_scale, run_sel, N, col0, wcol0, rows_b);
        ps.stage_b(lds0, 0, wave);
        ps.issue_b_scales(0, lane);
        if (nkb > 1) ps.stage_b(lds1, 1, wave);
        b_pre = true;
      }
    }

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
      if (ids[r] == -1 && col < N && run_sel == 0)
        *reinterpret_cast<uint4*>(C + (size_t)(row0 + r) * N + col) = make_uint4(0, 0, 0, 0);
    }

    // One pass per distinct expert present in the window, in increasing id;
    // in split mode, one pass for expert run_sel if the window holds a row
    // of it.  Every wave takes the same passes.
    int cur = -1;
    for (int pass = 0;; ++pass) {
      int e;
      if (split > 1) {
        if (pass > 0) break;
        e = run_sel;
        bool has = false;
        for (int r = lane; r < T::BM; r += 64) has |= ids[r] == e;
        if (__ballot(has) == 0) break;
      } else {
        e = INT_MAX;
        for (int r = lane; r < T::BM; r += 64) {
          const int v = ids[r];
          if (v > cur && v < e) e = v;
        }
        e = __builtin_amdgcn_readfirstlane(wave_min(e));
        if (e == INT_MAX) break;
        cur = e;
      }

      // Which rows this pass needs: A loads of 8-row groups without a row of
      // expert e are skipped, and a wave whose 64 rows hold none computes
      // nothing (a window that straddles a run boundary then costs little
      // more than its useful rows).
      {
        bool g = false;
        if (lane < T::BM / 8) {
#pragma unroll
          for (int q = 0; q < 8; ++q) g |= ids[lane * 8 + q] == e;
        }
        ps.a_groups = __ballot(g);
        ps.active = __ballot(ids[wm * T::WM + lane] == e) != 0;
      }
      ps.set_expert(B, b_scale, e, N, col0, wcol0, rows_b);
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) ps.acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

      k_loop<T>(ps, lds0, lds1, lds2, sa0, sa1, a_pre, b_pre, lane, wave, wm, wn);
      a_pre = b_pre = false;

      // Epilogue: this expert's rows only.
      epilogue<T>(ps, C, row0, wcol0, N, wm, lane,
                  [&](int rl) { return row0 + rl < M && ids[rl] == e; });
    }
    // No pass ran (a window of padding rows only, or a split item whose
    // expert has no row in the window): the early loads are still writing
    // the stages; let them land before the stages change hands or the
    // workgroup ends.
    if (a_pre || b_pre) wait_vmem<0>();
  }
}

// A batch of independent dense FP8 GEMMs of different shapes in one launch
// (the cutlass#3124 page's grouped block-scaled GEMM, "Intro": problems with
// their own M, N and K).  Work item t belongs to the problem whose range
// [tile_start[g], tile_start[g + 1]) holds it; inside a problem, tiles follow
// the XCD-aware map_tile order.  Every tile is one pass of the same K loop
// and epilogue as the grouped kernel's, with the problem's own K, offsets
// and b_scale row; rows and columns past the problem's M and N read zeros
// and are not stored.
template <class T>
__global__ __launch_bounds__(T::THREADS) void fp8_problems_kernel(const Fp8ProblemSet set,
                                                                  int group_w) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[T::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[T::STAGES > 2 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(256))) float sa0[T::BM * T::SA_ROW];
  __shared__ __attribute__((aligned(256))) float sa1[T::BM * T::SA_ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WAVES_N;
  const int wn = wave % T::WAVES_N;
  const int total = set.tile_start[set.count];
  Pass<T> ps;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int g = 0;
    while (g + 1 < set.count && set.tile_start[g + 1] <= tile) ++g;
    const Fp8Problem& p = set.p[g];
    const int M = p.M, N = p.N, K = p.K;
    const int num_windows = (M + T::BM - 1) / T::BM;
    const int num_ntiles = (N + T::BN - 1) / T::BN;
    int window, ntile;
    map_tile(tile - set.tile_start[g], set.tile_start[g + 1] - set.tile_start[g], num_windows,
             num_ntiles, group_w, window, ntile);
    const int row0 = window * T::BM;
    const int col0 = ntile * T::BN;
    const int rows_a = min(T::BM, M - row0);
    const int rows_b = min(T::BN, N - col0);
    const int wcol0 = col0 + wn * T::WN;

    __syncthreads();  // the previous tile is done with the stages
    ps.K = (uint32_t)K;
    ps.nkb = K >> 7;
    ps.lane_off = off::fp8_lane_off(wave, lane, (uint32_t)K);
    ps.ra = rsrc(p.A + (size_t)row0 * K, (uint32_t)rows_a * (uint32_t)K);
    ps.rsa = rsrc(p.a_scale + (size_t)row0 * ps.nkb, (uint32_t)rows_a * (uint32_t)ps.nkb * 4u);
    ps.a_groups = ~0ull;
    ps.active = wm * T::WM < rows_a;  // a wave whose rows are all past M computes nothing
    ps.set_expert(p.B, p.b_scale, 0, N, col0, wcol0, rows_b);
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j) ps.acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    k_loop<T>(ps, lds0, lds1, lds2, sa0, sa1, false, false, lane, wave, wm, wn);
    epilogue<T>(ps, p.C, row0, wcol0, N, wm, lane, [&](int rl) { return rl < rows_a; });
  }
}

// Compiled tile shapes.  `tput` is the relative per-CU throughput the ranker
// uses, measured on MI355X by timing every shape on an 8192 x 8192 x 7168
// problem that each of them tiles into whole waves of the 256 CUs (so the
// ranker's other terms are 1): 2181, 1861, 1831 and 1416 TFLOPS.  256x256
// is fastest per CU; the 128x128 shape runs one wave per SIMD and hides less
// latency.  The 256x128 and 128x256 shapes run 8 waves of 64x64 (two per
// SIMD): faster than 4 waves of 64x128 (1694 and 1744 TFLOPS), though each
// wave reads more LDS bytes per MFMA.  wg_per_cu follows from LDS use (the
// 3-stage shapes take 100-153 KB, so one workgroup per CU).
using Cfg0 = Fp8Cfg<256, 256, 4, 2, 2, 8, 8>;  // 8 waves, 64x128 per wave, 2 x 64 KB stages
using Cfg1 = Fp8Cfg<256, 128, 4, 2, 3, 3, 4>;  // 8 waves, 64x64 per wave,  3 x 48 KB stages
using Cfg2 = Fp8Cfg<128, 256, 2, 4, 3, 3, 4>;  // 8 waves, 64x64 per wave,  3 x 48 KB stages
using Cfg3 = Fp8Cfg<128, 128, 2, 2, 3, 3, 4>;  // 4 waves, 64x64 per wave,  3 x 32 KB stages

const TileCfg kFp8Tiles[] = {
    {0, 256, 256, 8, 1, 1.00f},
    {1, 256, 128, 8, 1, 0.85f},
    {2, 128, 256, 8, 1, 0.84f},
    {3, 128, 128, 4, 1, 0.65f},
};

template <class T>
hipError_t launch_cfg(const Fp8Args& a, const LaunchOpts& o, hipStream_t s) {
  const int num_windows = (a.M + T::BM - 1) / T::BM;
  const int num_ntiles = (a.N + T::BN - 1) / T::BN;
  const long long total = (long long)num_windows * num_ntiles;
  if (total <= 0) return hipSuccess;
  if (total > INT_MAX) return hipErrorInvalidValue;
  const int split = split_items(o.run_split, a.m_indices != nullptr, a.G, T::BM, total, o.num_cus);
  int grid = (int)(total * split);
  if (o.max_wg > 0 && o.max_wg < grid) grid = o.max_wg;
  // Row windows per tile group (all column tiles of a group run in one XCD,
  // window fastest).  4 windows: a model of each XCD's L2 over the tiles in
  // flight put c2's L2 misses at 770 MB against 1090 MB with 8 (it matches
  // the measured 1.23 GB and 50% hit rate of that order); measured c2 +3%,
  // c3 +1% on MI355X.
  const int group_w = 4;
  hipLaunchKernelGGL(fp8_grouped_kernel<T>, dim3(grid), dim3(T::THREADS), 0, s, a.A, a.B,
                     a.a_scale, a.b_scale, a.m_indices, a.C, a.M, a.N, a.K, a.G, num_windows,
                     num_ntiles, (int)total, group_w, split);
  return hipGetLastError();
}

// Tile ranges of a problem batch for tile shape BM x BN.
inline long long problem_tiles(Fp8ProblemSet& set, int BM, int BN) {
  long long total = 0;
  for (int g = 0; g < set.count; ++g) {
    set.tile_start[g] = (int)total;
    total += (long long)((set.p[g].M + BM - 1) / BM) * ((set.p[g].N + BN - 1) / BN);
    if (total > INT_MAX) return -1;
  }
  set.tile_start[set.count] = (int)total;
  return total;
}

template <class T>
hipError_t launch_problems_cfg(Fp8ProblemSet set, const LaunchOpts& o, hipStream_t s) {
  const long long total = problem_tiles(set, T::BM, T::BN);
  if (total < 0) return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  int grid = (int)total;
  if (o.max_wg > 0 && o.max_wg < grid) grid = o.max_wg;
  hipLaunchKernelGGL(fp8_problems_kernel<T>, dim3(grid), dim3(T::THREADS), 0, s, set, 4);
  return hipGetLastError();
}

}  // namespace fp8_detail

using namespace fp8_detail;

int fp8_num_tiles() { return (int)(sizeof(kFp8Tiles) / sizeof(kFp8Tiles[0])); }
const TileCfg& fp8_tile(int id) { return kFp8Tiles[id]; }

hipError_t launch_fp8_problems(const Fp8ProblemSet& in, int tile_id, const LaunchOpts& o,
                               hipStream_t s) {
  if (in.count < 1 || in.count > kMaxProblems) return hipErrorInvalidValue;
  // Longest K loops first (the order of the problems does not change any
  // result): workgroups that draw the short tiles last even out the finish.
  Fp8ProblemSet set = in;
  std::stable_sort(set.p, set.p + set.count,
                   [](const Fp8Problem& a, const Fp8Problem& b) { return a.K > b.K; });
  switch (tile_id) {
    case 0: return launch_problems_cfg<Cfg0>(set, o, s);
    case 1: return launch_problems_cfg<Cfg1>(set, o, s);
    case 2: return launch_problems_cfg<Cfg2>(set, o, s);
    case 3: return launch_problems_cfg<Cfg3>(set, o, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fp8(const Fp8Args& a, int tile_id, const LaunchOpts& o, hipStream_t s) {
  switch (tile_id) {
    case 0: return launch_cfg<Cfg0>(a, o, s);
    case 1: return launch_cfg<Cfg1>(a, o, s);
    case 2: return launch_cfg<Cfg2>(a, o, s);
    case 3: return launch_cfg<Cfg3>(a, o, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fgg
