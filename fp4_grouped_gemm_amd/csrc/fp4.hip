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
#include "offsets.h"

#include <algorithm>
#include <climits>
#include <utility>

namespace fgg {
namespace fp4_detail {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
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
  static_assert(WM == 64, "one row per lane in the pass masks");
};

__device__ __forceinline__ int swz(int r, int c) { return (r << 7) | ((c ^ (r & 7)) << 4); }

// Two E4M3FN codes (bytes 0 and 1 of `sc`) -> their values as an FP16 pair,
// with the hardware's pair convert at scale 1.0: exact (E4M3 has 4
// significant bits and spans 2^-9..448, all FP16 numbers), and the NaN codes
// S.1111.111 (E4M3FN has no infinities) come out as FP16 NaNs.
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t sc) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
}

// One 32-bit word (8 E2M1 codes, low nibble first) times its block scale ->
// 8 FP16 values in 16 bytes.  The hardware convert decodes the two codes of
// one byte; its scale operand contributes only a power of two, so it is 1.0
// here and the block scale is applied by an FP16 multiply, exact because
// q * s has at most 6 significant bits and lies in [2^-10, 2688].
__device__ __forceinline__ i32x4 dequant_word(uint32_t word, f16x2 ss) {
  const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * ss;
  const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * ss;
  const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * ss;
  const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * ss;
  return (i32x4){__builtin_bit_cast(int, v0), __builtin_bit_cast(int, v1),
                 __builtin_bit_cast(int, v2), __builtin_bit_cast(int, v3)};
}

// Fragment for v_mfma_f32_16x16x32_f16: lane l holds row (l % 16) and the
// 8 FP16 values of 16-byte chunk `kk * 4 + l / 16` of that row.  A and B use
// the same assignment, so every k is paired with itself.
__device__ __forceinline__ f16x8 read_frag(const uint8_t* tile, int row0, int lane, int kk) {
  const int r = row0 + (lane & 15);
  return *reinterpret_cast<const f16x8*>(tile + swz(r, kk * 4 + (lane >> 4)));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// A buffer offset past every buffer's end (buffers are below 2^31 bytes):
// a load there returns zeros.
constexpr uint32_t kSkip = 0x80000000u;

// Per-pass state.  Staging units: unit u of this thread covers tile row
// g / 2 (g = tid + u * THREADS), elements [32 h, 32 h + 32) of the K step,
// h = g % 2 = tid % 2.  Packed codes are loaded two steps ahead (two register
// sets, step s in set s % 2): the unit's row and half go in the VGPR offset
// (range-checked: rows past the tile read zeros) and the step's in-row
// displacement ks * 32 in the SGPR offset.  The four E4M3 scale codes of a
// row and step are contiguous, so the codes of four consecutive steps (16
// bytes) are loaded once per four steps, one group ahead (two groups, steps
// [4c, 4c + 4) in group c % 2), instead of four 2-byte loads that each touch
// one cache line per row; both lanes of a row load the same 16 bytes and
// each uses its half.
template <class T>
struct Pass {
  __amdgpu_buffer_rsrc_t ra, rsa, rb, rsb;  // window rows of A / a_scale, tile rows of B / b_scale
  uint32_t a_off[T::A_UNITS], as_off[T::A_UNITS], b_off[T::B_UNITS], bs_off[T::B_UNITS];
  // This pass's A offsets: those of rows of other experts are moved past the
  // end of the buffer, so their loads return zeros without touching memory
  // (a branch-free skip; the zeros are never stored).
  uint32_t pa_off[T::A_UNITS], pas_off[T::A_UNITS];
  i32x4 qa[2][T::A_UNITS], qb[2][T::B_UNITS];  // packed codes, two steps in flight
  i32x4 sa4[2][T::A_UNITS], sb4[2][T::B_UNITS];  // scale codes of 4 steps, two groups
  f32x4 acc[T::TM][T::TN];

  // Issue the loads of the packed codes of K step ks into register set `set`.
  __device__ __forceinline__ void load(int set, int ks) {
#pragma unroll
    for (int u = 0; u < T::A_UNITS; ++u)
      qa[set][u] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, pa_off[u], off::fp4_code_soff(ks), 0));
#pragma unroll
    for (int u = 0; u < T::B_UNITS; ++u)
      qb[set][u] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_off[u], off::fp4_code_soff(ks), 0));
  }

  // Issue the loads of the scale codes of steps [4c, 4c + 4) into group
  // `grp`: bytes [16c, 16c + 16) of the row's K / 16 codes, one 16-byte load
  // per unit with the whole offset (row and group) in the VGPR offset, which
  // the buffer range check covers dword by dword: a row's half-full last
  // group (K / 16 an odd multiple of 8) reads the next row's first codes,
  // or zeros past the tile's last row, never memory past the buffer.  Codes
  // past the last step are never used.
  __device__ __forceinline__ void load_scales(int grp, int c) {
#pragma unroll
    for (int u = 0; u < T::A_UNITS; ++u)
      sa4[grp][u] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(rsa, off::fp4_scale_voff(pas_off[u], c), 0, 0));
#pragma unroll
    for (int u = 0; u < T::B_UNITS; ++u)
      sb4[grp][u] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(rsb, off::fp4_scale_voff(bs_off[u], c), 0, 0));
  }

  // Chunk c of this thread's staging work for a step whose packed codes are
  // in register set `set` and scale codes at position `pos` of group `grp`:
  // unit c / 4 (A units first, then B units), 16-byte word c % 4 of it,
  // dequantised and written to LDS stage `st`.  Word 0 also decodes the
  // unit's two block scales (words 0-1 use the first, words 2-3 the second).
  f16x2 sdec[T::A_UNITS + T::B_UNITS];
  __device__ __forceinline__ void stage_chunk(int set, int grp, int pos, int c, uint8_t* st,
                                              int tid) {
    const int u = c >> 2, w = c & 3;
    const bool is_a = u < T::A_UNITS;
    const int v = is_a ? u : u - T::A_UNITS;
    const i32x4 q = is_a ? qa[set][v] : qb[set][v];
    if (w == 0) {
      const uint32_t codes = (uint32_t)(is_a ? sa4[grp][v][pos] : sb4[grp][v][pos]);
      sdec[u] = e4m3x2_to_f16x2(codes >> (16 * (tid & 1)));
    }
    const _Float16 s = w < 2 ? sdec[u][0] : sdec[u][1];
    const int g = tid + v * T::THREADS;
    uint8_t* dst = st + (is_a ? 0 : T::A_BYTES) + swz(g >> 1, (g & 1) * 4 + w);
    *reinterpret_cast<i32x4*>(dst) = dequant_word((uint32_t)q[w], (f16x2){s, s});
  }
  static constexpr int CHUNKS = 4 * (T::A_UNITS + T::B_UNITS);
  __device__ __forceinline__ void stage_all(int set, int grp, int pos, uint8_t* st, int tid) {
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) stage_chunk(set, grp, pos, c, st, tid);
  }
};

// Workgroup barrier ordering LDS accesses only.  __syncthreads() orders
// global memory too, which waits for every load in flight, the look-ahead
// loads included; nothing here shares global memory between waves.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The MFMAs of one K step from LDS stage `rd`, as 2 x TN slots (a K=32 half,
// one 16-column block of B: TM MFMAs).  With STAGE, slot k also stages chunks
// [k C / S, (k+1) C / S) of the next step (C chunks, S slots) from register
// set `set` into `wr`, so the dequantisation VALU work and LDS writes are
// spread evenly between the MFMAs of the wave; the scheduling fence after
// each slot keeps that spread.
template <class T, bool STAGE>
__device__ __forceinline__ void mma_step(Pass<T>& ps, const uint8_t* rd, uint8_t* wr, int set,
                                         int grp, int pos, int tid, int lane, int wm, int wn) {
  constexpr int S = 2 * T::TN, C = Pass<T>::CHUNKS;
  const uint8_t* rb = rd + T::A_BYTES;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f16x8 af[T::TM];
#pragma unroll
    for (int i = 0; i < T::TM; ++i) af[i] = read_frag(rd, wm * T::WM + i * 16, lane, h);
    f16x8 bnext = read_frag(rb, wn * T::WN, lane, h);
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const f16x8 bf = bnext;
      if (j + 1 < T::TN) bnext = read_frag(rb, wn * T::WN + (j + 1) * 16, lane, h);
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
        ps.acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[i], ps.acc[i][j], 0, 0, 0);
      if constexpr (STAGE) {
        const int k = h * T::TN + j;
#pragma unroll
        for (int c = 0; c < C; ++c)
          if (c * S / C == k) ps.stage_chunk(set, grp, pos, c, wr, tid);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One K step s = ks + Q from `rd` that also stages step s + 1 into `wr`:
// issue the packed-code loads of step min(s + 2, last) into register set
// s % 2 (free: it held step s, dequantised in the previous step) and, at the
// first step of a group of four, the scale codes of the next group; then the
// MFMAs with step s + 1 (set (s + 1) % 2, scales at position (s + 1) % 4 of
// group ((s + 1) / 4) % 2) dequantised between them.  ks is a multiple of 8,
// so all these indices are compile-time constants.  Every step issues the
// same loads (the last ones reload the last step), so the waits before the
// dequantisation count only older loads.  Returns false past the last step.
template <class T, int Q>
__device__ __forceinline__ bool kstep(Pass<T>& ps, uint8_t* lds0, uint8_t* lds1, int ks, int nks,
                                      int tid, int lane, int wm, int wn) {
  if (Q > 0 && ks + Q >= nks) return false;
  ps.load(Q & 1, min(ks + Q + 2, nks - 1));
  if constexpr (Q % 4 == 0) ps.load_scales((Q / 4 + 1) & 1, (ks + Q) / 4 + 1);
  mma_step<T, true>(ps, (Q & 1) ? lds1 : lds0, (Q & 1) ? lds0 : lds1, (Q + 1) & 1,
                    ((Q + 1) / 4) & 1, (Q + 1) % 4, tid, lane, wm, wn);
  lds_barrier();
  return true;
}

template <class T, int... Q>
__device__ __forceinline__ void ksteps8(Pass<T>& ps, uint8_t* lds0, uint8_t* lds1, int ks, int nks,
                                        int tid, int lane, int wm, int wn,
                                        std::integer_sequence<int, Q...>) {
  (kstep<T, Q>(ps, lds0, lds1, ks, nks, tid, lane, wm, wn) && ...);
}

// Per-thread staging offsets for rows of Kp packed bytes and Ks scale bytes.
template <class T>
__device__ __forceinline__ void init_offsets(Pass<T>& ps, int tid, uint32_t Kp, uint32_t Ks) {
#pragma unroll
  for (int u = 0; u < T::A_UNITS; ++u) {
    const int g = tid + u * T::THREADS;
    ps.a_off[u] = off::fp4_code_voff(g, Kp);
    ps.as_off[u] = off::fp4_scale_row_off(g, Ks);
  }
#pragma unroll
  for (int u = 0; u < T::B_UNITS; ++u) {
    const int g = tid + u * T::THREADS;
    ps.b_off[u] = off::fp4_code_voff(g, Kp);
    ps.bs_off[u] = off::fp4_scale_row_off(g, Ks);
  }
}

// The K loop of one pass (buffer resources and offsets set, accumulators
// zeroed): prologue staging of step 0, then eight steps per iteration
// (register set, LDS stage and scale group positions known at compile
// time).  The last step also stages (a reload, into the stage nobody reads
// any more).
template <class T>
__device__ __forceinline__ void k_loop(Pass<T>& ps, uint8_t* lds0, uint8_t* lds1, int nks, int tid,
                                       int lane, int wm, int wn) {
  ps.load(0, 0);
  ps.load(1, min(1, nks - 1));
  ps.load_scales(0, 0);
  ps.stage_all(0, 0, 0, lds0, tid);
  lds_barrier();
  for (int ks = 0; ks < nks; ks += 8)
    ksteps8<T>(ps, lds0, lds1, ks, nks, tid, lane, wm, wn, std::make_integer_sequence<int, 8>{});
}

// `alphas` (may be null): one factor per expert, alpha[g] = gA * gB[g],
// replacing the single `alpha` (a global scale per expert's B, the
// per-group scaling of the cutlass#3124 page's grouped block-scaled GEMM).
template <class T>
__global__ __launch_bounds__(T::THREADS) void fp4_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ a_scale, const uint8_t* __restrict__ b_scale,
    const int32_t* __restrict__ m_indices, float alpha, const float* __restrict__ alphas,
    uint16_t* __restrict__ C, int M, int N, int K, int G, int num_windows, int num_ntiles,
    int total_tiles, int group_w, int split) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[T::STAGE];
  __shared__ int ids[T::BM];
  __shared__ uint32_t plan_bits[kPlanWords];
  __shared__ int plan_heavy;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WAVES_N;
  const int wn = wave % T::WAVES_N;
  const int nks = K / T::BK;
  const uint32_t Kp = (uint32_t)K >> 1;  // packed bytes per row
  const uint32_t Ks = (uint32_t)K >> 4;  // scale bytes per row

  Pass<T> ps;
  init_offsets(ps, tid, Kp, Ks);

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

    for (int c = tid; c < T::BM * (T::BN / 8); c += T::THREADS) {
      const int r = c / (T::BN / 8);
      const int cc = c % (T::BN / 8);
      const int col = col0 + cc * 8;
      if (ids[r] == -1 && col < N && run_sel == 0)
        *reinterpret_cast<uint4*>(C + (size_t)(row0 + r) * N + col) = make_uint4(0, 0, 0, 0);
    }

    // Rows (A) and columns (B) of this tile that exist: loads past them read
    // zeros, and those rows / columns are never stored.
    const uint32_t rows_a = (uint32_t)min(T::BM, M - row0);
    const uint32_t rows_b = (uint32_t)min(T::BN, N - col0);
    ps.ra = rsrc(A + (size_t)row0 * Kp, rows_a * Kp);
    ps.rsa = rsrc(a_scale + (size_t)row0 * Ks, rows_a * Ks);
    const int wcol0 = col0 + wn * T::WN;

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

#pragma unroll
      for (int u = 0; u < T::A_UNITS; ++u) {
        const bool need = ids[(tid + u * T::THREADS) >> 1] == e;
        ps.pa_off[u] = need ? ps.a_off[u] : kSkip;
        ps.pas_off[u] = need ? ps.as_off[u] : kSkip;
      }
      ps.rb = rsrc(B + ((size_t)e * N + col0) * Kp, rows_b * Kp);
      ps.rsb = rsrc(b_scale + ((size_t)e * N + col0) * Ks, rows_b * Ks);
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) ps.acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

      k_loop(ps, lds0, lds1, nks, tid, lane, wm, wn);

      const float al = alphas ? alphas[e] : alpha;
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
                pack_bf16x4(al * ps.acc[i][j][0], al * ps.acc[i][j][1], al * ps.acc[i][j][2],
                            al * ps.acc[i][j][3]);
        }
      }
    }
  }
}

// A batch of independent dense NVFP4 GEMMs of different shapes in one launch
// (the cutlass#3124 page's grouped block-scaled GEMM, "Intro": problems with
// their own M, N and K).  Work item t belongs to the problem whose range
// [tile_start[g], tile_start[g + 1]) holds it; inside a problem, tiles follow
// the XCD-aware map_tile order.  Every tile is one pass (no routing) with the
// problem's own K loop, offsets and alpha; rows and columns past the
// problem's M and N read zeros and are not stored.
template <class T>
__global__ __launch_bounds__(T::THREADS) void fp4_problems_kernel(const Fp4ProblemSet set,
                                                                  int group_w) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[T::STAGE];

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
    const Fp4Problem& p = set.p[g];
    const int M = p.M, N = p.N, K = p.K;
    const int nks = K / T::BK;
    const uint32_t Kp = (uint32_t)K >> 1, Ks = (uint32_t)K >> 4;
    const int num_windows = (M + T::BM - 1) / T::BM;
    const int num_ntiles = (N + T::BN - 1) / T::BN;
    const int tiles_g = set.tile_start[g + 1] - set.tile_start[g];
    int window, ntile;
    map_tile(tile - set.tile_start[g], tiles_g, num_windows, num_ntiles, group_w, window, ntile);
    const int row0 = window * T::BM;
    const int col0 = ntile * T::BN;
    const uint32_t rows_a = (uint32_t)min(T::BM, M - row0);
    const uint32_t rows_b = (uint32_t)min(T::BN, N - col0);

    __syncthreads();  // the previous tile is done with the stages
    init_offsets(ps, tid, Kp, Ks);
#pragma unroll
    for (int u = 0; u < T::A_UNITS; ++u) {
      ps.pa_off[u] = ps.a_off[u];
      ps.pas_off[u] = ps.as_off[u];
    }
    ps.ra = rsrc(p.A + (size_t)row0 * Kp, rows_a * Kp);
    ps.rsa = rsrc(p.a_scale + (size_t)row0 * Ks, rows_a * Ks);
    ps.rb = rsrc(p.B + (size_t)col0 * Kp, rows_b * Kp);
    ps.rsb = rsrc(p.b_scale + (size_t)col0 * Ks, rows_b * Ks);
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j) ps.acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    k_loop(ps, lds0, lds1, nks, tid, lane, wm, wn);

    const float al = p.alpha;
    const int wcol0 = col0 + wn * T::WN;
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
      const int gr = row0 + wm * T::WM + i * 16 + (lane & 15);
      if (gr >= M) continue;
      uint16_t* crow = p.C + (size_t)gr * N;
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        const int n = wcol0 + j * 16 + 4 * (lane >> 4);
        if (n < N)
          *reinterpret_cast<uint2*>(crow + n) =
              pack_bf16x4(al * ps.acc[i][j][0], al * ps.acc[i][j][1], al * ps.acc[i][j][2],
                          al * ps.acc[i][j][3]);
      }
    }
  }
}

using Cfg0 = Fp4Cfg<256, 256, 4, 2>;  // 8 waves, 64x128 per wave, 128 KB LDS
using Cfg1 = Fp4Cfg<256, 128, 4, 1>;  // 4 waves, 64x128 per wave,  96 KB LDS
using Cfg2 = Fp4Cfg<128, 256, 2, 2>;  // 4 waves, 64x128 per wave,  96 KB LDS
using Cfg3 = Fp4Cfg<128, 128, 2, 2>;  // 4 waves, 64x64 per wave,   64 KB LDS

// `tput`: relative per-CU throughput, measured on MI355X by timing every
// shape on an 8192 x 8192 x 4096 dense problem that each tiles into whole
// waves: 1185, 956, 979 and 1022 TFLOPS (the 128x128 shape runs two
// workgroups per CU).
const TileCfg kFp4Tiles[] = {
    {0, 256, 256, 8, 1, 1.00f},
    {1, 256, 128, 4, 1, 0.81f},
    {2, 128, 256, 4, 1, 0.83f},
    {3, 128, 128, 4, 2, 0.86f},
};

template <class T>
hipError_t launch_cfg(const Fp4Args& a, const LaunchOpts& o, hipStream_t s) {
  const int num_windows = (a.M + T::BM - 1) / T::BM;
  const int num_ntiles = (a.N + T::BN - 1) / T::BN;
  const long long total = (long long)num_windows * num_ntiles;
  if (total <= 0) return hipSuccess;
  if (total > INT_MAX) return hipErrorInvalidValue;
  const int split = split_items(o.run_split, a.m_indices != nullptr, a.G, T::BM, total, o.num_cus);
  int grid = (int)(total * split);
  if (o.max_wg > 0 && o.max_wg < grid) grid = o.max_wg;
  const int group_w = 8;  // row windows per XCD tile group
  hipLaunchKernelGGL(fp4_gemm_kernel<T>, dim3(grid), dim3(T::THREADS), 0, s, a.A, a.B, a.a_scale,
                     a.b_scale, a.m_indices, a.alpha, a.alphas, a.C, a.M, a.N, a.K, a.G,
                     num_windows, num_ntiles, (int)total, group_w, split);
  return hipGetLastError();
}

// Tile ranges of a problem batch for tile shape BM x BN.
inline long long problem_tiles(Fp4ProblemSet& set, int BM, int BN) {
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
hipError_t launch_problems_cfg(Fp4ProblemSet set, const LaunchOpts& o, hipStream_t s) {
  const long long total = problem_tiles(set, T::BM, T::BN);
  if (total < 0) return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  int grid = (int)total;
  if (o.max_wg > 0 && o.max_wg < grid) grid = o.max_wg;
  hipLaunchKernelGGL(fp4_problems_kernel<T>, dim3(grid), dim3(T::THREADS), 0, s, set, 8);
  return hipGetLastError();
}

}  // namespace fp4_detail

using namespace fp4_detail;

int fp4_num_tiles() { return (int)(sizeof(kFp4Tiles) / sizeof(kFp4Tiles[0])); }
const TileCfg& fp4_tile(int id) { return kFp4Tiles[id]; }

hipError_t launch_fp4_problems(const Fp4ProblemSet& in, int tile_id, const LaunchOpts& o,
                               hipStream_t s) {
  if (in.count < 1 || in.count > kMaxProblems) return hipErrorInvalidValue;
  // Longest K loops first (the order of the problems does not change any
  // result): workgroups that draw the short tiles last even out the finish.
  Fp4ProblemSet set = in;
  std::stable_sort(set.p, set.p + set.count,
                   [](const Fp4Problem& a, const Fp4Problem& b) { return a.K > b.K; });
  switch (tile_id) {
    case 0: return launch_problems_cfg<Cfg0>(set, o, s);
    case 1: return launch_problems_cfg<Cfg1>(set, o, s);
    case 2: return launch_problems_cfg<Cfg2>(set, o, s);
    case 3: return launch_problems_cfg<Cfg3>(set, o, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fp4(const Fp4Args& a, int tile_id, const LaunchOpts& o, hipStream_t s) {
  switch (tile_id) {
    case 0: return launch_cfg<Cfg0>(a, o, s);
    case 1: return launch_cfg<Cfg1>(a, o, s);
    case 2: return launch_cfg<Cfg2>(a, o, s);
    case 3: return launch_cfg<Cfg3>(a, o, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fgg
