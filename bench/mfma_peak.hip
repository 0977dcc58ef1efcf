// Roofline microbenchmarks for MI355X (gfx950): the denominators and the
// per-instruction limits that the GEMM kernels of this repository are
// measured against.
//
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature \
//         -Xclang -packed-fp32-ops -mllvm -amdgpu-mfma-vgpr-form \
//         bench/mfma_peak.hip -o bench/mfma_peak
//   bench/mfma_peak            (prints a text summary)
//
// Legs:
//  1. MFMA issue rate of the matrix instructions the kernels use (FP8 with
//     unit E8M0 scales, 16x16x128 and 32x32x64; FP16 16x16x32 and 32x32x16),
//     each wave issuing independent accumulator chains back to back, one or
//     two waves per SIMD on every CU.  Cycles per MFMA per SIMD come from the
//     shader clock (s_memtime) and the clock frequency from the same interval
//     on the 100 MHz constant clock (s_memrealtime); PFLOP/s from HIP events.
//  2. LDS read bandwidth: conflict-free 16-byte reads (8 in flight per lane)
//     with 4, 8 and 16 waves per CU, bytes per clock per CU.
//  3. MFMA + LDS in the shape of the grouped FP8 GEMM's inner loop: a
//     64 x 128 wave tile, 16x16x128 FP8 MFMAs, fragments read from LDS, 8
//     waves per CU, with parts switched on one at a time (reads, per-step
//     barrier, per-K-block FP32 promotion), cycles per K step of 128.
//  4. HBM: a device-to-device copy of 1 GiB with 16-byte loads and stores.
//  5. L2 -> LDS staging: the A and B tile rows of the grouped FP8 MoE
//     prefill shape streamed through LDS rings of different depth and K
//     width with direct-to-LDS loads, no compute (loads alone), plus the
//     same stream with every load an L2 hit.
//  6. HBM read only: 1 GiB streamed with 16-byte loads, 4 or 8 in flight per
//     lane, nothing written but one word per thread (the ceiling of kernels
//     that mostly read, such as the decode GEMM and the quantisers).
//  7. Launch floor and dependent-load latency: an empty kernel, and one
//     thread running a chain of n dependent 4-byte loads (scalar or vector)
//     from a 256 KB table (cache-resident after the first launch) before one
//     store, each captured
//     100 times in a HIP graph (and also launched 100 times on a stream),
//     microseconds per launch; the slope over n is one load round trip.
//
// Every launch below is sized on the host: grids are whole multiples of the
// work each workgroup owns, and every LDS and global index is masked into
// its buffer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                        \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) {                                                             \
      std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      std::exit(1);                                                                     \
    }                                                                                   \
  } while (0)

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------ 1. issue rate
enum Shape { F8_16x16x128 = 0, F8_32x32x64 = 1, F16_16x16x32 = 2, F16_32x32x16 = 3, F4_16x16x128 = 4 };
constexpr int kChains = 8;

template <int S>
struct Acc;
template <> struct Acc<F8_16x16x128> { typedef f32x4 T; static constexpr double flop = 2.0 * 16 * 16 * 128; };
template <> struct Acc<F8_32x32x64> { typedef f32x16 T; static constexpr double flop = 2.0 * 32 * 32 * 64; };
template <> struct Acc<F16_16x16x32> { typedef f32x4 T; static constexpr double flop = 2.0 * 16 * 16 * 32; };
template <> struct Acc<F16_32x32x16> { typedef f32x16 T; static constexpr double flop = 2.0 * 32 * 32 * 16; };
template <> struct Acc<F4_16x16x128> { typedef f32x4 T; static constexpr double flop = 2.0 * 16 * 16 * 128; };

template <int S>
__device__ __forceinline__ typename Acc<S>::T mfma(typename Acc<S>::T c, i32x8 a8, f16x8 a16) {
  if constexpr (S == F8_16x16x128)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, a8, c, 0, 0, 0, 127, 0, 127);
  else if constexpr (S == F8_32x32x64)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, c, 0, 0, 0, 127, 0, 127);
  else if constexpr (S == F4_16x16x128)  // E2M1 x E2M1 (format code 4), unit scales
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, a8, c, 4, 4, 0, 127, 0, 127);
  else if constexpr (S == F16_16x16x32)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a16, a16, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a16, a16, c, 0, 0, 0);
}

// Each wave: kChains independent accumulators, `iters` rounds of one MFMA
// per chain.  Inputs are small normal values (FP8 0x30 = 0.5, FP16 0.25).
// out[tid] keeps the sums alive; cyc[wave] = shader cycles, rt[wave] =
// 100 MHz ticks over the loop.
template <int S>
__global__ __launch_bounds__(512) void mfma_rate(float* out, long long* cyc, long long* rt,
                                                  int iters) {
  typedef typename Acc<S>::T T;
  T acc[kChains];
  for (int c = 0; c < kChains; ++c) acc[c] = T{} ;
  const i32x8 a8 = {0x30303030, 0x30303030, 0x30303030, 0x30303030,
                    0x30303030, 0x30303030, 0x30303030, 0x30303030};
  f16x8 a16;
  for (int i = 0; i < 8; ++i) a16[i] = (_Float16)0.25f;
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = mfma<S>(acc[c], a8, a16);
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int c = 0; c < kChains; ++c) s += acc[c][0];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) {
    const int w = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    cyc[w] = t1 - t0;
    rt[w] = r1 - r0;
  }
}

struct RateResult {
  double cyc_per_mfma, ghz, pflops;
};

template <int S>
RateResult run_rate(int cus, int waves_per_simd) {
  const int threads = 256 * waves_per_simd;  // 4 SIMDs x waves_per_simd
  const int iters = 4000;
  const int nw = cus * threads / 64;
  float* out;
  long long *cyc, *rt;
  CHECK(hipMalloc(&out, sizeof(float) * cus * threads));
  CHECK(hipMalloc(&cyc, sizeof(long long) * nw));
  CHECK(hipMalloc(&rt, sizeof(long long) * nw));
  hipLaunchKernelGGL(mfma_rate<S>, dim3(cus), dim3(threads), 0, 0, out, cyc, rt, 200);  // warm-up
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0, 0));
  hipLaunchKernelGGL(mfma_rate<S>, dim3(cus), dim3(threads), 0, 0, out, cyc, rt, iters);
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  std::vector<long long> c(nw), r(nw);
  CHECK(hipMemcpy(c.data(), cyc, sizeof(long long) * nw, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(r.data(), rt, sizeof(long long) * nw, hipMemcpyDeviceToHost));
  double cs = 0, rs = 0;
  for (int i = 0; i < nw; ++i) cs += (double)c[i], rs += (double)r[i];
  RateResult res;
  // per SIMD: waves_per_simd waves each issue iters x kChains MFMAs
  res.cyc_per_mfma = cs / nw / ((double)iters * kChains * waves_per_simd);
  res.ghz = cs / rs * 0.1;  // shader cycles per 10 ns tick
  res.pflops = Acc<S>::flop * (double)iters * kChains * nw / (ms * 1e-3) / 1e15;
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  CHECK(hipFree(rt));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return res;
}

// ------------------------------------------------------- 2. LDS bandwidth
constexpr int kLdsBytes = 96 * 1024;  // one workgroup per CU (LDS is 160 KB)

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void lds_read(unsigned* out, long long* cyc, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  const int tid = threadIdx.x;
  for (int i = tid * 16; i < kLdsBytes; i += 64 * WAVES * 16)
    *reinterpret_cast<i32x4*>(lds + i) = (i32x4){i, i + 1, i + 2, i + 3};
  __syncthreads();
  // lane l of wave w reads 16 bytes at (w * 8 + u) KB + 16 l: each read of
  // a wave covers 1 KB of consecutive bytes (conflict-free)
  const int lane = tid & 63, wave = tid >> 6;
  i32x4 x = {0, 0, 0, 0};
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    i32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int off = (((wave * 8 + u + it) * 1024) % kLdsBytes) + lane * 16;
      v[u] = *reinterpret_cast<const i32x4*>(lds + off);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u];
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  out[blockIdx.x * blockDim.x + tid] = (unsigned)(x[0] ^ x[1] ^ x[2] ^ x[3]);
  if (tid == 0) cyc[blockIdx.x] = t1 - t0;
}

template <int WAVES>
double run_lds(int cus) {
  const int iters = 2000;
  unsigned* out;
  long long* cyc;
  CHECK(hipMalloc(&out, sizeof(unsigned) * cus * 64 * WAVES));
  CHECK(hipMalloc(&cyc, sizeof(long long) * cus));
  hipLaunchKernelGGL(lds_read<WAVES>, dim3(cus), dim3(64 * WAVES), 0, 0, out, cyc, 100);
  hipLaunchKernelGGL(lds_read<WAVES>, dim3(cus), dim3(64 * WAVES), 0, 0, out, cyc, iters);
  CHECK(hipDeviceSynchronize());
  std::vector<long long> c(cus);
  CHECK(hipMemcpy(c.data(), cyc, sizeof(long long) * cus, hipMemcpyDeviceToHost));
  double cs = 0;
  for (long long v : c) cs += (double)v;
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  // bytes read per CU over the loop, per shader cycle
  return (double)iters * 8 * 1024 * WAVES / (cs / cus);
}

// ------------------------------------------------ 3. MFMA + LDS, GEMM loop
// One workgroup per CU, 8 waves (4 x 2), wave tile 64 x 128 = 4 x 8
// subtiles of 16 x 16; a 256 x 256 x 128 stage of FP8 codes sits in LDS
// (64 KB: A rows then B rows, 128 bytes each, XOR-swizzled 16-byte chunks).
// Per K step each wave reads its 4 A fragments and 8 B fragments (two
// 16-byte reads each) and issues 32 MFMAs.  MODE bits:
//   1: fragments read from LDS every step (else read once, before the loop)
//   2: s_barrier at the end of every step
//   4: per-K-block promotion acc += partial * s (else the MFMA accumulates)
constexpr int kStage = 256 * 128 * 2;

__device__ __forceinline__ int swz(int r, int c) { return (r << 7) | ((c ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ i32x8 frag(const unsigned char* tile, int row0, int lane) {
  const int r = row0 + (lane & 15), q = lane >> 4;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(tile + swz(r, 2 * q));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(tile + swz(r, 2 * q + 1));
  return (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int MODE>
__global__ __launch_bounds__(512) void gemm_loop(float* out, long long* cyc, int steps) {
  // 96 KB allocated (64 KB used) so that one workgroup runs per CU
  __shared__ __attribute__((aligned(1024))) unsigned char st[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / 2, wn = wave % 2;
  // FP8 codes: a fixed pattern, or (MODE & 8) pseudo-random finite codes
  // (bit 3 of every byte cleared, so never 0x7F / 0xFF)
  for (int i = tid * 16; i < kStage; i += 512 * 16) {
    i32x4 v = {0x30303030, 0x38383838, 0x30303030, 0x28282828};
    if constexpr (MODE & 8) {
      for (int w = 0; w < 4; ++w) {
        unsigned x = (unsigned)(i + 4 * w) * 2654435761u ^ 0x9e3779b9u;
        x ^= x >> 13;
        x *= 0x5bd1e995u;
        x ^= x >> 15;
        v[w] = (int)(x & 0xF7F7F7F7u);
      }
    }
    *reinterpret_cast<i32x4*>(st + i) = v;
  }
  __syncthreads();
  const unsigned char* A = st;
  const unsigned char* B = st + kStage / 2;
  constexpr int TM = 4, TN = 8;
  f32x4 acc[TM][TN];
  for (int i = 0; i < TM; ++i)
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  float s[TM];
  for (int i = 0; i < TM; ++i) s[i] = 1.0f + 0.001f * (lane + i);
  i32x8 af[TM], bf0, bnext;
  for (int i = 0; i < TM; ++i) af[i] = frag(A, wm * 64 + i * 16, lane);
  bf0 = frag(B, wn * 128, lane);
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int step = 0; step < steps; ++step) {
    i32x8 bf = bf0;
    // Without LDS reads the fragments would not change from column to
    // column or step to step, and with the promotion (MFMA results not
    // chained) the compiler would share and hoist the MFMAs: vary one B
    // word per step and per column block.
    if constexpr (!(MODE & 1) && (MODE & 4)) bf[0] ^= step & 1;
    if constexpr (MODE & 1) {
      bf = frag(B, wn * 128, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = frag(A, wm * 64 + i * 16, lane);
    }
    bnext = bf;
    constexpr int NT = TM * TN, LAG = 3;
    f32x4 ring[LAG + 1];
#pragma unroll
    for (int t = 0; t < NT + LAG; ++t) {
      if (t < NT) {
        const int j = t / TM, i = t % TM;
        if (i == 0) {
          if (j > 0) bf = bnext;
          if ((MODE & 1) && j + 1 < TN) bnext = frag(B, wn * 128 + (j + 1) * 16, lane);
          if (!(MODE & 1) && (MODE & 4) && j + 1 < TN) bnext[1] ^= 1 << (j + 1);
        }
        if constexpr (MODE & 4)
          ring[t % (LAG + 1)] =
              __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], zero, 0, 0, 0, 127, 0, 127);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], acc[i][j], 0, 0, 0,
                                                                       127, 0, 127);
      }
      if constexpr (MODE & 4) {
        if (t >= LAG) {
          const int u = t - LAG, j = u / TM, i = u % TM;
          acc[i][j] += ring[u % (LAG + 1)] * s[i];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MODE & 2) __builtin_amdgcn_s_barrier();
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float sum = 0.f;
  for (int i = 0; i < TM; ++i)
    for (int j = 0; j < TN; ++j) sum += acc[i][j][0] + acc[i][j][3];
  out[blockIdx.x * 512 + tid] = sum;
  if (tid == 0) cyc[blockIdx.x] = t1 - t0;
}

struct LoopResult {
  double cycles, ns;
};

// Cycles per K step of one wave (its own loop, shader clock) and wall
// nanoseconds per K step of the whole launch (HIP events): without a
// per-step barrier the two waves of a SIMD drift apart and the per-wave
// figure undercounts, so the wall figure is the one to compare.
template <int MODE>
LoopResult run_gemm_loop(int cus) {
  const int steps = 400;
  float* out;
  long long* cyc;
  CHECK(hipMalloc(&out, sizeof(float) * cus * 512));
  CHECK(hipMalloc(&cyc, sizeof(long long) * cus));
  hipLaunchKernelGGL(gemm_loop<MODE>, dim3(cus), dim3(512), 0, 0, out, cyc, 20);
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0, 0));
  hipLaunchKernelGGL(gemm_loop<MODE>, dim3(cus), dim3(512), 0, 0, out, cyc, steps);
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  std::vector<long long> c(cus);
  CHECK(hipMemcpy(c.data(), cyc, sizeof(long long) * cus, hipMemcpyDeviceToHost));
  double cs = 0;
  for (long long v : c) cs += (double)v;
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return LoopResult{cs / cus / steps, ms * 1e6 / steps};
}

// ------------------------------------------------------------------- 4. HBM
// n is a multiple of 4 x the grid's thread count (checked by the caller):
// each thread keeps four 16-byte loads in flight.
__global__ __launch_bounds__(256) void copy16(const i32x4* __restrict__ src, i32x4* __restrict__ dst,
                                              long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += 4 * stride) {
    i32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[i + u * stride] = v[u];
  }
}

double run_copy(int cus) {
  const long long bytes = 1ll << 30, n = bytes / 16;
  i32x4 *a, *b;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMemset(a, 1, bytes));
  const int grid = cus * 8;
  if (n % (4ll * grid * 256)) {
    std::fprintf(stderr, "copy size not a multiple of the grid's work\n");
    std::exit(1);
  }
  for (int i = 0; i < 3; ++i) hipLaunchKernelGGL(copy16, dim3(grid), dim3(256), 0, 0, a, b, n);
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const int reps = 10;
  CHECK(hipEventRecord(e0, 0));
  for (int i = 0; i < reps; ++i) hipLaunchKernelGGL(copy16, dim3(grid), dim3(256), 0, 0, a, b, n);
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return 2.0 * bytes * reps / (ms * 1e-3) / 1e9;  // GB/s, read + write
}

// ------------------------------------------------------- 6. HBM read only
// n is a multiple of U x the grid's thread count (checked by the caller).
template <int U>
__global__ __launch_bounds__(256) void read16(const i32x4* __restrict__ src, int* __restrict__ out,
                                              long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  i32x4 x = {0, 0, 0, 0};
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += U * stride) {
    i32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u];
  }
  out[(long long)blockIdx.x * blockDim.x + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

template <int U>
double run_read(int cus, int wg_per_cu) {
  const long long bytes = 1ll << 30, n = bytes / 16;
  const int grid = cus * wg_per_cu;
  if (n % ((long long)U * grid * 256)) {
    std::fprintf(stderr, "read size not a multiple of the grid's work\n");
    std::exit(1);
  }
  i32x4* a;
  int* out;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&out, sizeof(int) * grid * 256));
  CHECK(hipMemset(a, 1, bytes));
  for (int i = 0; i < 3; ++i) hipLaunchKernelGGL(read16<U>, dim3(grid), dim3(256), 0, 0, a, out, n);
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const int reps = 10;
  CHECK(hipEventRecord(e0, 0));
  for (int i = 0; i < reps; ++i) hipLaunchKernelGGL(read16<U>, dim3(grid), dim3(256), 0, 0, a, out, n);
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipFree(a));
  CHECK(hipFree(out));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return (double)bytes * reps / (ms * 1e-3) / 1e9;  // GB/s read
}

// ---------------------------------------- 7. launch floor, load round trip
__global__ void empty_kernel() {}

// One thread: n dependent loads (each index comes from the previous load,
// masked into the table), then one store.  VEC keeps the index in a vector
// register, so the loads take the vector memory path (L1, L2) that the
// GEMMs' loads take; otherwise the compiler, seeing a uniform index, issues
// scalar loads through the scalar cache.
template <bool VEC>
__global__ void chase(const unsigned* __restrict__ table, unsigned mask, int n,
                      unsigned* __restrict__ out) {
  unsigned i = blockIdx.x;
  for (int k = 0; k < n; ++k) {
    if (VEC) asm volatile("" : "+v"(i));
    i = table[i & mask];
  }
  out[blockIdx.x] = i;
}

// Microseconds per launch of `launch` (which enqueues one kernel on the
// given stream): 100 launches captured in a HIP graph (best of 3 replays),
// and 100 plain launches on the same stream.
template <class F>
void launch_us(F launch, double& graph_us, double& stream_us) {
  const int reps = 100;
  hipStream_t s;
  CHECK(hipStreamCreate(&s));
  hipGraph_t g;
  hipGraphExec_t ge;
  CHECK(hipStreamBeginCapture(s, hipStreamCaptureModeGlobal));
  for (int i = 0; i < reps; ++i) launch(s);
  CHECK(hipStreamEndCapture(s, &g));
  CHECK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
  CHECK(hipGraphLaunch(ge, s));
  CHECK(hipStreamSynchronize(s));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  graph_us = 1e30;
  for (int r = 0; r < 3; ++r) {
    CHECK(hipEventRecord(e0, s));
    CHECK(hipGraphLaunch(ge, s));
    CHECK(hipEventRecord(e1, s));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    graph_us = std::min(graph_us, (double)ms * 1e3 / reps);
  }
  CHECK(hipEventRecord(e0, s));
  for (int i = 0; i < reps; ++i) launch(s);
  CHECK(hipEventRecord(e1, s));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  stream_us = ms * 1e3 / reps;
  CHECK(hipGraphExecDestroy(ge));
  CHECK(hipGraphDestroy(g));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  CHECK(hipStreamDestroy(s));
}

void run_latency() {
  const unsigned len = 1u << 16, mask = len - 1;  // 256 KB table
  std::vector<unsigned> h(len);
  for (unsigned i = 0; i < len; ++i) h[i] = (i + 16411u) & mask;  // a new cache line every hop
  unsigned *table, *out;
  CHECK(hipMalloc(&table, sizeof(unsigned) * len));
  CHECK(hipMalloc(&out, sizeof(unsigned) * 64));
  CHECK(hipMemcpy(table, h.data(), sizeof(unsigned) * len, hipMemcpyHostToDevice));
  std::printf("kernel | us per launch (HIP graph) | us per launch (stream)\n");
  double gu, su;
  launch_us([](hipStream_t s) { hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s); }, gu, su);
  std::printf("empty, 1 workgroup | %.2f | %.2f\n", gu, su);
  std::fflush(stdout);
  for (int vec = 0; vec < 2; ++vec)
    for (int n : {0, 1, 2, 4, 8, 16, 32}) {
      launch_us(
          [=](hipStream_t s) {
            hipLaunchKernelGGL(vec ? chase<true> : chase<false>, dim3(1), dim3(1), 0, s,
                               (const unsigned*)table, mask, n, out);
          },
          gu, su);
      std::printf("%d dependent %s loads + 1 store | %.2f | %.2f\n", n, vec ? "vector" : "scalar",
                  gu, su);
      std::fflush(stdout);
    }
  CHECK(hipFree(table));
  CHECK(hipFree(out));
}

// --------------------------------------------- 5. L2 -> LDS tile staging
// Loads only: every workgroup (8 waves, one per CU) streams the A and B
// rows of 256 x 256 output tiles of the grouped FP8 MoE prefill shape (A
// [8192, 7168], B [8, 4096, 7168], expert e owning rows 1024 e ..), two
// tiles each, through an LDS ring of STAGES stages of BK bytes per row with
// 16-byte direct-to-LDS loads, waiting for each stage and a barrier per
// stage; no compute.  Tiles are dealt to the XCDs in contiguous ranges of
// 4 row windows x 16 column tiles, as the FP8 kernel orders them.  HIT:
// every stage reloads the first K slice (all L2 hits after the first).
constexpr int kSM = 8192, kSN = 4096, kSK = 7168, kSG = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ unsigned lds_u32(const void* p) {
  return (unsigned)(uintptr_t)(lds_ptr_t)(const_cast<void*>(p));
}
__device__ __forceinline__ i32x4 buf_rsrc(const void* base, unsigned bytes) {
  const unsigned long long a = (unsigned long long)base;
  return (i32x4){(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}
// 16 bytes per lane from VGPR offset voff (range-checked) + SGPR offset soff
// into LDS at lds + 16 lane
__device__ __forceinline__ void dma16(i32x4 rs, unsigned lds, unsigned voff, unsigned soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds),
               "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int STAGES, int BK, bool HIT>
__global__ __launch_bounds__(512) void stage_stream(const unsigned char* A, const unsigned char* B,
                                                    int* out, int tiles) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char ring[];
  constexpr int STAGE = 512 * BK;             // 256 A rows + 256 B rows
  constexpr int ROWS = 1024 / BK;             // rows per 1 KB load
  constexpr int LOADS = 512 / ROWS / 8;       // loads per wave per stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int steps = kSK / BK;
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int q = tiles / 8, r = tiles % 8, xcd = tile % 8, slot = tile / 8;
    const int logical = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
    const int grp = logical / 64, in = logical % 64;
    const int window = grp * 4 + in % 4, ntile = in / 4, e = window / 4;
    const i32x4 ra = buf_rsrc(A + (size_t)window * 256 * kSK, 256u * kSK);
    const i32x4 rb = buf_rsrc(B + ((size_t)e * kSN + ntile * 256) * kSK, 256u * kSK);
    const int rl = lane / (BK / 16), ch = lane % (BK / 16);
    auto issue = [&](int st, int k) {
#pragma unroll
      for (int s = 0; s < LOADS; ++s) {
        const int blk = s * 8 + wave;  // uniform
        const bool isa = blk * ROWS < 256;
        const int row = (isa ? blk * ROWS : blk * ROWS - 256) + rl;
        dma16(isa ? ra : rb, __builtin_amdgcn_readfirstlane(lds_u32(ring + st * STAGE + blk * 1024)),
              (unsigned)(row * kSK + ch * 16), (unsigned)((HIT ? 0 : k) * BK));
      }
    };
    __syncthreads();
    for (int k = 0; k < STAGES - 1 && k < steps; ++k) issue(k, k);
    for (int k = 0; k < steps; ++k) {
      if (k + STAGES - 1 < steps) {
        issue((k + STAGES - 1) % STAGES, k + STAGES - 1);
        vm_wait<(STAGES - 1) * LOADS>();  // stage k landed; later ones may be in flight
      } else {
        vm_wait<0>();
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  }
  if (tid == 0) out[blockIdx.x] = ring[lane];
}

template <int STAGES, int BK, bool HIT>
double run_stage(const unsigned char* A, const unsigned char* B, int* out, int cus) {
  const int tiles = 2 * cus;  // the c2 shape has 512 tiles of 256 x 256
  const size_t lds = (size_t)STAGES * 512 * BK;
  auto k = stage_stream<STAGES, BK, HIT>;
  CHECK(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  for (int i = 0; i < 3; ++i) hipLaunchKernelGGL(k, dim3(cus), dim3(512), lds, 0, A, B, out, tiles);
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const int reps = 10;
  CHECK(hipEventRecord(e0, 0));
  for (int i = 0; i < reps; ++i) hipLaunchKernelGGL(k, dim3(cus), dim3(512), lds, 0, A, B, out, tiles);
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return ms * 1e3 / reps;  // us per launch
}

// ------------------------------------------------------ 8. VALU issue rate
// Each wave: 8 independent chains of one instruction, `iters` rounds; the
// output of a round is the next round's input (a chain per register), so
// the loop measures issue throughput once the chains cover the latency.
enum ValuOp { CVT_F16_FP4 = 0, CVT_F32_FP4 = 1, PK_MUL_F16 = 2, MUL_F32 = 3, CVT_F16_FP8 = 4, CVT_BF16_F32 = 5, PERM = 6 };
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

template <int OP>
__global__ __launch_bounds__(512) void valu_rate(unsigned* out, long long* cyc, int iters) {
  unsigned w[kChains];
  for (int c = 0; c < kChains; ++c) w[c] = 0x3C003C00u + threadIdx.x * 7u + (unsigned)c;
  const f16x2v kh = {(_Float16)1.0009765625f, (_Float16)1.0009765625f};
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (OP == CVT_F16_FP4)
        w[c] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[c], 1.0f, 0));
      else if constexpr (OP == CVT_F32_FP4)
        w[c] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[c], 1.0f, 0)[0]);
      else if constexpr (OP == PK_MUL_F16)
        w[c] = __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2v, w[c]) * kh);
      else if constexpr (OP == MUL_F32)
        w[c] = __builtin_bit_cast(unsigned, __builtin_bit_cast(float, w[c]) * 1.0000001f);
      else if constexpr (OP == CVT_F16_FP8)
        w[c] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[c], 1.0f, false));
      else if constexpr (OP == CVT_BF16_F32) {  // two FP32 values -> a rounded BF16 pair
        const float f = __builtin_bit_cast(float, w[c]);
        w[c] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2v){f, f}, bf16x2v));
      } else
        w[c] = __builtin_amdgcn_perm(w[c], w[c] + 1u, 0x07060302u);
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  unsigned x = 0;
  for (int c = 0; c < kChains; ++c) x ^= w[c];
  out[blockIdx.x * blockDim.x + threadIdx.x] = x;
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = t1 - t0;
}

// Cycles per instruction per SIMD (waves_per_simd waves each issuing
// iters x kChains of them).
template <int OP>
double run_valu(int cus, int waves_per_simd) {
  const int threads = 256 * waves_per_simd;
  const int iters = 4000;
  const int nw = cus * threads / 64;
  unsigned* out;
  long long* cyc;
  CHECK(hipMalloc(&out, sizeof(unsigned) * cus * threads));
  CHECK(hipMalloc(&cyc, sizeof(long long) * nw));
  hipLaunchKernelGGL(valu_rate<OP>, dim3(cus), dim3(threads), 0, 0, out, cyc, 200);  // warm-up
  CHECK(hipDeviceSynchronize());
  hipLaunchKernelGGL(valu_rate<OP>, dim3(cus), dim3(threads), 0, 0, out, cyc, iters);
  CHECK(hipDeviceSynchronize());
  std::vector<long long> c(nw);
  CHECK(hipMemcpy(c.data(), cyc, sizeof(long long) * nw, hipMemcpyDeviceToHost));
  double cs = 0;
  for (int i = 0; i < nw; ++i) cs += (double)c[i];
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  return cs / nw / ((double)iters * kChains * waves_per_simd);
}

// ------------------------------------- 9. MFMAs with VALU work between them
// Each wave: 8 independent FP16 16x16x32 MFMA chains and, after each MFMA,
// V independent v_pk_mul_f16 on registers the MFMAs do not touch: whether
// VALU instructions issue in the shadow of the matrix pipe.
template <int V>
__global__ __launch_bounds__(512) void mfma_valu(float* out, long long* cyc, int iters) {
  f32x4 acc[kChains];
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{};
  f16x8 a16;
  for (int i = 0; i < 8; ++i) a16[i] = (_Float16)0.25f;
  f16x2v h[8];
  for (int i = 0; i < 8; ++i) h[i] = (f16x2v){(_Float16)(1.0f + 0.01f * i), (_Float16)1.0f};
  const f16x2v k = {(_Float16)1.0009765625f, (_Float16)1.0009765625f};
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a16, a16, acc[c], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < V; ++v) h[(c * V + v) & 7] = h[(c * V + v) & 7] * k;
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int c = 0; c < kChains; ++c) s += acc[c][0];
  for (int i = 0; i < 8; ++i) s += (float)h[i][0];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = t1 - t0;
}

// Cycles per MFMA per SIMD at two waves per SIMD.
template <int V>
double run_mfma_valu(int cus) {
  const int threads = 512, iters = 4000, nw = cus * threads / 64;
  float* out;
  long long* cyc;
  CHECK(hipMalloc(&out, sizeof(float) * cus * threads));
  CHECK(hipMalloc(&cyc, sizeof(long long) * nw));
  hipLaunchKernelGGL(mfma_valu<V>, dim3(cus), dim3(threads), 0, 0, out, cyc, 200);  // warm-up
  CHECK(hipDeviceSynchronize());
  hipLaunchKernelGGL(mfma_valu<V>, dim3(cus), dim3(threads), 0, 0, out, cyc, iters);
  CHECK(hipDeviceSynchronize());
  std::vector<long long> c(nw);
  CHECK(hipMemcpy(c.data(), cyc, sizeof(long long) * nw, hipMemcpyDeviceToHost));
  double cs = 0;
  for (int i = 0; i < nw; ++i) cs += (double)c[i];
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  return cs / nw / ((double)iters * kChains * 2);
}

int main() {
  hipDeviceProp_t p;
  CHECK(hipGetDeviceProperties(&p, 0));
  const int cus = p.multiProcessorCount;
  std::printf("# device %s, %d CUs, clockRate %d kHz, LDS/block %zu B\n", p.gcnArchName, cus,
              p.clockRate, (size_t)p.sharedMemPerBlock);
  std::fflush(stdout);
  const char* names[] = {"v_mfma_scale_f32_16x16x128_f8f6f4 (FP8)",
                         "v_mfma_scale_f32_32x32x64_f8f6f4 (FP8)",
                         "v_mfma_f32_16x16x32_f16", "v_mfma_f32_32x32x16_f16",
                         "v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 E2M1)"};
  std::printf("\n## 1. MFMA issue rate (8 independent chains per wave, every CU)\n");
  std::printf("instruction | waves/SIMD | cycles per MFMA per SIMD | shader clock GHz | PFLOP/s\n");
  for (int w = 1; w <= 2; ++w) {
    RateResult r[5] = {run_rate<F8_16x16x128>(cus, w), run_rate<F8_32x32x64>(cus, w),
                       run_rate<F16_16x16x32>(cus, w), run_rate<F16_32x32x16>(cus, w),
                       run_rate<F4_16x16x128>(cus, w)};
    for (int s = 0; s < 5; ++s)
      std::printf("%s | %d | %.1f | %.2f | %.2f\n", names[s], w, r[s].cyc_per_mfma, r[s].ghz,
                  r[s].pflops);
    std::fflush(stdout);
  }
  std::printf("\n## 2. LDS read bandwidth (ds_read_b128, conflict-free, 8 in flight per lane)\n");
  std::printf("waves per CU | bytes per clock per CU\n");
  std::printf("4 | %.1f\n8 | %.1f\n16 | %.1f\n", run_lds<4>(cus), run_lds<8>(cus), run_lds<16>(cus));
  std::fflush(stdout);
  std::printf("\n## 3. FP8 GEMM inner loop: 8 waves, 64x128 per wave, 32 MFMAs 16x16x128 per K step\n");
  std::printf("(MFMA-only limit per K step: 2 waves x 32 MFMAs x 32 cycles = 2048 cycles per SIMD)\n");
  std::printf("variant | cycles per K step (per wave) | ns per K step (wall)\n");
  auto row = [](const char* name, LoopResult r) {
    std::printf("%s | %.0f | %.0f\n", name, r.cycles, r.ns);
    std::fflush(stdout);
  };
  row("MFMA only (fragments in registers)", run_gemm_loop<0>(cus));
  row("+ promotion FMAs", run_gemm_loop<4>(cus));
  row("+ LDS fragment reads", run_gemm_loop<1>(cus));
  row("+ LDS reads + barrier", run_gemm_loop<3>(cus));
  row("+ LDS reads + barrier + promotion", run_gemm_loop<7>(cus));
  row("+ LDS reads + promotion (no barrier)", run_gemm_loop<5>(cus));
  row("MFMA only, random FP8 operands", run_gemm_loop<8>(cus));
  row("+ LDS reads + barrier + promotion, random FP8 operands", run_gemm_loop<15>(cus));
  std::printf("\n## 4. HBM copy, 1 GiB, 16-byte loads/stores\n");
  std::printf("GB/s (read + write) | %.0f\n", run_copy(cus));
  std::fflush(stdout);

  std::printf("\n## 6. HBM read only, 1 GiB, 16-byte loads\n");
  std::printf("loads in flight per lane | workgroups (256 threads) per CU | GB/s\n");
  std::printf("4 | 8 | %.0f\n", run_read<4>(cus, 8));
  std::printf("8 | 8 | %.0f\n", run_read<8>(cus, 8));
  std::printf("4 | 16 | %.0f\n", run_read<4>(cus, 16));
  std::fflush(stdout);
  std::printf("\n## 7. Launch floor and dependent-load round trip (100 launches)\n");
  run_latency();

  std::printf("\n## 8. VALU issue rate (8 independent chains per wave, every CU)\n");
  std::printf("instruction | cycles per instruction per SIMD, 1 wave/SIMD | 2 waves/SIMD\n");
  auto vrow = [](const char* name, double a, double b) {
    std::printf("%s | %.1f | %.1f\n", name, a, b);
    std::fflush(stdout);
  };
  vrow("v_cvt_scalef32_pk_f16_fp4", run_valu<CVT_F16_FP4>(cus, 1), run_valu<CVT_F16_FP4>(cus, 2));
  vrow("v_cvt_scalef32_pk_f32_fp4", run_valu<CVT_F32_FP4>(cus, 1), run_valu<CVT_F32_FP4>(cus, 2));
  vrow("v_cvt_scalef32_pk_f16_fp8", run_valu<CVT_F16_FP8>(cus, 1), run_valu<CVT_F16_FP8>(cus, 2));
  vrow("v_pk_mul_f16", run_valu<PK_MUL_F16>(cus, 1), run_valu<PK_MUL_F16>(cus, 2));
  vrow("v_mul_f32", run_valu<MUL_F32>(cus, 1), run_valu<MUL_F32>(cus, 2));
  vrow("v_cvt_pk_bf16_f32", run_valu<CVT_BF16_F32>(cus, 1), run_valu<CVT_BF16_F32>(cus, 2));
  vrow("v_perm_b32 (+ v_add_u32)", run_valu<PERM>(cus, 1), run_valu<PERM>(cus, 2));

  std::printf("\n## 9. FP16 MFMAs with independent VALU work between them (2 waves/SIMD)\n");
  std::printf("v_pk_mul_f16 per MFMA | cycles per MFMA per SIMD\n");
  std::printf("0 | %.1f\n", run_mfma_valu<0>(cus));
  std::printf("1 | %.1f\n", run_mfma_valu<1>(cus));
  std::printf("2 | %.1f\n", run_mfma_valu<2>(cus));
  std::printf("3 | %.1f\n", run_mfma_valu<3>(cus));
  std::printf("4 | %.1f\n", run_mfma_valu<4>(cus));
  std::fflush(stdout);

  std::printf("\n## 5. L2 -> LDS staging of 256x256 tiles (loads only), grouped FP8 MoE prefill shape\n");
  std::printf("(2 tiles per CU x 56 K steps of 128; 64 KB per step per CU)\n");
  if (cus != 256) {
    std::printf("skipped: written for 256 CUs\n");
    return 0;
  }
  unsigned char *A, *B;
  int* out;
  CHECK(hipMalloc(&A, (size_t)kSM * kSK));
  CHECK(hipMalloc(&B, (size_t)kSG * kSN * kSK));
  CHECK(hipMalloc(&out, sizeof(int) * cus));
  CHECK(hipMemset(A, 0x38, (size_t)kSM * kSK));
  CHECK(hipMemset(B, 0x38, (size_t)kSG * kSN * kSK));
  std::printf("ring | us per launch | ns per K step of 128 | bytes per ns per CU\n");
  auto srow = [&](const char* name, double us) {
    const double ns = us * 1e3 / 112.0;
    std::printf("%s | %.1f | %.0f | %.1f\n", name, us, ns, 65536.0 / ns);
    std::fflush(stdout);
  };
  srow("2 stages x 64 KB (BK 128)", run_stage<2, 128, false>(A, B, out, cus));
  srow("2 stages x 64 KB (BK 128), every load an L2 hit", run_stage<2, 128, true>(A, B, out, cus));
  srow("2 stages x 32 KB (BK 64)", run_stage<2, 64, false>(A, B, out, cus));
  srow("4 stages x 32 KB (BK 64)", run_stage<4, 64, false>(A, B, out, cus));
  srow("4 stages x 32 KB (BK 64), every load an L2 hit", run_stage<4, 64, true>(A, B, out, cus));
  CHECK(hipFree(A));
  CHECK(hipFree(B));
  CHECK(hipFree(out));
  return 0;
}
