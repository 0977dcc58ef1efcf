// LDS bank-conflict probe for gfx950: which lanes of a wave a 16-byte LDS
// read (ds_read_b128) serves together, and whether the FP8 kernel's
// fragment reads are free of conflicts.
//
// Each pattern gives every lane a 16-byte address in one 16 KB quarter of a
// 64 KB LDS buffer; the kernel repeats ds_read_b128 at those addresses (four
// quarters per iteration).  The program prints the pattern names in launch
// order; the counts come from the profiler:
//
//   rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS
//             --output-format csv -d <out> -o b -- bench/lds_banks
//
// For each pattern (the second of its two launches), LDS cycles per read =
// SQ_LDS_IDX_ACTIVE / reads and conflict cycles per read =
// SQ_LDS_BANK_CONFLICT / reads, where reads = SQ_INSTS_LDS minus the 16384
// stores that fill the buffer.  4 cycles per read is conflict-free.
//
// Patterns "slot bits abcd": lane l reads 16-byte slot (bits a, b, c, d of
// l) of a 256-byte line (line l).  A slot pattern is conflict-free exactly
// when the lanes served in one cycle see 16 distinct slots, so the set of
// conflict-free bit choices fixes the grouping.  "fragment ... key" patterns
// are the FP8 kernel's fragment reads (rows r0 + l % 16, chunk 2 (l / 16) or
// 2 (l / 16) + 1, 128-byte rows) under the old swizzle key (row bits 1..3)
// and the kept one (row bit 1, row bit 2, row bits 2 ^ 3).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

typedef int i32x4 __attribute__((ext_vector_type(4)));
#define CHECK(x)                                                                \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                             \
    }                                                                           \
  } while (0)

constexpr int kLds = 65536, kQuarter = 16384, kThreads = 256;

__global__ __launch_bounds__(kThreads) void reads(const int* __restrict__ table, int* out,
                                                  int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid * 16; i < kLds; i += kThreads * 16)
    *reinterpret_cast<i32x4*>(lds + i) = (i32x4){i, i + 1, i + 2, i + 3};
  __syncthreads();
  int o = table[lane];  // below kQuarter, 16-byte aligned (checked on the host)
  i32x4 x = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(o));  // keeps the reads inside the loop
    i32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const i32x4*>(lds + o + u * kQuarter);
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= v[u];
  }
  out[blockIdx.x * kThreads + tid] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

static int key_old(int r) { return (r >> 1) & 7; }
static int key_new(int r) {
  return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 2);
}

int main() {
  std::vector<std::pair<std::string, std::vector<int>>> pats;
  auto add = [&](const std::string& n, auto f) {
    std::vector<int> t(64);
    for (int l = 0; l < 64; ++l) t[l] = f(l);
    pats.push_back({n, t});
  };
  add("contiguous 1 KB (16 l)", [](int l) { return 16 * l; });
  for (int a = 0; a < 6; ++a)
    for (int b = a + 1; b < 6; ++b)
      for (int c = b + 1; c < 6; ++c)
        for (int d = c + 1; d < 6; ++d) {
          char n[32];
          std::snprintf(n, sizeof n, "slot bits %d%d%d%d", a, b, c, d);
          add(n, [=](int l) {
            const int s = ((l >> a) & 1) | (((l >> b) & 1) << 1) | (((l >> c) & 1) << 2) |
                          (((l >> d) & 1) << 3);
            return l * 256 + s * 16;
          });
        }
  for (int half = 0; half < 2; ++half) {
    add(std::string("fragment, old key, chunk ") + (half ? "2q+1" : "2q"), [=](int l) {
      const int r = 16 + (l & 15), c = 2 * (l >> 4) + half;
      return (r << 7) | ((c ^ key_old(r)) << 4);
    });
    add(std::string("fragment, kept key, chunk ") + (half ? "2q+1" : "2q"), [=](int l) {
      const int r = 16 + (l & 15), c = 2 * (l >> 4) + half;
      return (r << 7) | ((c ^ key_new(r)) << 4);
    });
  }
  int *dt, *dout;
  CHECK(hipMalloc(&dt, 64 * sizeof(int)));
  CHECK(hipMalloc(&dout, 256 * kThreads * sizeof(int)));
  for (auto& p : pats) {
    for (int v : p.second)
      if (v < 0 || v + 16 > kQuarter || (v & 15)) {
        std::printf("pattern %s leaves its quarter\n", p.first.c_str());
        return 1;
      }
    CHECK(hipMemcpy(dt, p.second.data(), 64 * sizeof(int), hipMemcpyHostToDevice));
    hipLaunchKernelGGL(reads, dim3(256), dim3(kThreads), 0, 0, dt, dout, 100);
    hipLaunchKernelGGL(reads, dim3(256), dim3(kThreads), 0, 0, dt, dout, 2000);
    CHECK(hipDeviceSynchronize());
    std::printf("%s\n", p.first.c_str());
  }
  CHECK(hipFree(dt));
  CHECK(hipFree(dout));
  return 0;
}
