// C ABI of the block-scaled GEMM library: argument validation, device facts,
// the tile ranker and dispatch.  Declared in include/fgg.h.
//
// Validation follows the pattern of the flashinfer#7877 page's host binding
// ("Code analysis 1"): every check names the entry point and the violated
// condition (K a multiple of 128, 16-byte aligned addresses and strides,
// 1 <= M <= 2^24, 64 <= N <= 2^19 from the launch contract in "Code analysis
// 2"); here a failed check returns a status and sets a per-thread message
// instead of raising.  The device check caches gcnArchName once per device,
// the runtime detection pattern of the sglang#27745 page ("Code analysis 1").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <map>
#include <mutex>
#include <tuple>
#include <string>
#include <vector>

#include "../../include/fgg.h"
#include "common.h"

namespace {

thread_local std::string g_err;

fgg_status fail(fgg_status st, const char* fn, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = std::string(fn) + ": " + buf;
  return st;
}

struct DeviceFacts {
  bool probed = false;
  bool ok = false;
  int num_cus = 0;
  int lds = 0;
  int clock_khz = 0;
  char arch[64] = {0};
  std::string err;
};

std::mutex g_dev_mu;
std::vector<DeviceFacts> g_devs;

// Facts of the current device, probed once.  Returns nullptr and sets the
// message when no gfx950 device is current.
const DeviceFacts* current_device(const char* fn, fgg_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    *st = fail(FGG_EDEVICE, fn, "no HIP device available (%s)", hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_devs.size() <= dev) g_devs.resize(dev + 1);
  DeviceFacts& f = g_devs[dev];
  if (!f.probed) {
    f.probed = true;
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) {
      f.err = std::string("hipGetDeviceProperties failed: ") + hipGetErrorString(e);
    } else {
      std::snprintf(f.arch, sizeof(f.arch), "%s", p.gcnArchName);
      f.num_cus = p.multiProcessorCount;
      f.lds = (int)p.sharedMemPerBlock;
      f.clock_khz = p.clockRate;
      f.ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
      if (!f.ok) f.err = std::string("device architecture is ") + p.gcnArchName + ", need gfx950";
    }
  }
  if (!f.ok) {
    *st = fail(FGG_EDEVICE, fn, "%s", f.err.c_str());
    return nullptr;
  }
  return &f;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape and pointer checks shared by every entry point.  Pure host logic.
// `k_unit` is the K divisibility the format itself needs (128 for FP8's
// 1x128 / 128x128 scale blocks, 16 for NVFP4's scale blocks): violating it
// is FGG_EINVAL.  Shapes inside the method's limits that this library does
// not implement (N % 128 != 0: partial b_scale blocks; NVFP4 K % 128 != 0)
// are FGG_EUNSUPPORTED.
fgg_status check_common(const char* fn, const void* A, const void* B, const void* sa,
                        const void* sb, const void* C, int M, int N, int K, int G,
                        bool grouped, const void* m_indices, uintptr_t scale_align,
                        int k_unit = 128) {
  if (!A || !B || !sa || !sb || !C) return fail(FGG_EINVAL, fn, "null pointer among A, B, a_scale, b_scale, C");
  if (grouped && !m_indices) return fail(FGG_EINVAL, fn, "m_indices is null");
  if (M < 1 || M > (1 << 24)) return fail(FGG_EINVAL, fn, "requires 1 <= M <= 2^24, got M=%d", M);
  if (N < 64 || N > (1 << 19)) return fail(FGG_EINVAL, fn, "requires 64 <= N <= 2^19, got N=%d", N);
  if (N % 64) return fail(FGG_EINVAL, fn, "requires N %% 64 == 0, got N=%d", N);
  if (K < k_unit || K > (1 << 20)) return fail(FGG_EINVAL, fn, "requires %d <= K <= 2^20, got K=%d", k_unit, K);
  if (K % k_unit) return fail(FGG_EINVAL, fn, "requires K %% %d == 0, got K=%d", k_unit, K);
  if (G < 1 || G > (1 << 16)) return fail(FGG_EINVAL, fn, "requires 1 <= G <= 2^16, got G=%d", G);
  if (N % 128)
    return fail(FGG_EUNSUPPORTED, fn, "N %% 128 != 0 (N=%d) is not supported: whole 128-column blocks only", N);
  if (K % 128)
    return fail(FGG_EUNSUPPORTED, fn, "K %% 128 != 0 (K=%d) is not supported: whole 128-wide K steps only", K);
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16))
    return fail(FGG_EALIGN, fn, "A, B and C must be 16-byte aligned");
  if (!aligned(sa, scale_align) || !aligned(sb, scale_align))
    return fail(FGG_EALIGN, fn, "a_scale and b_scale must be %d-byte aligned", (int)scale_align);
  if (grouped && !aligned(m_indices, 4)) return fail(FGG_EALIGN, fn, "m_indices must be 4-byte aligned");
  return FGG_OK;
}

// ------------------------------------------------------------------ ranker
// Time of `tiles` tiles on `slots` workgroup slots, in rounds of full-slot
// time.  A partly filled last round, with a fraction f of the slots busy,
// costs about kPartialRound + (1 - kPartialRound) f of a full round: its
// workgroups run little faster than a full round's.  Measured on MI355X
// (bench.py --round-sweep: 256x256 tiles of dense FP8 and NVFP4 problems
// from one to two rounds in eighths; least-squares fits 0.66 and 0.61).
constexpr double kPartialRound = 0.65;
double round_cost(long long tiles, long long slots) {
  const long long full = tiles / slots, rem = tiles % slots;
  return (double)full +
         (rem ? kPartialRound + (1.0 - kPartialRound) * (double)rem / (double)slots : 0.0);
}

// Score of a tile config, the tile-efficiency x wave-quantisation form of
// the flashinfer#3948 page ("Code analysis 2"): m_eff * n_eff * throughput /
// num_waves, with the terms defined for this device:
//   row_tiles = ceil(M / BM) + (G - 1): every expert boundary that falls
//               inside a window adds one pass over that window (the routing
//               is unknown on the host, so each boundary is assumed to);
//   m_eff     = M / (row_tiles * BM)   useful rows per computed row;
//   n_eff     = N / (ceil(N / BN) * BN);
//   num_waves = ceil(tiles / (CUs * wg_per_cu)), and the page's division by
//               num_waves is normalised to the fraction of workgroup slots
//               busy, tiles / (rounds * CUs * wg_per_cu), where a partly
//               filled last round counts by round_cost above, not whole;
//   throughput= per-CU efficiency of the tile shape.
// The page's 2-CTA and cluster-multicast factors have no gfx950 counterpart.
float score_tile(const fgg::TileCfg& t, int M, int N, int G, int num_cus, int run_align,
                 int variant = FGG_SCORE_KEPT) {
  const long long windows = (M + t.block_m - 1) / t.block_m;
  // every expert boundary in its own window, unless the runs start on
  // multiples of the tile height
  const bool aligned = run_align > 0 && run_align % t.block_m == 0;
  const long long row_tiles = windows + (aligned ? 0 : std::min<long long>(G - 1, windows * 4));
  const long long ntiles = (N + t.block_n - 1) / t.block_n;
  const double m_eff = (double)M / (double)(row_tiles * t.block_m);
  const double n_eff = (double)N / (double)(ntiles * t.block_n);
  const long long tiles = row_tiles * ntiles;
  const long long slots = (long long)std::max(1, num_cus) * t.wg_per_cu;
  const long long num_waves = (tiles + slots - 1) / slots;
  if (variant == FGG_SCORE_LITERAL)  // the page's printed form, for comparison
    return (float)(std::min(1.0, m_eff) * n_eff * t.tput / ((double)num_waves * t.block_n));
  const double busy = (double)tiles / (round_cost(tiles, slots) * (double)slots);
  return (float)(std::min(1.0, m_eff) * n_eff * busy * t.tput);
}

int rank(int kind, int M, int N, int G, int num_cus, int run_align, fgg_tile* out, int max_out,
         int variant = FGG_SCORE_KEPT) {
  const int n = kind == FGG_KIND_FP8 ? fgg::fp8_num_tiles() : fgg::fp4_num_tiles();
  std::vector<fgg_tile> v;
  for (int i = 0; i < n; ++i) {
    const fgg::TileCfg& t = kind == FGG_KIND_FP8 ? fgg::fp8_tile(i) : fgg::fp4_tile(i);
    fgg_tile r{t.id, t.block_m, t.block_n, t.waves, t.wg_per_cu,
               score_tile(t, M, N, G, num_cus, run_align, variant), t.tput};
    v.push_back(r);
  }
  std::stable_sort(v.begin(), v.end(), [](const fgg_tile& a, const fgg_tile& b) { return a.score > b.score; });
  const int k = std::min<int>(max_out, (int)v.size());
  for (int i = 0; i < k; ++i) out[i] = v[i];
  return k;
}

// ------------------------------------------------------------ autotuning
// Configs chosen by the *_tune entry points, per (kind, device, shape).
struct TuneKey {
  int kind, dev, M, N, K, G;
  bool operator<(const TuneKey& o) const {
    return std::tie(kind, dev, M, N, K, G) < std::tie(o.kind, o.dev, o.M, o.N, o.K, o.G);
  }
};
std::mutex g_tune_mu;
std::map<TuneKey, int> g_tuned;

int current_dev() {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess ? dev : -1;
}

int tuned_tile(int kind, int M, int N, int K, int G) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  auto it = g_tuned.find(TuneKey{kind, current_dev(), M, N, K, G});
  return it == g_tuned.end() ? -1 : it->second;
}

// Tile for a call: the explicit option, else the recorded tuning result for
// this shape, else the ranker's top choice.
// Tile config for a problem batch: the ranker's terms summed over the
// problems (useful over computed elements, busy fraction of the slots over
// the rounds of tiles, per-CU efficiency of the shape).  Set: Fp4ProblemSet or
// Fp8ProblemSet; tiles: the kind's config table.
template <class Set>
int rank_problems(const Set& set, int num_cus, int num_tiles, const fgg::TileCfg& (*tile_of)(int)) {
  int best = 0;
  double best_score = -1.0;
  for (int i = 0; i < num_tiles; ++i) {
    const fgg::TileCfg& t = tile_of(i);
    double useful = 0.0, computed = 0.0;
    long long tiles = 0;
    for (int g = 0; g < set.count; ++g) {
      const long long tg = (long long)((set.p[g].M + t.block_m - 1) / t.block_m) *
                           ((set.p[g].N + t.block_n - 1) / t.block_n);
      tiles += tg;
      useful += (double)set.p[g].M * set.p[g].N * set.p[g].K;
      computed += (double)tg * t.block_m * t.block_n * set.p[g].K;
    }
    const long long slots = (long long)std::max(1, num_cus) * t.wg_per_cu;
    const double busy = (double)tiles / (round_cost(tiles, slots) * (double)slots);
    const double score = useful / computed * busy * t.tput;
    if (score > best_score) {
      best_score = score;
      best = i;
    }
  }
  return best;
}

fgg_status pick_tile(const char* fn, int kind, int M, int N, int K, int G, int num_cus,
                     const fgg_options* opt, int* tile_id) {
  const int n = kind == FGG_KIND_FP8 ? fgg::fp8_num_tiles() : fgg::fp4_num_tiles();
  if (opt && opt->tile_id >= 0) {
    if (opt->tile_id >= n) return fail(FGG_EINVAL, fn, "tile_id %d out of range [0, %d)", opt->tile_id, n);
    *tile_id = opt->tile_id;
    return FGG_OK;
  }
  const int align = opt ? opt->run_align : 0;
  if (align < 0) return fail(FGG_EINVAL, fn, "run_align must be >= 0, got %d", align);
  const int t = tuned_tile(kind, M, N, K, G);
  if (t >= 0) {
    *tile_id = t;
    return FGG_OK;
  }
  fgg_tile best;
  rank(kind, M, N, G, num_cus, align, &best, 1);
  *tile_id = best.id;
  return FGG_OK;
}

// Time the ranker's top candidates with `launch(tile_id)` (returns the
// launch's hipError_t) and record the fastest.  Bounded: at most
// FGG_TUNE_MAX configs x (reps + 1) launches.
// Arguments of a *_tune call beyond its GEMM's (checked before the device).
fgg_status check_tune(const char* fn, int top_k, int reps, const fgg_options* opt) {
  if (top_k < 1) return fail(FGG_EINVAL, fn, "top_k must be >= 1, got %d", top_k);
  if (reps < 1 || reps > 100000) return fail(FGG_EINVAL, fn, "reps must be in [1, 100000], got %d", reps);
  if (opt && opt->tile_id >= 0)
    return fail(FGG_EINVAL, fn, "tile_id must be -1 when tuning (the tuning chooses it), got %d", opt->tile_id);
  if (opt && opt->run_align < 0) return fail(FGG_EINVAL, fn, "run_align must be >= 0, got %d", opt->run_align);
  return FGG_OK;
}

template <class Launch>
fgg_status run_tune(const char* fn, int kind, int M, int N, int K, int G, int num_cus, int top_k,
                    int reps, fgg_tune_report* report, const fgg_options* opt, hipStream_t s,
                    Launch launch) {
  const int align = opt ? opt->run_align : 0;
  fgg_tile cand[FGG_TUNE_MAX];
  const int n = rank(kind, M, N, G, num_cus, align, cand, std::min(top_k, FGG_TUNE_MAX));
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  fgg_tune_report r;
  std::memset(&r, 0, sizeof(r));
  r.n = n;
  // Three rounds over the candidates in turn, each config's fastest round
  // kept: the first config timed no longer pays for the clock ramp of a GPU
  // coming out of idle.
  constexpr int kRounds = 3;
  for (int i = 0; i < n; ++i) {
    r.tile_id[i] = cand[i].id;
    r.ms[i] = std::numeric_limits<float>::infinity();
  }
  for (int round = 0; round < kRounds && e == hipSuccess; ++round) {
    for (int i = 0; i < n && e == hipSuccess; ++i) {
      e = launch(cand[i].id);  // untimed (the first round: first use of this config's code)
      if (e == hipSuccess) e = hipEventRecord(e0, s);
      for (int k = 0; k < reps && e == hipSuccess; ++k) e = launch(cand[i].id);
      if (e == hipSuccess) e = hipEventRecord(e1, s);
      if (e == hipSuccess) e = hipEventSynchronize(e1);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
      if (e == hipSuccess) r.ms[i] = std::min(r.ms[i], ms / (float)reps);
    }
  }
  for (int i = 1; i < n; ++i)
    if (r.ms[i] < r.ms[r.best]) r.best = i;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return fail(FGG_EHIP, fn, "tuning failed: %s", hipGetErrorString(e));
  {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    g_tuned[TuneKey{kind, current_dev(), M, N, K, G}] = r.tile_id[r.best];
  }
  if (report) *report = r;
  g_err.clear();
  return FGG_OK;
}

fgg::LaunchOpts launch_opts(const fgg_options* opt, const DeviceFacts* d) {
  return fgg::LaunchOpts{opt ? opt->max_workgroups : 0, d->num_cus, opt ? opt->run_split : 0};
}

fgg_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(FGG_EHIP, fn, "kernel launch failed: %s", hipGetErrorString(e));
  g_err.clear();
  return FGG_OK;
}

}  // namespace

extern "C" {

const char* fgg_last_error(void) { return g_err.c_str(); }

int fgg_num_tiles(int kind) {
  if (kind == FGG_KIND_FP8) return fgg::fp8_num_tiles();
  if (kind == FGG_KIND_FP4) return fgg::fp4_num_tiles();
  return -1;
}

int fgg_rank_tiles_variant(int kind, int M, int N, int K, int G, int run_align, int variant,
                           int num_cus, fgg_tile* out, int max_out) {
  const char* fn = "fgg_rank_tiles";
  if (variant != FGG_SCORE_KEPT && variant != FGG_SCORE_LITERAL)
    return (fail(FGG_EINVAL, fn, "bad score variant %d", variant), -1);
  (void)K;
  if (kind != FGG_KIND_FP8 && kind != FGG_KIND_FP4) return (fail(FGG_EINVAL, fn, "bad kind %d", kind), -1);
  if (!out || max_out < 1) return (fail(FGG_EINVAL, fn, "need an output array"), -1);
  if (M < 1 || N < 1 || G < 1) return (fail(FGG_EINVAL, fn, "sizes must be positive"), -1);
  if (run_align < 0) return (fail(FGG_EINVAL, fn, "run_align must be >= 0, got %d", run_align), -1);
  if (num_cus <= 0) {
    fgg_status st;
    const DeviceFacts* d = current_device(fn, &st);
    if (!d) return -1;
    num_cus = d->num_cus;
  }
  return rank(kind, M, N, G, num_cus, run_align, out, max_out, variant);
}

int fgg_rank_tiles_aligned(int kind, int M, int N, int K, int G, int run_align, int num_cus,
                           fgg_tile* out, int max_out) {
  return fgg_rank_tiles_variant(kind, M, N, K, G, run_align, FGG_SCORE_KEPT, num_cus, out,
                                max_out);
}

int fgg_rank_tiles(int kind, int M, int N, int K, int G, int num_cus, fgg_tile* out, int max_out) {
  return fgg_rank_tiles_aligned(kind, M, N, K, G, 0, num_cus, out, max_out);
}

fgg_status fgg_device_info(int* num_cus, int* lds_per_block, int* clock_khz, char* arch,
                           int arch_len) {
  fgg_status st;
  const DeviceFacts* d = current_device("fgg_device_info", &st);
  if (!d) return st;
  if (num_cus) *num_cus = d->num_cus;
  if (lds_per_block) *lds_per_block = d->lds;
  if (clock_khz) *clock_khz = d->clock_khz;
  if (arch && arch_len > 0) std::snprintf(arch, arch_len, "%s", d->arch);
  return FGG_OK;
}

// Checks and device facts of a grouped FP8 call; fills the kernel arguments.
static fgg_status fp8_prepare(const char* fn, const void* A, const void* B, const float* a_scale,
                              const float* b_scale, const int32_t* m_indices, void* C, int M,
                              int N, int K, int G, fgg::Fp8Args* a, const DeviceFacts** d) {
  fgg_status st = check_common(fn, A, B, a_scale, b_scale, C, M, N, K, G, true, m_indices, 4);
  if (st != FGG_OK) return st;
  if (!(*d = current_device(fn, &st))) return st;
  *a = fgg::Fp8Args{static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B), a_scale,
                    b_scale, m_indices, static_cast<uint16_t*>(C), M, N, K, G};
  return FGG_OK;
}

fgg_status grouped_fp8_gemm_ex(const void* A, const void* B, const float* a_scale,
                               const float* b_scale, const int32_t* m_indices, void* C, int M,
                               int N, int K, int G, const fgg_options* opt, void* stream) {
  const char* fn = "grouped_fp8_gemm";
  fgg::Fp8Args a;
  const DeviceFacts* d = nullptr;
  fgg_status st = fp8_prepare(fn, A, B, a_scale, b_scale, m_indices, C, M, N, K, G, &a, &d);
  if (st != FGG_OK) return st;
  int tile;
  if ((st = pick_tile(fn, FGG_KIND_FP8, M, N, K, G, d->num_cus, opt, &tile)) != FGG_OK) return st;
  return launched(fn, fgg::launch_fp8(a, tile, launch_opts(opt, d), static_cast<hipStream_t>(stream)));
}

fgg_status grouped_fp8_gemm_tune(const void* A, const void* B, const float* a_scale,
                                 const float* b_scale, const int32_t* m_indices, void* C, int M,
                                 int N, int K, int G, int top_k, int reps,
                                 fgg_tune_report* report, const fgg_options* opt, void* stream) {
  const char* fn = "grouped_fp8_gemm_tune";
  fgg::Fp8Args a;
  const DeviceFacts* d = nullptr;
  fgg_status st = check_tune(fn, top_k, reps, opt);
  if (st != FGG_OK) return st;
  st = fp8_prepare(fn, A, B, a_scale, b_scale, m_indices, C, M, N, K, G, &a, &d);
  if (st != FGG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const fgg::LaunchOpts o = launch_opts(opt, d);
  return run_tune(fn, FGG_KIND_FP8, M, N, K, G, d->num_cus, top_k, reps, report, opt, s,
                  [&](int tile) { return fgg::launch_fp8(a, tile, o, s); });
}

fgg_status grouped_fp8_gemm(const void* A, const void* B, const float* a_scale,
                            const float* b_scale, const int32_t* m_indices, void* C, int M, int N,
                            int K, int G, void* stream) {
  return grouped_fp8_gemm_ex(A, B, a_scale, b_scale, m_indices, C, M, N, K, G, nullptr, stream);
}

// Checks and device facts of an NVFP4 call; fills the kernel arguments.
static fgg_status fp4_prepare(const char* fn, const void* A, const void* B, const void* a_scale,
                              const void* b_scale, const int32_t* m_indices, float alpha, void* C,
                              int M, int N, int K, int G, bool grouped, fgg::Fp4Args* a,
                              const DeviceFacts** d, const float* alphas = nullptr) {
  fgg_status st = check_common(fn, A, B, a_scale, b_scale, C, M, N, K, G, grouped, m_indices, 16, 16);
  if (st != FGG_OK) return st;
  if (!std::isfinite(alpha)) return fail(FGG_EINVAL, fn, "alpha must be finite");
  if (!(*d = current_device(fn, &st))) return st;
  *a = fgg::Fp4Args{static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(B),
                    static_cast<const uint8_t*>(a_scale), static_cast<const uint8_t*>(b_scale),
                    grouped ? m_indices : nullptr, alpha, alphas, static_cast<uint16_t*>(C), M, N,
                    K, G};
  return FGG_OK;
}

static fgg_status fp4_common(const char* fn, const void* A, const void* B, const void* a_scale,
                             const void* b_scale, const int32_t* m_indices, float alpha, void* C,
                             int M, int N, int K, int G, bool grouped, const fgg_options* opt,
                             void* stream) {
  fgg::Fp4Args a;
  const DeviceFacts* d = nullptr;
  fgg_status st = fp4_prepare(fn, A, B, a_scale, b_scale, m_indices, alpha, C, M, N, K, G, grouped,
                              &a, &d);
  if (st != FGG_OK) return st;
  int tile;
  if ((st = pick_tile(fn, FGG_KIND_FP4, M, N, K, G, d->num_cus, opt, &tile)) != FGG_OK) return st;
  return launched(fn, fgg::launch_fp4(a, tile, launch_opts(opt, d), static_cast<hipStream_t>(stream)));
}

static fgg_status fp4_tune(const char* fn, const void* A, const void* B, const void* a_scale,
                           const void* b_scale, const int32_t* m_indices, float alpha, void* C,
                           int M, int N, int K, int G, bool grouped, int top_k, int reps,
                           fgg_tune_report* report, const fgg_options* opt, void* stream) {
  fgg::Fp4Args a;
  const DeviceFacts* d = nullptr;
  fgg_status st = check_tune(fn, top_k, reps, opt);
  if (st != FGG_OK) return st;
  st = fp4_prepare(fn, A, B, a_scale, b_scale, m_indices, alpha, C, M, N, K, G, grouped, &a, &d);
  if (st != FGG_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const fgg::LaunchOpts o = launch_opts(opt, d);
  return run_tune(fn, FGG_KIND_FP4, M, N, K, G, d->num_cus, top_k, reps, report, opt, s,
                  [&](int tile) { return fgg::launch_fp4(a, tile, o, s); });
}

fgg_status fp4_gemm_ex(const void* A, const void* B, const void* a_scale, const void* b_scale,
                       float alpha, void* C, int M, int N, int K, const fgg_options* opt,
                       void* stream) {
  return fp4_common("fp4_gemm", A, B, a_scale, b_scale, nullptr, alpha, C, M, N, K, 1, false, opt,
                    stream);
}

fgg_status fp4_gemm(const void* A, const void* B, const void* a_scale, const void* b_scale,
                    float alpha, void* C, int M, int N, int K, void* stream) {
  return fp4_gemm_ex(A, B, a_scale, b_scale, alpha, C, M, N, K, nullptr, stream);
}

fgg_status grouped_fp4_gemm_ex(const void* A, const void* B, const void* a_scale,
                               const void* b_scale, const int32_t* m_indices, float alpha, void* C,
                               int M, int N, int K, int G, const fgg_options* opt, void* stream) {
  return fp4_common("grouped_fp4_gemm", A, B, a_scale, b_scale, m_indices, alpha, C, M, N, K, G,
                    true, opt, stream);
}

fgg_status grouped_fp4_gemm(const void* A, const void* B, const void* a_scale,
                            const void* b_scale, const int32_t* m_indices, float alpha, void* C,
                            int M, int N, int K, int G, void* stream) {
  return grouped_fp4_gemm_ex(A, B, a_scale, b_scale, m_indices, alpha, C, M, N, K, G, nullptr,
                             stream);
}

fgg_status fp4_gemm_tune(const void* A, const void* B, const void* a_scale, const void* b_scale,
                         float alpha, void* C, int M, int N, int K, int top_k, int reps,
                         fgg_tune_report* report, const fgg_options* opt, void* stream) {
  return fp4_tune("fp4_gemm_tune", A, B, a_scale, b_scale, nullptr, alpha, C, M, N, K, 1, false,
                  top_k, reps, report, opt, stream);
}

fgg_status grouped_fp4_gemm_tune(const void* A, const void* B, const void* a_scale,
                                 const void* b_scale, const int32_t* m_indices, float alpha,
                                 void* C, int M, int N, int K, int G, int top_k, int reps,
                                 fgg_tune_report* report, const fgg_options* opt,
                                 void* stream) {
  return fp4_tune("grouped_fp4_gemm_tune", A, B, a_scale, b_scale, m_indices, alpha, C, M, N, K, G,
                  true, top_k, reps, report, opt, stream);
}

fgg_status grouped_fp4_gemm_alpha_ex(const void* A, const void* B, const void* a_scale,
                                     const void* b_scale, const int32_t* m_indices,
                                     const float* alpha, void* C, int M, int N, int K, int G,
                                     const fgg_options* opt, void* stream) {
  const char* fn = "grouped_fp4_gemm_alpha";
  if (!alpha) return fail(FGG_EINVAL, fn, "alpha is null");
  if (!aligned(alpha, 4)) return fail(FGG_EALIGN, fn, "alpha must be 4-byte aligned");
  fgg::Fp4Args a;
  const DeviceFacts* d = nullptr;
  fgg_status st = fp4_prepare(fn, A, B, a_scale, b_scale, m_indices, 1.0f, C, M, N, K, G, true,
                              &a, &d, alpha);
  if (st != FGG_OK) return st;
  int tile;
  if ((st = pick_tile(fn, FGG_KIND_FP4, M, N, K, G, d->num_cus, opt, &tile)) != FGG_OK) return st;
  return launched(fn, fgg::launch_fp4(a, tile, launch_opts(opt, d), static_cast<hipStream_t>(stream)));
}

fgg_status grouped_fp4_gemm_alpha(const void* A, const void* B, const void* a_scale,
                                  const void* b_scale, const int32_t* m_indices, const float* alpha,
                                  void* C, int M, int N, int K, int G, void* stream) {
  return grouped_fp4_gemm_alpha_ex(A, B, a_scale, b_scale, m_indices, alpha, C, M, N, K, G, nullptr,
                                   stream);
}

fgg_status fp4_gemm_problems_ex(const fgg_fp4_problem* problems, int count,
                                const fgg_options* opt, void* stream) {
  const char* fn = "fp4_gemm_problems";
  if (!problems) return fail(FGG_EINVAL, fn, "problems is null");
  if (count < 1 || count > FGG_MAX_PROBLEMS)
    return fail(FGG_EINVAL, fn, "requires 1 <= count <= %d, got %d", FGG_MAX_PROBLEMS, count);
  fgg::Fp4ProblemSet set;
  std::memset(&set, 0, sizeof(set));
  set.count = count;
  for (int g = 0; g < count; ++g) {
    const fgg_fp4_problem& q = problems[g];
    char where[64];
    std::snprintf(where, sizeof(where), "%s (problem %d)", fn, g);
    fgg_status st = check_common(where, q.A, q.B, q.a_scale, q.b_scale, q.C, q.M, q.N, q.K, 1,
                                 false, nullptr, 16, 16);
    if (st != FGG_OK) return st;
    if (!std::isfinite(q.alpha)) return fail(FGG_EINVAL, where, "alpha must be finite");
    set.p[g] = fgg::Fp4Problem{static_cast<const uint8_t*>(q.A), static_cast<const uint8_t*>(q.B),
                               static_cast<const uint8_t*>(q.a_scale),
                               static_cast<const uint8_t*>(q.b_scale), static_cast<uint16_t*>(q.C),
                               q.M, q.N, q.K, q.alpha};
  }
  fgg_status st;
  const DeviceFacts* d = current_device(fn, &st);
  if (!d) return st;
  int tile = -1;
  if (opt && opt->tile_id >= 0) {
    if (opt->tile_id >= fgg::fp4_num_tiles())
      return fail(FGG_EINVAL, fn, "tile_id %d out of range [0, %d)", opt->tile_id, fgg::fp4_num_tiles());
    tile = opt->tile_id;
  } else {
    tile = rank_problems(set, d->num_cus, fgg::fp4_num_tiles(), fgg::fp4_tile);
  }
  return launched(fn, fgg::launch_fp4_problems(set, tile, launch_opts(opt, d),
                                               static_cast<hipStream_t>(stream)));
}

fgg_status fp4_gemm_problems(const fgg_fp4_problem* problems, int count, void* stream) {
  return fp4_gemm_problems_ex(problems, count, nullptr, stream);
}

fgg_status fp8_gemm_problems_ex(const fgg_fp8_problem* problems, int count,
                                const fgg_options* opt, void* stream) {
  const char* fn = "fp8_gemm_problems";
  if (!problems) return fail(FGG_EINVAL, fn, "problems is null");
  if (count < 1 || count > FGG_MAX_PROBLEMS)
    return fail(FGG_EINVAL, fn, "requires 1 <= count <= %d, got %d", FGG_MAX_PROBLEMS, count);
  fgg::Fp8ProblemSet set;
  std::memset(&set, 0, sizeof(set));
  set.count = count;
  for (int g = 0; g < count; ++g) {
    const fgg_fp8_problem& q = problems[g];
    char where[64];
    std::snprintf(where, sizeof(where), "%s (problem %d)", fn, g);
    fgg_status st = check_common(where, q.A, q.B, q.a_scale, q.b_scale, q.C, q.M, q.N, q.K, 1,
                                 false, nullptr, 4);
    if (st != FGG_OK) return st;
    set.p[g] = fgg::Fp8Problem{static_cast<const uint8_t*>(q.A), static_cast<const uint8_t*>(q.B),
                               q.a_scale, q.b_scale, static_cast<uint16_t*>(q.C), q.M, q.N, q.K};
  }
  fgg_status st;
  const DeviceFacts* d = current_device(fn, &st);
  if (!d) return st;
  int tile = -1;
  if (opt && opt->tile_id >= 0) {
    if (opt->tile_id >= fgg::fp8_num_tiles())
      return fail(FGG_EINVAL, fn, "tile_id %d out of range [0, %d)", opt->tile_id, fgg::fp8_num_tiles());
    tile = opt->tile_id;
  } else {
    tile = rank_problems(set, d->num_cus, fgg::fp8_num_tiles(), fgg::fp8_tile);
  }
  return launched(fn, fgg::launch_fp8_problems(set, tile, launch_opts(opt, d),
                                               static_cast<hipStream_t>(stream)));
}

fgg_status fp8_gemm_problems(const fgg_fp8_problem* problems, int count, void* stream) {
  return fp8_gemm_problems_ex(problems, count, nullptr, stream);
}

fgg_status grouped_w4a16_gemm(const void* A, const void* B, const void* b_scale,
                              const int32_t* m_indices, float b_global, void* C, int M, int N,
                              int K, int G, void* stream) {
  const char* fn = "grouped_w4a16_gemm";
  // A stands in for a_scale in the shared checks (16-byte aligned, non-null).
  fgg_status st = check_common(fn, A, B, A, b_scale, C, M, N, K, G, true, m_indices, 16, 16);
  if (st != FGG_OK) return st;
  if (!std::isfinite(b_global)) return fail(FGG_EINVAL, fn, "b_global must be finite");
  if ((long long)M * K * 2 > 0x7FFFFFFFLL)
    return fail(FGG_EUNSUPPORTED, fn, "requires M * K * 2 < 2^31 bytes of activations (decode path), got M=%d K=%d", M, K);
  const DeviceFacts* d = current_device(fn, &st);
  if (!d) return st;
  const fgg::W4A16Args a{static_cast<const uint16_t*>(A), static_cast<const uint8_t*>(B),
                         static_cast<const uint8_t*>(b_scale), m_indices, b_global,
                         static_cast<uint16_t*>(C), M, N, K, G};
  return launched(fn, fgg::launch_w4a16(a, static_cast<hipStream_t>(stream)));
}

int fgg_tuned_tile(int kind, int M, int N, int K, int G) { return tuned_tile(kind, M, N, K, G); }

void fgg_tune_clear(void) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tuned.clear();
}

// Activation quantisers (the step before the GEMM).
static fgg_status check_quant(const char* fn, const void* X, const void* Q, const void* S, int M,
                              int K, uintptr_t scale_align, int k_unit) {
  if (!X || !Q || !S) return fail(FGG_EINVAL, fn, "null pointer among X, Q, scale");
  if (M < 1 || M > (1 << 24)) return fail(FGG_EINVAL, fn, "requires 1 <= M <= 2^24, got M=%d", M);
  if (K < k_unit || K > (1 << 20)) return fail(FGG_EINVAL, fn, "requires %d <= K <= 2^20, got K=%d", k_unit, K);
  if (K % k_unit) return fail(FGG_EINVAL, fn, "requires K %% %d == 0, got K=%d", k_unit, K);
  if (K % 128)
    return fail(FGG_EUNSUPPORTED, fn, "K %% 128 != 0 (K=%d) is not supported", K);
  if (!aligned(X, 16) || !aligned(Q, 16))
    return fail(FGG_EALIGN, fn, "X and Q must be 16-byte aligned");
  if (!aligned(S, scale_align))
    return fail(FGG_EALIGN, fn, "scale must be %d-byte aligned", (int)scale_align);
  return FGG_OK;
}

fgg_status quantize_fp8_1x128(const void* X, void* Q, float* scale, int M, int K, void* stream) {
  const char* fn = "quantize_fp8_1x128";
  fgg_status st = check_quant(fn, X, Q, scale, M, K, 4, 128);
  if (st != FGG_OK) return st;
  const DeviceFacts* d = current_device(fn, &st);
  if (!d) return st;
  return launched(fn, fgg::launch_quant_fp8(static_cast<const uint16_t*>(X), static_cast<uint8_t*>(Q),
                                            scale, M, K, d->num_cus,
                                            static_cast<hipStream_t>(stream)));
}

fgg_status quantize_nvfp4(const void* X, void* Q, void* scale, float* global_scale, int M, int K,
                          void* stream) {
  const char* fn = "quantize_nvfp4";
  fgg_status st = check_quant(fn, X, Q, scale, M, K, 1, 16);
  if (st != FGG_OK) return st;
  if (!global_scale) return fail(FGG_EINVAL, fn, "global_scale is null");
  if (!aligned(global_scale, 4)) return fail(FGG_EALIGN, fn, "global_scale must be 4-byte aligned");
  const DeviceFacts* d = current_device(fn, &st);
  if (!d) return st;
  return launched(fn, fgg::launch_quant_nvfp4(static_cast<const uint16_t*>(X),
                                              static_cast<uint8_t*>(Q), static_cast<uint8_t*>(scale),
                                              global_scale, M, K, d->num_cus,
                                              static_cast<hipStream_t>(stream)));
}

fgg_status quantize_nvfp4_static(const void* X, void* Q, void* scale, float global_scale, int M,
                                 int K, void* stream) {
  const char* fn = "quantize_nvfp4_static";
  fgg_status st = check_quant(fn, X, Q, scale, M, K, 1, 16);
  if (st != FGG_OK) return st;
  if (!std::isfinite(global_scale) || !(global_scale >= std::numeric_limits<float>::min()))
    return fail(FGG_EINVAL, fn, "global_scale must be a finite normal positive float, got %g",
                (double)global_scale);
  const DeviceFacts* d = current_device(fn, &st);
  if (!d) return st;
  return launched(fn, fgg::launch_quant_nvfp4_static(static_cast<const uint16_t*>(X),
                                                     static_cast<uint8_t*>(Q),
                                                     static_cast<uint8_t*>(scale), global_scale, M,
                                                     K, d->num_cus,
                                                     static_cast<hipStream_t>(stream)));
}

// Row-expansion variants: output row r from token row rows[r].
static fgg_status check_rows(const char* fn, const int32_t* rows, int R, int T, int K) {
  if (!rows) return fail(FGG_EINVAL, fn, "rows is null");
  if (!aligned(rows, 4)) return fail(FGG_EALIGN, fn, "rows must be 4-byte aligned");
  if (T < 1 || T > (1 << 24)) return fail(FGG_EINVAL, fn, "requires 1 <= T <= 2^24, got T=%d", T);
  if ((long long)R * (K / 32) > 0x7FFFFFFFLL)
    return fail(FGG_EUNSUPPORTED, fn, "requires R * K / 32 < 2^31, got R=%d K=%d", R, K);
  return FGG_OK;
}

fgg_status quantize_fp8_1x128_rows(const void* X, const int32_t* rows, void* Q, float* scale,
                                   int R, int T, int K, void* stream) {
  const char* fn = "quantize_fp8_1x128_rows";
  fgg_status st = check_quant(fn, X, Q, scale, R, K, 4, 128);
  if (st != FGG_OK) return st;
  if ((st = check_rows(fn, rows, R, T, K)) != FGG_OK) return st;
  const DeviceFacts* d = current_device(fn, &st);
  if (!d) return st;
  return launched(fn, fgg::launch_quant_fp8(static_cast<const uint16_t*>(X), static_cast<uint8_t*>(Q),
                                            scale, R, K, d->num_cus,
                                            static_cast<hipStream_t>(stream), rows, T));
}

fgg_status quantize_nvfp4_static_rows(const void* X, const int32_t* rows, void* Q, void* scale,
                                      float global_scale, int R, int T, int K, void* stream) {
  const char* fn = "quantize_nvfp4_static_rows";
  fgg_status st = check_quant(fn, X, Q, scale, R, K, 1, 16);
  if (st != FGG_OK) return st;
  if ((st = check_rows(fn, rows, R, T, K)) != FGG_OK) return st;
  if (!std::isfinite(global_scale) || !(global_scale >= std::numeric_limits<float>::min()))
    return fail(FGG_EINVAL, fn, "global_scale must be a finite normal positive float, got %g",
                (double)global_scale);
  const DeviceFacts* d = current_device(fn, &st);
  if (!d) return st;
  return launched(fn, fgg::launch_quant_nvfp4_static(static_cast<const uint16_t*>(X),
                                                     static_cast<uint8_t*>(Q),
                                                     static_cast<uint8_t*>(scale), global_scale, R,
                                                     K, d->num_cus,
                                                     static_cast<hipStream_t>(stream), rows, T));
}

}  // extern "C"
