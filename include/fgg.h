/*
 * fgg.h -- block-scaled low-precision (grouped) GEMM for AMD MI355X (gfx950).
 *
 * C ABI of libfgg.so.  Every pointer argument named A, B, a_scale, b_scale,
 * m_indices or C is a DEVICE pointer (HIP global memory of the current
 * device); sizes are plain ints; `stream` is a hipStream_t passed as void*
 * (NULL = the default stream), so that this header needs no HIP header and
 * plain C or ctypes callers can use it as it is.  The library reads A, B,
 * the scales and m_indices, writes every element of C (C need not be
 * initialised), keeps no
 * pointer after the call returns, allocates no device memory and never
 * synchronises: work is enqueued on `stream` and the call returns.  It never
 * reads m_indices on the host, so a call can be captured in a HIP graph and
 * replayed after the contents of m_indices change.
 *
 * Errors: each entry point validates its arguments on the host before
 * touching the GPU and returns a status; on a non-OK status nothing is
 * enqueued and fgg_last_error() returns a message (per calling thread) that
 * names the entry point and the violated condition.  Device faults from bad
 * pointer *contents* (e.g. a buffer shorter than the sizes say) are not
 * detectable and are the caller's responsibility.
 *
 * Definitions come from the pages on the method (cited by page and section):
 *  - grouped FP8: flashinfer#7877 page ("cake_grouped_fp8_gemm" window-segment
 *    program), "Intro" and "Code analysis 1": FP8 E4M3 inputs, BF16 output,
 *    rows grouped by m_indices, FP32 per-128 block scales, kernel arguments
 *    A, B, C, a_scale, b_scale, m_indices, M, N, K, G; A is a row-major byte
 *    matrix whose inner extent K is a multiple of 128 and whose rows may run
 *    past a tile (tail rows are masked), strides and addresses 16-byte
 *    aligned; launch contract 1 <= M <= 2^24, 64 <= N <= 2^19.
 *  - E4M3FN with largest finite value 448 on gfx950: sglang#27745 page,
 *    "Code analysis 1: FP8 quantisation".
 *  - NVFP4 W4A4 (E2M1 values, an E4M3 scale per 16 elements, FP32 global
 *    scale): onnxruntime#29824 page, "Code analysis 1"; dense mm_fp4:
 *    flashinfer#3948 page.
 */
#ifndef FGG_H
#define FGG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FGG_OK = 0,
  FGG_EINVAL = 1,        /* null pointer, size outside the method's limits, a
                          * divisibility the method itself requires violated  */
  FGG_EUNSUPPORTED = 2,  /* a shape the method allows but this library does
                          * not implement (N a multiple of 64 but not of 128;
                          * NVFP4 K a multiple of 16 but not of 128; a W4A16
                          * activation array of 2^31 bytes or more)          */
  FGG_EALIGN = 3,        /* a pointer is not 16-byte aligned (4 for scales)   */
  FGG_EDEVICE = 4,       /* no HIP device, or the current device is not gfx950 */
  FGG_EHIP = 5           /* a HIP runtime call or kernel launch failed        */
} fgg_status;

/* Message for the last non-OK status returned on this thread ("" if none).
 * The pointer stays valid until the next fgg call on the same thread. */
const char* fgg_last_error(void);

/*
 * grouped_fp8_gemm -- C = grouped block-scaled FP8 GEMM, BF16 out.
 *
 *   A         [M, K]       E4M3FN bytes, row-major (K contiguous)
 *   B         [G, N, K]    E4M3FN bytes, expert g's weights B[g] row-major
 *   a_scale   [M, K/128]   float32, row-major: scale of row i, K block kb
 *   b_scale   [G, N/128, K/128] float32, row-major: scale of the 128x128
 *                          block (n/128, kb) of B[g]
 *   m_indices [M]          int32: expert of row i, or -1 for a padding row.
 *                          Any value outside [-1, G) is treated as -1.  Rows
 *                          need not be sorted; contiguous runs are fastest.
 *   C         [M, N]       BF16 (uint16 bits), row-major, written in full
 *
 *   C[i, n] = bf16( sum_kb a_scale[i,kb] * b_scale[g,n/128,kb]
 *                          * sum_{k in kb} A[i,k] * B[g,n,k] ),  g = m_indices[i]
 *   C[i, :] = 0 when g is -1 (or out of range).
 *   Accumulation is FP32; the BF16 conversion rounds to nearest even.
 *
 * Requirements: 1 <= M <= 2^24, 64 <= N <= 2^19 with N % 64 == 0,
 * 128 <= K <= 2^20 with K % 128 == 0, 1 <= G <= 2^16, every pointer
 * non-null (else FGG_EINVAL); N % 128 == 0, whole b_scale blocks (else
 * FGG_EUNSUPPORTED); A, B and C 16-byte aligned, a_scale, b_scale and
 * m_indices 4-byte aligned (else FGG_EALIGN).  Rows of A whose m_indices
 * entry is -1 (or out of range) may hold any bytes: they never reach a
 * stored output.
 */
fgg_status grouped_fp8_gemm(const void* A, const void* B, const float* a_scale,
                            const float* b_scale, const int32_t* m_indices, void* C,
                            int M, int N, int K, int G, void* stream);

/*
 * fp4_gemm -- dense NVFP4 GEMM, BF16 out.
 *
 *   A        [M, K/2]   packed E2M1 (element 2j in the low nibble of byte j)
 *   B        [N, K/2]   packed E2M1, row n holds column n of the product
 *   a_scale  [M, K/16]  E4M3FN bytes: scale of A's 16-element K block
 *   b_scale  [N, K/16]  E4M3FN bytes
 *   alpha    float      product of the two per-tensor FP32 global scales
 *   C        [M, N]     BF16, row-major, written in full
 *
 *   C[i, n] = bf16( alpha * sum_k (A[i,k] a_scale[i,k/16]) (B[n,k] b_scale[n,k/16]) )
 *
 * Requirements: 1 <= M <= 2^24, 64 <= N <= 2^19 with N % 64 == 0,
 * 16 <= K <= 2^20 with K % 16 == 0 (whole scale blocks), pointers non-null
 * (else FGG_EINVAL); N % 128 == 0 and K % 128 == 0 (else FGG_EUNSUPPORTED);
 * pointers 16-byte aligned (else FGG_EALIGN).  A scale code that is an
 * E4M3FN NaN (0x7F / 0xFF) makes every output it reaches NaN.
 */
fgg_status fp4_gemm(const void* A, const void* B, const void* a_scale, const void* b_scale,
                    float alpha, void* C, int M, int N, int K, void* stream);

/*
 * grouped_fp4_gemm -- grouped NVFP4 GEMM (MoE W4A4), BF16 out.
 *
 *   A        [M, K/2]      packed E2M1;   a_scale [M, K/16] E4M3FN bytes
 *   B        [G, N, K/2]   packed E2M1;   b_scale [G, N, K/16] E4M3FN bytes
 *   m_indices[M]           int32 expert id or -1 (as for grouped_fp8_gemm)
 *   alpha                  product of the global scales of A and of B (one
 *                          global scale for all experts' B)
 *   C        [M, N]        BF16, written in full; -1 rows are zero
 *
 * Requirements: as fp4_gemm plus 1 <= G <= 2^16.
 */
fgg_status grouped_fp4_gemm(const void* A, const void* B, const void* a_scale,
                            const void* b_scale, const int32_t* m_indices, float alpha,
                            void* C, int M, int N, int K, int G, void* stream);

/*
 * grouped_fp4_gemm_alpha -- grouped_fp4_gemm with one global scale per
 * expert: row i of expert g is multiplied by alpha[g] (= gA * gB[g]) instead
 * of one alpha for all experts (the per-group scaling of the cutlass#3124
 * page's grouped block-scaled GEMM).  `alpha` is a device array of G finite
 * floats, 4-byte aligned, read on the device at every launch (graph replay
 * sees new values); everything else as grouped_fp4_gemm.
 */
fgg_status grouped_fp4_gemm_alpha(const void* A, const void* B, const void* a_scale,
                                  const void* b_scale, const int32_t* m_indices,
                                  const float* alpha, void* C, int M, int N, int K, int G,
                                  void* stream);

/*
 * fp4_gemm_problems -- a batch of independent dense NVFP4 GEMMs whose M, N
 * and K may all differ, in one launch (the cutlass#3124 page's grouped
 * block-scaled GEMM, "Intro").  Problem g computes its own
 *   C_g[i, n] = alpha_g * sum_k (qA sA)(qB sB)
 * exactly as fp4_gemm does on its operands.  `problems` is a host array of
 * `count` descriptors (1 <= count <= FGG_MAX_PROBLEMS), read during the call
 * and passed to the kernel by value: no device allocation, no host
 * synchronisation, capturable in a HIP graph (the descriptors are captured
 * with it).  Every problem must meet fp4_gemm's requirements; an error names
 * the problem's index.  Problems must not write overlapping C.
 */
#define FGG_MAX_PROBLEMS 32

typedef struct {
  const void* A;        /* [M, K/2] packed E2M1                               */
  const void* B;        /* [N, K/2] packed E2M1                               */
  const void* a_scale;  /* [M, K/16] E4M3FN                                   */
  const void* b_scale;  /* [N, K/16] E4M3FN                                   */
  void* C;              /* [M, N] BF16, written in full                       */
  int M, N, K;
  float alpha;          /* product of the two global scales                   */
} fgg_fp4_problem;

fgg_status fp4_gemm_problems(const fgg_fp4_problem* problems, int count, void* stream);

/*
 * fp8_gemm_problems -- a batch of independent dense block-scaled FP8 GEMMs
 * whose M, N and K may all differ, in one launch (the same "Intro" of the
 * cutlass#3124 page, which names no number format; here the library's main
 * FP8 form).  Problem g computes
 *   C_g[i, n] = sum_kb a_scale_g[i, kb] * b_scale_g[n/128, kb] * sum_{k in kb} A_g[i,k] B_g[n,k]
 * with the arithmetic of grouped_fp8_gemm at G = 1 with every row routed to
 * expert 0 (so the same bits on the same tile config).  Descriptors, count,
 * capture and error reporting as for fp4_gemm_problems; every problem must
 * meet grouped_fp8_gemm's requirements (as at G = 1).  Problems must not
 * write overlapping C.
 */
typedef struct {
  const void* A;         /* [M, K] E4M3FN codes                               */
  const void* B;         /* [N, K] E4M3FN codes                               */
  const float* a_scale;  /* [M, K/128] FP32                                   */
  const float* b_scale;  /* [N/128, K/128] FP32                               */
  void* C;               /* [M, N] BF16, written in full                      */
  int M, N, K;
} fgg_fp8_problem;

fgg_status fp8_gemm_problems(const fgg_fp8_problem* problems, int count, void* stream);

/*
 * grouped_w4a16_gemm -- grouped GEMM of BF16 activations with NVFP4 weights
 * (W4A16), BF16 out: the decode / small-M path of the onnxruntime#29824 page
 * ("Code analysis 1": FP4 weights with 16-bit activations, dequantised).
 *
 *   A        [M, K]        BF16 activations (row i routed by m_indices[i])
 *   B        [G, N, K/2]   packed E2M1;   b_scale [G, N, K/16] E4M3FN bytes
 *   m_indices[M]           int32 expert id or -1 (as for grouped_fp8_gemm)
 *   b_global               FP32 global scale of B (one for all experts)
 *   C        [M, N]        BF16, written in full; -1 rows are zero
 *
 *   C[i, n] = b_global * sum_k A[i, k] * qB[g, n, k] * sB[g, n, k / 16]
 *
 * Weights are dequantised exactly (E2M1 x E4M3 has at most 6 significant
 * bits) and multiplied with FP32 accumulation.  Built for few rows per expert
 * (decode): m_indices is scanned 1024 entries at a time, and an expert's
 * weights are streamed once per 32 of its rows found in a scan (rounded up
 * per scan).  So for M <= 1024 every expert's weights stream
 * ceil(rows_e / 32) times, and an expert with no rows costs no weight
 * traffic; for larger M each further scan that holds rows of an expert
 * streams its weights again (results are the same at any M; prefill-sized
 * batches belong on grouped_fp4_gemm after quantize_nvfp4).  Requirements as
 * grouped_fp4_gemm (A 16-byte aligned); b_global finite; M * K * 2 < 2^31,
 * the activations of a decode batch (else FGG_EUNSUPPORTED).  Rows routed
 * to an expert must be finite; rows marked -1 (or out of range) may hold
 * anything, as may the memory around A: neither is ever multiplied.
 */
fgg_status grouped_w4a16_gemm(const void* A, const void* B, const void* b_scale,
                              const int32_t* m_indices, float b_global, void* C, int M, int N,
                              int K, int G, void* stream);

/* ------------------------------------------------------------------------
 * Activation quantisers: the step before the GEMM, producing its A operand.
 *
 * quantize_fp8_1x128 -- BF16 X [M, K] -> E4M3FN codes Q [M, K] and one FP32
 * scale per row and 128-wide K block, scale [M, K/128] (the a_scale layout of
 * grouped_fp8_gemm).  scale = amax(block) / 448 (1.0 for an all-zero block);
 * code = E4M3FN round-to-nearest-even of clamp(x / scale, -448, 448), every
 * step an FP32 operation rounded to nearest even (sglang#27745 page, "Code
 * analysis 1: FP8 quantisation": clamp to the gfx950 E4M3FN maximum 448, then
 * encode; flashinfer#7877 page: FP32 per-128 block scales).
 *
 * quantize_nvfp4 -- BF16 X [M, K] -> packed E2M1 Q [M, K/2] (element 2j in the
 * low nibble of byte j), E4M3FN block-scale codes scale [M, K/16] and the FP32
 * global scale written to the device scalar *global_scale (the A-side factor
 * of the GEMM's alpha; the W4A4 activations of the onnxruntime#29824 page).
 * g = amax(X) / 2688 (1.0 for all-zero X), s = E4M3FN(min(amax(block) /
 * (6 g), 448)), code = E2M1(clamp(x / (value(s) g), -6, 6)), 0 where
 * value(s) g is 0.  Four kernel launches on `stream` (clear, amax, encode,
 * finalise); no host synchronisation, no allocation.
 *
 * quantize_nvfp4_static -- the same encoding with the global scale g given by
 * the caller (a calibrated, static activation scale; the NVFP4 format has one
 * FP32 scale per tensor, and how it is chosen is left open by the pages)
 * instead of amax(X) / 2688: one kernel launch that reads X once.  Values
 * whose block amax exceeds 448 * 6 * g saturate (block scale 448, codes clamped to +-6).  g must be a
 * finite normal positive float (FGG_EINVAL otherwise).
 *
 * Requirements: 1 <= M <= 2^24; 128 <= K <= 2^20 with K % 128 == 0 for
 * FP8 (FGG_EINVAL otherwise); for NVFP4 16 <= K <= 2^20 with K % 16 == 0
 * (FGG_EINVAL) and K % 128 == 0 (FGG_EUNSUPPORTED); X, Q 16-byte aligned
 * (scale: 4-byte for FP8, any for NVFP4; the global_scale pointer of
 * quantize_nvfp4 4-byte; FGG_EALIGN); X finite.
 * ------------------------------------------------------------------------ */
fgg_status quantize_fp8_1x128(const void* X, void* Q, float* scale, int M, int K, void* stream);
fgg_status quantize_nvfp4(const void* X, void* Q, void* scale, float* global_scale, int M, int K,
                          void* stream);
fgg_status quantize_nvfp4_static(const void* X, void* Q, void* scale, float global_scale, int M,
                                 int K, void* stream);

/*
 * quantize_fp8_1x128_rows, quantize_nvfp4_static_rows -- the same encodings,
 * fused with the row expansion of an MoE layer (the onnxruntime#29824 page,
 * "Code analysis 1": expandInputRowsKernel quantises while it copies each
 * token's activations to the rows of the experts it is routed to).
 *
 *   X     [T, K]   BF16 token activations
 *   rows  [R]      int32, device: output row r holds token rows[r]; a value
 *                  outside [0, T) makes row r a padding row, encoded as
 *                  zeros (FP8: codes 0, scale 1.0; NVFP4: codes 0, scale
 *                  code 0).  Read on the device at every launch.
 *   Q, scale       as quantize_fp8_1x128 / quantize_nvfp4_static with R rows
 *
 * Row r of the output equals the row-wise quantisation of X[rows[r]] (the
 * encodings are per row), so with rows sorted by expert the result is the
 * A operand of grouped_fp8_gemm / grouped_fp4_gemm directly.  One kernel
 * launch reading each routed token row once per expert it goes to.
 * Requirements as the row-wise quantisers with M = R, plus 1 <= T <= 2^24,
 * rows non-null and 4-byte aligned, and R * K / 32 < 2^31
 * (FGG_EUNSUPPORTED).
 */
fgg_status quantize_fp8_1x128_rows(const void* X, const int32_t* rows, void* Q, float* scale,
                                   int R, int T, int K, void* stream);
fgg_status quantize_nvfp4_static_rows(const void* X, const int32_t* rows, void* Q, void* scale,
                                      float global_scale, int R, int T, int K, void* stream);

/* ------------------------------------------------------------------------
 * Tile configurations and the ranker.
 *
 * The kernels are compiled for a small set of tile shapes.  For each call
 * the host ranks them with a tile-efficiency x wave-quantisation score sized
 * to the device's compute-unit count (the heuristic-ranking idea of the
 * flashinfer#3948 page, "Code analysis 2": score = m_eff * n_eff *
 * throughput / num_waves, with terms defined for this device) and launches
 * the top one.  These calls are pure host logic and need no GPU.
 * ------------------------------------------------------------------------ */

typedef enum { FGG_KIND_FP8 = 0, FGG_KIND_FP4 = 1 } fgg_kind;

typedef struct {
  int id;          /* index of the compiled tile config                     */
  int block_m;     /* rows per work tile (the row window)                   */
  int block_n;     /* columns per work tile                                 */
  int waves;       /* 64-lane wavefronts per workgroup                      */
  int wg_per_cu;   /* workgroups resident per compute unit                  */
  float score;     /* ranker score (higher is better); 0 = not applicable   */
  float tput;      /* the shape's relative per-CU throughput (1.0 = best),
                    * the ranker's throughput term                         */
} fgg_tile;

/* Number of compiled tile configs for `kind`, or -1 for a bad kind. */
int fgg_num_tiles(int kind);

/* Rank every tile config of `kind` for a problem of M rows (G experts; the
 * routing is unknown on the host, so every expert boundary is assumed to fall
 * inside a row window), N columns and K; `num_cus` the compute units (256 on
 * MI355X; <= 0 means query the current device).  Writes up to `max_out`
 * entries, best first, and returns how many were written, or -1 with
 * fgg_last_error() set. */
int fgg_rank_tiles(int kind, int M, int N, int K, int G, int num_cus, fgg_tile* out,
                   int max_out);
/* The same with the run_align promise of fgg_options (0 = none). */
int fgg_rank_tiles_aligned(int kind, int M, int N, int K, int G, int run_align, int num_cus,
                           fgg_tile* out, int max_out);

/* The ranking under a chosen form of the score (for comparing them; the
 * entry points always use FGG_SCORE_KEPT):
 *   FGG_SCORE_KEPT     m_eff * n_eff * busy * throughput, busy = tiles /
 *                      (num_waves * CUs * wg_per_cu): the page's structure
 *                      with the division by num_waves read as the busy
 *                      fraction of the last wave.  It equals throughput /
 *                      (num_waves * CUs * wg_per_cu * BM * BN) up to the
 *                      constant M * N, i.e. the inverse of a predicted
 *                      time (rounds of tiles times the per-tile time).
 *   FGG_SCORE_LITERAL  m_eff * n_eff * throughput / (num_waves * tile_n),
 *                      the page's printed form ("Code analysis 2") with
 *                      the terms defined as above. */
#define FGG_SCORE_KEPT 0
#define FGG_SCORE_LITERAL 1
int fgg_rank_tiles_variant(int kind, int M, int N, int K, int G, int run_align, int variant,
                           int num_cus, fgg_tile* out, int max_out);

/* Optional overrides for the *_ex entry points (NULL = defaults).  Initialise
 * the whole struct (e.g. `fgg_options o = {-1};` then set fields): a field
 * left out means 0, and new fields are only ever added at the end. */
typedef struct {
  int tile_id;         /* -1: use the ranker's top choice                    */
  int max_workgroups;  /* > 0: cap the persistent grid (testing / tuning)    */
  int run_split;       /* grouped calls: 0 automatic, < 0 never, > 0 always.
                        * Split mode runs each expert pass of a row window as
                        * its own workgroup (G items per tile, item r running
                        * expert r if the window holds a row of it) instead
                        * of one after the other; automatic mode uses it when
                        * every item runs at once on the device (small M:
                        * latency).  Results are identical either way.       */
  int run_align;       /* grouped calls: > 0 promises that every expert run
                        * starts at a row index that is a multiple of
                        * run_align (MoE alignment padding); the ranker then
                        * charges no two-expert windows to tile heights that
                        * divide it.  0: unknown.  Only the tile choice
                        * depends on it: results are correct whatever the
                        * routing (and identical to asking for that tile).    */
} fgg_options;

fgg_status grouped_fp8_gemm_ex(const void* A, const void* B, const float* a_scale,
                               const float* b_scale, const int32_t* m_indices, void* C,
                               int M, int N, int K, int G, const fgg_options* opt,
                               void* stream);
fgg_status fp4_gemm_ex(const void* A, const void* B, const void* a_scale, const void* b_scale,
                       float alpha, void* C, int M, int N, int K, const fgg_options* opt,
                       void* stream);
fgg_status grouped_fp4_gemm_ex(const void* A, const void* B, const void* a_scale,
                               const void* b_scale, const int32_t* m_indices, float alpha,
                               void* C, int M, int N, int K, int G, const fgg_options* opt,
                               void* stream);
fgg_status grouped_fp4_gemm_alpha_ex(const void* A, const void* B, const void* a_scale,
                                     const void* b_scale, const int32_t* m_indices,
                                     const float* alpha, void* C, int M, int N, int K, int G,
                                     const fgg_options* opt, void* stream);
/* run_split is ignored (a batch has no routing). */
fgg_status fp4_gemm_problems_ex(const fgg_fp4_problem* problems, int count,
                                const fgg_options* opt, void* stream);
fgg_status fp8_gemm_problems_ex(const fgg_fp8_problem* problems, int count,
                                const fgg_options* opt, void* stream);

/* ------------------------------------------------------------------------
 * Bounded autotuning of the ranker's top choices (the flashinfer#3948 page,
 * "Code analysis 1": rank the candidate configs with the heuristic and
 * profile only the top few instead of all of them).
 *
 * Each *_tune call takes the arguments of its GEMM (same checks, same
 * errors), times the ranker's best min(top_k, FGG_TUNE_MAX) tile configs on
 * those inputs and records the fastest for (kind, M, N, K, G) on the current
 * device.  Timing: three rounds that visit the configs in turn, each visit
 * one untimed launch and then `reps` launches between two HIP events on
 * `stream`; a config's time is its fastest round (so no config pays for the
 * clock ramp of a GPU coming out of idle, whatever its place in the order).
 * Later calls of that GEMM on that shape with no explicit tile_id launch the
 * recorded config instead of the ranker's top one.  `opt` (may be NULL) is
 * read as by the *_ex calls: run_align shapes the ranking the candidates
 * come from, max_workgroups and run_split apply to every timed launch, and
 * tile_id must be -1 (the tuning chooses it; FGG_EINVAL otherwise).  C is overwritten (with the GEMM's result).  The call
 * synchronises `stream` and is not graph-capturable; it allocates no device
 * memory.  `report` (may be NULL) receives the candidates in ranker order
 * with their milliseconds per launch.  Recorded choices are process-wide
 * and thread-safe; fgg_tune_clear() forgets them all.
 * ------------------------------------------------------------------------ */
#define FGG_TUNE_MAX 8

typedef struct {
  int n;                      /* candidates timed                              */
  int tile_id[FGG_TUNE_MAX];  /* ranker order: tile_id[0] is the heuristic's   */
  float ms[FGG_TUNE_MAX];     /* time per launch, fastest of the three rounds  */
  int best;                   /* index (into tile_id / ms) of the fastest      */
} fgg_tune_report;

fgg_status grouped_fp8_gemm_tune(const void* A, const void* B, const float* a_scale,
                                 const float* b_scale, const int32_t* m_indices, void* C, int M,
                                 int N, int K, int G, int top_k, int reps,
                                 fgg_tune_report* report, const fgg_options* opt, void* stream);
fgg_status fp4_gemm_tune(const void* A, const void* B, const void* a_scale, const void* b_scale,
                         float alpha, void* C, int M, int N, int K, int top_k, int reps,
                         fgg_tune_report* report, const fgg_options* opt, void* stream);
fgg_status grouped_fp4_gemm_tune(const void* A, const void* B, const void* a_scale,
                                 const void* b_scale, const int32_t* m_indices, float alpha,
                                 void* C, int M, int N, int K, int G, int top_k, int reps,
                                 fgg_tune_report* report, const fgg_options* opt,
                                 void* stream);

/* The recorded config for a shape on the current device (kind as
 * fgg_rank_tiles; G = 1 for fp4_gemm), or -1 when none is recorded. */
int fgg_tuned_tile(int kind, int M, int N, int K, int G);

/* Forget every recorded choice. */
void fgg_tune_clear(void);

/* Device facts cached once per device (gfx950 check, CU count, LDS bytes per
 * workgroup).  Returns FGG_EDEVICE when no usable device is present. */
fgg_status fgg_device_info(int* num_cus, int* lds_per_block, int* clock_khz, char* arch,
                           int arch_len);

#ifdef __cplusplus
}
#endif

#endif /* FGG_H */
