// Host check of the staging loads' buffer offsets (fp4_grouped_gemm_amd/
// csrc/offsets.h, the functions the kernels call): for every tile config,
// every load of a pass is enumerated on tail shapes (a tile's last rows,
// short and long K), and every access whose VGPR offset passes the range
// check must lie inside the row it is meant for and inside the buffer; an
// access that fails the check reads zeros and touches nothing.  The FP8
// tiles' and the W4A16 activation and weight stages' LDS layouts are checked too: the
// loads put every chunk where the fragment reads look for it, and those
// reads are free of bank conflicts.
//
//   g++ -O1 -std=c++17 -I fp4_grouped_gemm_amd/csrc tests/offsets_check.cpp -o offsets_check
//
// Exit status 0 and a summary line when every access is in bounds.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "offsets.h"

using namespace fgg::off;

static long long checked = 0, skipped = 0, bad = 0;

// An access of `size` bytes at voff + soff through a buffer of `records`
// bytes, meant for bytes [lo, hi) of the buffer.
static void access(uint64_t voff, uint64_t soff, uint64_t size, uint64_t records, uint64_t lo,
                   uint64_t hi, const char* what) {
  if (voff >= records) {  // fails the range check: zeros, no access
    ++skipped;
    return;
  }
  ++checked;
  const uint64_t a = voff + soff, b = a + size;
  if (a < lo || b > hi || b > records) {
    if (++bad <= 10)
      std::printf("OUT OF BOUNDS %s: [%llu, %llu) not in [%llu, %llu), records %llu\n", what,
                  (unsigned long long)a, (unsigned long long)b, (unsigned long long)lo,
                  (unsigned long long)hi, (unsigned long long)records);
  }
}

struct Fp8Cfg {
  int BM, BN, WAVES, SA_BLK, SA_ROW;
};

static void check_fp8(const Fp8Cfg& c, int rows, int K, bool is_a) {
  const int nkb = K / 128;
  const int tile_rows = is_a ? c.BM : c.BN;
  const int loads = tile_rows / 8 / c.WAVES;
  const uint64_t records = (uint64_t)rows * K;
  for (int w = 0; w < c.WAVES; ++w)
    for (int lane = 0; lane < 64; ++lane) {
      const uint32_t lo = fp8_lane_off(w, lane, (uint32_t)K);
      for (int s = 0; s < loads; ++s) {
        const uint64_t row = 8ull * (s * c.WAVES + w) + lane / 8;
        const uint32_t v = fp8_tile_voff(lo, s, c.WAVES, (uint32_t)K, true);
        if (v != kSkip && v / K != row) {
          ++bad;
          std::printf("FP8 load s=%d w=%d lane=%d reads row %u, not %llu\n", s, w, lane, v / K,
                      (unsigned long long)row);
        }
        for (int kb = 0; kb < nkb; ++kb)
          access(v, fp8_step_soff(kb), 16, records, row * K, (row + 1) * K,
                 is_a ? "fp8 A tile" : "fp8 B tile");
        // a load that is not needed
        access(fp8_tile_voff(lo, s, c.WAVES, (uint32_t)K, false), 0, 16, records, 0, 0,
               "fp8 skipped load");
      }
    }
  if (is_a) {  // the a_scale chunks of the tile rows
    const uint64_t srec = (uint64_t)rows * nkb * 4;
    const int chunks = (nkb + c.SA_BLK - 1) / c.SA_BLK + 1;
    for (int ch = 0; ch < chunks; ++ch)
      for (int g = 0; g < c.BM * c.SA_ROW; ++g) {
        const uint64_t row = g / c.SA_ROW;
        access(fp8_scale_voff(g, ch, c.SA_BLK, c.SA_ROW, nkb), 0, 4, srec, row * nkb * 4,
               (row + 1) * nkb * 4, "fp8 a_scale");
      }
  }
}

// The LDS side of the FP8 staging: the direct-to-LDS loads (lane l of load
// b writes bytes [16 l, 16 l + 16) of the load's 1 KB) must put tile row r,
// chunk c where the fragment reads look for it (fp8_lds_off), and each
// 16-lane cycle of a fragment read (lanes with equal bit 5 and equal parity
// of bits 2..4) must hit 16 distinct 16-byte bank groups.
static long long layout_checked = 0;
static void check_fp8_layout(const Fp8Cfg& c, int tile_rows) {
  const uint32_t K = 1024;  // any row length: the chunk is the in-row offset
  std::vector<int> at(tile_rows * 8, -1);  // physical 16-byte slot -> row * 8 + chunk
  for (int w = 0; w < c.WAVES; ++w)
    for (int lane = 0; lane < 64; ++lane)
      for (int s = 0; s < tile_rows / 8 / c.WAVES; ++s) {
        const uint32_t v = fp8_tile_voff(fp8_lane_off(w, lane, K), s, c.WAVES, K, true);
        const int slot = (s * c.WAVES + w) * 64 + lane;
        at[slot] = (int)(v / K) * 8 + (int)(v % K) / 16;
      }
  for (int row = 0; row < tile_rows; ++row)
    for (int ch = 0; ch < 8; ++ch) {
      ++layout_checked;
      if (at[fp8_lds_off(row, ch) / 16] != row * 8 + ch && ++bad <= 10)
        std::printf("FP8 LDS layout: row %d chunk %d is not where the fragment read looks\n", row,
                    ch);
    }
  for (int r0 = 0; r0 < tile_rows; r0 += 16)
    for (int half = 0; half < 2; ++half)
      for (int cyc = 0; cyc < 4; ++cyc) {
        int seen = 0;
        for (int lane = 0; lane < 64; ++lane) {
          const int par = ((lane >> 2) ^ (lane >> 3) ^ (lane >> 4)) & 1;
          if (((lane >> 5) & 1) * 2 + par != cyc) continue;
          const int bank = (fp8_lds_off(r0 + (lane & 15), 2 * (lane >> 4) + half) / 16) % 16;
          seen |= 1 << bank;
        }
        ++layout_checked;
        if (seen != 0xffff && ++bad <= 10)
          std::printf("FP8 fragment read rows %d.. half %d cycle %d: bank conflict\n", r0, half, cyc);
      }
}

// The W4A16 activation stage: staging chunk p (row p / 32, physical chunk
// p % 32) fetches logical chunk (p % 32) ^ key(row), which must be where
// the fragment reads look for it; each 16-lane cycle of a read (rows
// 16 rb + l % 16, chunk 8 (l / 16) + t) must hit 16 distinct bank groups.
static void check_w4a16_layout() {
  for (int p = 0; p < 32 * 32; ++p) {
    const int row = p / 32, phys = p % 32;
    const int lc = phys ^ w4a16_swz_key(row);
    ++layout_checked;
    if (w4a16_lds_off(row, lc) != row * 512 + phys * 16 && ++bad <= 10)
      std::printf("W4A16 layout: row %d chunk %d misplaced\n", row, lc);
  }
  for (int rb = 0; rb < 2; ++rb)
    for (int t = 0; t < 8; ++t)
      for (int cyc = 0; cyc < 4; ++cyc) {
        int seen = 0;
        for (int lane = 0; lane < 64; ++lane) {
          const int par = ((lane >> 2) ^ (lane >> 3) ^ (lane >> 4)) & 1;
          if (((lane >> 5) & 1) * 2 + par != cyc) continue;
          seen |= 1 << ((w4a16_lds_off(16 * rb + (lane & 15), 8 * (lane >> 4) + t) / 16) % 16);
        }
        ++layout_checked;
        if (seen != 0xffff && ++bad <= 10)
          std::printf("W4A16 read rb %d t %d cycle %d: bank conflict\n", rb, t, cyc);
      }
}

// W4A16 weight staging: a wave's rows of Kp packed bytes (Ks scale bytes),
// every whole-line load and scale load of every group.  Used code bytes
// stay inside their row; chunks past the row's end read zeros.  Scale
// loads must keep their used bytes (those of k below K) inside the row;
// the rest may run into the next row or, past the buffer's end, read zeros.
static void check_w4a16_weights(int rows, int K) {
  const uint32_t Kp = K / 2, Ks = K / 16;
  const int ngroups = (K + 255) / 256;
  const uint64_t crec = (uint64_t)rows * Kp, srec = (uint64_t)rows * Ks;
  for (int g = 0; g < ngroups; ++g)
    for (int row = 0; row < rows; ++row) {
      for (int lc = 0; lc < 8; ++lc)
        access(w4a16_w_voff((uint32_t)row, lc, g, Kp), 0, 16, crec, (uint64_t)row * Kp,
               (uint64_t)(row + 1) * Kp, "w4a16 weight codes");
      const uint64_t used = Ks - 16ull * g < 16 ? Ks - 16ull * g : 16;
      access(w4a16_s_voff((uint32_t)row, g, Ks), 0, used, srec, (uint64_t)row * Ks,
             (uint64_t)(row + 1) * Ks, "w4a16 weight scales (used bytes)");
    }
}

// Where the whole-line loads put each weight chunk (load j, lane l: row
// 8 j + l / 8, physical chunk l % 8, logical chunk (l % 8) ^ key) against
// where the fragment reads look for it, and the reads' banks.
static void check_w4a16_weight_layout() {
  for (int j = 0; j < 4; ++j)
    for (int l = 0; l < 64; ++l) {
      const int row = 8 * j + l / 8, lc = (l % 8) ^ w4a16_wkey(row);
      ++layout_checked;
      if (w4a16_w_lds_off(row, lc) != 1024 * j + 16 * l && ++bad <= 10)
        std::printf("W4A16 weight layout: load %d lane %d misplaced\n", j, l);
    }
  for (int b = 0; b < 2; ++b)
    for (int h = 0; h < 2; ++h)
      for (int cyc = 0; cyc < 4; ++cyc) {
        int seen = 0;
        for (int lane = 0; lane < 64; ++lane) {
          const int par = ((lane >> 2) ^ (lane >> 3) ^ (lane >> 4)) & 1;
          if (((lane >> 5) & 1) * 2 + par != cyc) continue;
          seen |= 1 << ((w4a16_w_lds_off(16 * b + (lane & 15), 2 * (lane >> 4) + h) / 16) % 16);
        }
        ++layout_checked;
        if (seen != 0xffff && ++bad <= 10)
          std::printf("W4A16 weight read b %d h %d cycle %d: bank conflict\n", b, h, cyc);
      }
}

static void check_fp4(int BM, int rows, int K) {
  const uint32_t Kp = K / 2, Ks = K / 16;
  const int nks = K / 64;
  const uint64_t crec = (uint64_t)rows * Kp, srec = (uint64_t)rows * Ks;
  for (int g = 0; g < 2 * BM; ++g) {
    const uint64_t row = g / 2;
    const uint32_t v = fp4_code_voff(g, Kp);
    for (int ks = 0; ks < nks; ++ks)
      access(v, fp4_code_soff(ks), 16, crec, row * Kp, (row + 1) * Kp, "fp4 codes");
    // scale groups up to one past the last (the kernel loads a group ahead);
    // only the codes of steps below nks are used, and those must be in the
    // row; the rest of a 16-byte load may run into the next row, and past
    // the buffer's end the range check (dword by dword) returns zeros
    const uint32_t ro = fp4_scale_row_off(g, Ks);
    for (int c = 0; c <= nks / 4 + 1; ++c) {
      const int used = nks - 4 * c < 4 ? nks - 4 * c : 4;
      if (used <= 0) {
        access(fp4_scale_voff(ro, c), 0, 0, srec, 0, srec, "fp4 scales past the last step");
        continue;
      }
      access(fp4_scale_voff(ro, c), 0, 4ull * used, srec, row * Ks, (row + 1) * Ks,
             "fp4 scales (used bytes)");
    }
  }
}

static void check_w4a16(int M, int K) {
  const uint64_t rec = (uint64_t)M * K * 2;
  const int ngroups = (K + 255) / 256;
  for (int row : {0, M / 2, M - 1})
    for (int gc = 0; gc < ngroups; ++gc)
      for (int lc = 0; lc < 32; ++lc)
        access(w4a16_act_voff((uint32_t)row, lc, gc, K), 0, 16, rec, (uint64_t)row * K * 2,
               (uint64_t)(row + 1) * K * 2, "w4a16 activations");
}

int main() {
  const Fp8Cfg fp8[] = {{256, 256, 8, 8, 8}, {256, 128, 8, 3, 4}, {128, 256, 8, 3, 4},
                        {128, 128, 4, 3, 4}};
  for (const Fp8Cfg& c : fp8) {
    check_fp8_layout(c, c.BM);
    check_fp8_layout(c, c.BN);
  }
  for (const Fp8Cfg& c : fp8)
    for (int K : {128, 384, 640, 7168})
      for (int rows : {1, 7, 8, 9, 63, 64, 65, 127, 128, 129, 255, 256}) {
        if (rows <= c.BM) check_fp8(c, rows, K, true);
        if (rows <= c.BN) check_fp8(c, rows, K, false);
      }
  for (int BM : {128, 256})
    for (int K : {128, 256, 384, 640, 4608})
      for (int rows : {1, 2, 63, 64, 65, 127, 128, 255, 256})
        if (rows <= BM) check_fp4(BM, rows, K);
  for (int K : {128, 384, 640, 1408, 8192})
    for (int M : {1, 2, 33, 1025}) check_w4a16(M, K);
  check_w4a16_layout();
  for (int K : {128, 384, 640, 1408, 8192})
    for (int rows : {1, 2, 31, 32}) check_w4a16_weights(rows, K);
  check_w4a16_weight_layout();
  std::printf("offsets: %lld accesses checked in range, %lld skipped by the range check, %lld LDS "
              "layout and bank checks, %lld failed\n", checked, skipped, layout_checked, bad);
  return bad == 0 ? 0 : 1;
}
