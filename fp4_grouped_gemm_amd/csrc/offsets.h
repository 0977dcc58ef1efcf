// Buffer offsets of the staging loads, shared by the kernels (device) and a
// host check that enumerates every load of a launch (tests/offsets_check.cpp).
// Plain integer arithmetic, no HIP types.
//
// Every staging load reads through a raw buffer resource over one tile's
// rows (or a whole operand).  The resource's range check covers the VGPR
// offset of the load; the functions below put each lane's row (and the
// parts that depend on the lane) in that offset, so that a row past the
// tile's last row fails the check and reads zeros, and keep the SGPR
// offset to a displacement inside the row.  kSkip is past every buffer
// (all are below 2^31 bytes): loads that are not needed read zeros there.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define FGG_HD __host__ __device__ __forceinline__
#else
#define FGG_HD inline
#endif

namespace fgg {
namespace off {

constexpr uint32_t kSkip = 0x80000000u;

// ---- grouped FP8 (tile rows of K bytes, K steps of 128 bytes) -------------
// LDS layout of a staged tile: row r at 128 r, its 16-byte chunk c at
// physical chunk c ^ fp8_swz_key(r).  A 16-byte LDS read serves a wave's 64
// lanes in four cycles of 16 lanes, grouping the lanes with equal bit 5 and
// equal parity of bits 2..4 of the lane index (measured with the LDS
// bank-conflict counter on gfx950); a cycle's 16 lanes must hit 16 distinct
// 16-byte bank groups of a 256-byte bank line (two tile rows).  A fragment
// read gives lane l row r0 + l % 16 (r0 a multiple of 16) and chunk
// 2 (l / 16) or 2 (l / 16) + 1.  Within one cycle, the 8 lanes of each row
// parity then see rows bits (1, 2, 3) and chunk bit 1 (lane bit 4) tied by
// the parity; the key (row bit 1, row bit 2, row bits 2 ^ 3) maps those 8
// lanes to 8 distinct chunks.
FGG_HD int fp8_swz_key(int row) {
  return ((row >> 1) & 1) | (((row >> 2) & 1) << 1) | ((((row >> 2) ^ (row >> 3)) & 1) << 2);
}
FGG_HD int fp8_lds_off(int row, int chunk) { return (row << 7) | ((chunk ^ fp8_swz_key(row)) << 4); }
// One 16-byte direct-to-LDS load per lane moves 8 tile rows (64 lanes x 16
// bytes): lane l writes physical chunk l % 8 of row 8 b + l / 8 of load b,
// so it reads logical chunk (l % 8) ^ fp8_swz_key(row).  For load s of wave
// w (W waves, W even), row = 8 (s W + w) + l / 8, whose bits 1..3 (all the
// key reads) depend on w % 2 and l / 8 only.
FGG_HD uint32_t fp8_lane_off(int wave, int lane, uint32_t K) {
  const int r8 = lane >> 3;
  const int chunk = (lane & 7) ^ fp8_swz_key(((wave & 1) << 3) + r8);
  return (uint32_t)(wave * 8 + r8) * K + (uint32_t)(chunk << 4);
}
// VGPR offset of load s (rows 8 (s W + w) ..) of a wave; kSkip when the load
// is not needed.  The SGPR offset is fp8_step_soff(kb).
FGG_HD uint32_t fp8_tile_voff(uint32_t lane_off, int s, int waves, uint32_t K, bool need) {
  return need ? lane_off + (uint32_t)(s * waves * 8) * K : kSkip;
}
FGG_HD uint32_t fp8_step_soff(int kb) { return (uint32_t)kb * 128u; }
// a_scale chunk c (sa_blk K blocks of every tile row, sa_row floats per row
// in LDS): 4-byte load g of the chunk reads row g / sa_row, block
// c sa_blk + g % sa_row; blocks past the row's last read zeros.
FGG_HD uint32_t fp8_scale_voff(int g, int c, int sa_blk, int sa_row, int nkb) {
  const uint32_t blk = (uint32_t)(c * sa_blk) + (uint32_t)g % (uint32_t)sa_row;
  return blk < (uint32_t)nkb ? ((uint32_t)g / (uint32_t)sa_row * (uint32_t)nkb + blk) * 4u : kSkip;
}

// ---- NVFP4 (rows of Kp = K / 2 packed bytes and Ks = K / 16 scale bytes) --
// Staging unit g covers half a 64-element K step of tile row g / 2: the 16
// packed bytes at g % 2 * 16 of the step; the step's 32 bytes are the SGPR
// offset fp4_code_soff(ks).
FGG_HD uint32_t fp4_code_voff(int g, uint32_t Kp) {
  return (uint32_t)(g >> 1) * Kp + (uint32_t)(g & 1) * 16u;
}
FGG_HD uint32_t fp4_code_soff(int ks) { return (uint32_t)ks * 32u; }
// The scale codes of four steps [4c, 4c + 4) of row g / 2: 16 bytes at 16 c
// of the row, the whole offset in the VGPR (row_off = row * Ks, or kSkip).
FGG_HD uint32_t fp4_scale_row_off(int g, uint32_t Ks) { return (uint32_t)(g >> 1) * Ks; }
FGG_HD uint32_t fp4_scale_voff(uint32_t row_off, int c) { return row_off + (uint32_t)c * 16u; }

// ---- W4A16 (BF16 activation rows of K values, groups of 256) --------------
// LDS layout of a staged activation group: row r (0..31) at 512 r, its
// 16-byte chunk c (0..31) at physical chunk c ^ w4a16_swz_key(r).  A
// fragment read gives lane l row 16 rb + l % 16 and chunk 8 (l / 16) + t;
// under the 16-lane read grouping (see the FP8 layout above) the key (row
// bits 0, 1, 2 ^ 3, 3, 4) gives each cycle's lanes 16 distinct bank groups
// (row bits 0..4 as the key would give 8).
FGG_HD int w4a16_swz_key(int row) {
  return (row & 3) | ((((row >> 2) ^ (row >> 3)) & 1) << 2) | (row & 24);
}
FGG_HD int w4a16_lds_off(int row, int chunk) { return row * 512 + ((chunk ^ w4a16_swz_key(row)) << 4); }
// Chunk lc (8 values) of group gc of activation row `row`; chunks at or past
// K read zeros.
FGG_HD uint32_t w4a16_act_voff(uint32_t row, int lc, int gc, int K) {
  return gc * 256 + lc * 8 < K ? row * (uint32_t)K * 2u + (uint32_t)(gc * 512 + lc * 16) : kSkip;
}

// Weights (packed E2M1 rows of Kp = K / 2 bytes, one row per output
// column): a staged group holds a wave's 32 weight rows x 128 bytes (256
// codes each), row w (0..31) at 128 w, its 16-byte chunk c (0..7) at
// physical chunk c ^ w4a16_wkey(w).  A fragment read gives lane l row
// 16 b + l % 16 and chunk 2 (l / 16) + h; under the 16-lane read grouping
// the key (row bit 1 as key bit 0, row bit 2 as key bit 2) gives each
// cycle's lanes 16 distinct bank groups.
FGG_HD int w4a16_wkey(int row) { return ((row >> 1) & 1) | (((row >> 2) & 1) << 2); }
FGG_HD int w4a16_w_lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ w4a16_wkey(row)) << 4);
}
// Chunk lc (16 bytes, 32 codes) of group g of weight row `row`; chunks at
// or past the row's end (the half-full last group when K is an odd
// multiple of 128) read zeros.
FGG_HD uint32_t w4a16_w_voff(uint32_t row, int lc, int g, uint32_t Kp) {
  const uint32_t b = (uint32_t)g * 128u + (uint32_t)lc * 16u;
  return b < Kp ? row * Kp + b : kSkip;
}
// The 16 scale bytes of group g of weight row `row` (rows of Ks = K / 16
// bytes), the whole offset in the VGPR: the half-full last group's second
// half reads the next row's first codes, or zeros past the buffer's end
// (the range check goes dword by dword); the kernel zeroes the scales of
// the lanes past K.
FGG_HD uint32_t w4a16_s_voff(uint32_t row, int g, uint32_t Ks) {
  return row * Ks + (uint32_t)g * 16u;
}

}  // namespace off
}  // namespace fgg
