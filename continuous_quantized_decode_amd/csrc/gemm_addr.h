// gemm_addr.h -- address arithmetic of the GEMM's weight staging loads.
//
// Pure integer functions shared by the kernel (gemm.hip) and a host-side bounds check
// that enumerates every lane, instruction, super-block and tile shape (the check is
// compiled with a plain C++ compiler, so this header needs no HIP).
//
// A stage holds one super-block of the tile's 16 rows.  Load instruction i of lane l
// handles unit c = l + 64 i of the stage: the stage is the 16 row blocks one after the
// other, each cut into 16-byte units, so each instruction reads a few long contiguous
// runs; units past the stage's last one repeat it.  The rows' LDS stride is chosen so
// that the compute's reads (lane (n, g) reads row n at an offset of 4 g or 8 g bytes)
// spread evenly over the LDS banks: 144 bytes (36 dwords) for Q4_K, and for Q6_K one
// padding unit after each 224-byte window, 240 bytes (60 dwords), since 56 dwords would
// put rows n and n + 8 on the same banks.  A padding unit repeats a valid unit of the
// same row (its LDS destination is never read).
//
// Q4_K (144-byte blocks, 16-byte aligned): 9 chunks per row, 144 units per stage; unit c
// is row c / 9, chunk c % 9; LDS byte 16 c (row r at 144 r).
//
// Q6_K (210-byte blocks, 2-byte aligned): let A be a row block's address and s16 =
// A % 16 (even).  The row's window is the 224 bytes [A - s16, A - s16 + 224), i.e. 14
// whole 16-byte units: block byte b sits at window byte s16 + b, so the whole block
// (quants, scales and d) is inside.  Every unit is 16-byte aligned and starts inside the
// matrix (A - s16 >= the matrix start, which is 16-byte aligned), so a unit running past
// the matrix's end stays within the aligned 16 bytes holding that end (no page is
// crossed) and lies beyond the buffer descriptor's size.  14 units + 1 padding per row,
// 240 units per stage; unit c is row c / 15, window unit min(c % 15, 13); LDS byte 16 c
// (row r at 240 r).
#ifndef GR_GEMM_ADDR_H_
#define GR_GEMM_ADDR_H_

#include <stdint.h>

#ifdef __HIPCC__
#define GR_HD __host__ __device__ inline
#else
#define GR_HD inline
#endif

namespace gr {
namespace addr {

constexpr int kQ4Instr = 3;   // 16-byte loads per lane and stage (144 units)
constexpr int kQ6Instr = 4;   // 16-byte loads per lane and stage (240 units)
constexpr int kQ4RowUnits = 9;   // chunks per Q4_K row
constexpr int kQ4Units = 16 * kQ4RowUnits;
constexpr int kQ6RowUnits = 15;  // 14 window units + 1 padding per Q6_K row
constexpr int kQ6Units = 16 * kQ6RowUnits;

// Formats whose 256 weights take a multiple of 16 bytes in a row (Q4_K 144 B above; Q5_K
// 176 B; Q8_0, eight 34-byte blocks, 272 B) stage the same way: RU 16-byte units per row
// block, unit c is row c / RU, chunk c % RU, LDS byte 16 c (row r at 16 RU r).
constexpr int kQ5Instr = 3;       // 176 units per stage
constexpr int kQ5RowUnits = 11;
constexpr int kQ8Instr = 5;       // 272 units per stage
constexpr int kQ8RowUnits = 17;

GR_HD int al_unit(int lane, int i, int ru) { const int c = lane + 64 * i; return c < 16 * ru ? c : 16 * ru - 1; }
GR_HD int al_row(int c, int ru) { return c / ru; }
GR_HD uint32_t al_in_block(int c, int ru) { return 16u * (uint32_t)(c % ru); }
GR_HD uint32_t al_lds_byte(int r, uint32_t b, int ru) { return 16u * (uint32_t)ru * (uint32_t)r + b; }
GR_HD uint32_t al_lds(int lane, int i) { return 1024u * (uint32_t)i + 16u * (uint32_t)lane; }

// Byte offset from the tile's first row of tile row r: a ragged last tile (nvalid < 16
// rows inside the matrix) repeats its last row.
GR_HD uint32_t row_off(int r, int nvalid, uint32_t row_bytes) {
  return (uint32_t)(r < nvalid - 1 ? r : nvalid - 1) * row_bytes;
}

// Unit handled by lane `lane` in instruction i (clamped to the stage's last unit).
GR_HD int q4_unit(int lane, int i) { const int c = lane + 64 * i; return c < kQ4Units ? c : kQ4Units - 1; }
GR_HD int q6_unit(int lane, int i) { const int c = lane + 64 * i; return c < kQ6Units ? c : kQ6Units - 1; }

GR_HD int q4_row(int c) { return c / kQ4RowUnits; }
GR_HD uint32_t q4_in_block(int c) { return 16u * (uint32_t)(c % kQ4RowUnits); }  // byte offset in the row block

GR_HD int q6_row(int c) { return c / kQ6RowUnits; }

// Q6_K: s16 of a row block starting at an address with low 32 bits `addr_lo`.
GR_HD uint32_t q6_s16(uint32_t addr_lo) { return addr_lo & 15u; }

// Q6_K: per-lane constant of a unit: its offset from (the row's block address - s16),
// measured from the tile's block address.
GR_HD uint32_t q6_pre(uint32_t row_offset, int c) {
  const int u = c % kQ6RowUnits;
  return row_offset + 16u * (uint32_t)(u < 14 ? u : 13);
}

// Q6_K, rows of a multiple of 16 bytes (every row block has the tile's s16): the load
// address is (tile block address - s16) + pre.
// Q6_K, general rows: the load address is (tile block address - 16) + q6_rel(pre, s16),
// s16 that of the unit's row.
GR_HD uint32_t q6_rel(uint32_t pre, uint32_t s16) { return pre + 16u - s16; }

// Q6_K: LDS byte offset, within a stage, of block byte b of row r.
GR_HD uint32_t q6_lds_byte(int r, uint32_t b, uint32_t s16) { return 240u * (uint32_t)r + s16 + b; }

// Q4_K: LDS byte offset, within a stage, of block byte b of row r.
GR_HD uint32_t q4_lds_byte(int r, uint32_t b) { return 144u * (uint32_t)r + b; }

// LDS byte offset, within a stage, where lane `lane`'s load of instruction i lands.
// Whole-tile staging (the tile loop's Q4_K gate/up pairs): the workgroup's waves load a
// tile's 16 rows together; row r is the tile's bytes [r row_bytes, (r + 1) row_bytes),
// U = 9 nsb units of 16 bytes.  LDS unit L = 64 i + lane (load instruction i of the tile)
// holds row r = L / U's unit c = (L % U - rot) mod U: row r is rotated by rot = r units
// (2 r for odd U), so that reading one unit column of the 16 rows touches different LDS
// banks (4 (U r + rot) dwords: 4 (U + 1) r or 4 (U + 2) r mod 64, distinct for r < 16
// until the rotation wraps; a wrap moves a row by 4 U dwords, a multiple of 64 at
// K = 4096), and an instruction reads at most a few runs of consecutive bytes.  Units past the tile's last one repeat it;
// their LDS destination (inside the slot) is never read.  A wave's instruction k is
// wt_instr(wave, waves, k, nsb); those past the tile's last repeat it.
constexpr int kWtInstr = 5;  // the most load instructions per wave and tile
GR_HD int wt_units(int nsb) { return 9 * nsb; }
// rotation of row r, in units (below U)
GR_HD int wt_rot(int r, int U) { return ((U & 1) ? 2 * r : r) % U; }
GR_HD int wt_instrs(int nsb) { return (16 * 9 * nsb + 63) / 64; }
GR_HD uint32_t wt_slot_bytes(int nsb) { return 1024u * (uint32_t)wt_instrs(nsb); }
GR_HD int wt_instr(int wave, int nwaves, int k, int nsb) {
  const int i = wave + nwaves * k, n = wt_instrs(nsb);
  return i < n ? i : n - 1;
}
// byte offset, from the tile's first row, of the unit lane `lane` of instruction i loads
GR_HD uint32_t wt_src(int i, int lane, int nsb) {
  const int U = wt_units(nsb);
  int L = 64 * i + lane;
  if (L > 16 * U - 1) L = 16 * U - 1;
  const int r = L / U;
  int c = L - r * U - wt_rot(r, U);
  if (c < 0) c += U;
  return 16u * ((uint32_t)r * (uint32_t)U + (uint32_t)c);
}
// The same staging for a K range of nsb super-blocks of the tile's 16 rows when the rows
// are not consecutive in memory: byte offset, from row 0's first byte of the range, of the
// unit lane `lane` of instruction i loads (row r at r row_bytes); LDS layout as above.
GR_HD uint32_t wt_src_rows(int i, int lane, int nsb, uint32_t row_bytes) {
  const int U = wt_units(nsb);
  int L = 64 * i + lane;
  if (L > 16 * U - 1) L = 16 * U - 1;
  const int r = L / U;
  int c = L - r * U - wt_rot(r, U);
  if (c < 0) c += U;
  return (uint32_t)r * row_bytes + 16u * (uint32_t)c;
}
GR_HD uint32_t wt_lds(int i, int lane) { return 1024u * (uint32_t)i + 16u * (uint32_t)lane; }
// LDS byte holding byte b (< 16 U) of row r
GR_HD uint32_t wt_lds_byte(int r, uint32_t b, int nsb) {
  const int U = wt_units(nsb);
  int c = (int)(b / 16u) + wt_rot(r, U);
  if (c >= U) c -= U;
  return 16u * ((uint32_t)r * (uint32_t)U + (uint32_t)c) + b % 16u;
}

// K-chunk staging (the Q6_K residual GEMM -- down -- on rows of a multiple of 16 bytes):
// stage c holds super-blocks [C c, C c + C) of the tile's 16 rows.  Row r's window is
// kc_units(C) aligned 16-byte units from kc_window(C, c) bytes into the row (the chunk
// starts kc_s16 bytes in: 2-byte aligned, at most 14, so the window holds it whole).
// Windows sit kc_stride(C) units apart in LDS, an odd count, so one byte column of the 16
// rows falls on 16 different banks (4 stride r dwords; odd stride: distinct mod 64 for
// r < 16); the padding unit repeats the window's last.  LDS unit L = 64 i + lane of load
// instruction i is row L / stride, window unit min(L % stride, units - 1); units past the
// stage repeat its last, instructions past it repeat the last.
GR_HD int kc_units(int C) { return (14 + 210 * C + 15) / 16; }
GR_HD int kc_stride(int C) { return kc_units(C) | 1; }
GR_HD int kc_instrs(int C) { return (16 * kc_stride(C) + 63) / 64; }
GR_HD uint32_t kc_slot_bytes(int C) { return 1024u * (uint32_t)kc_instrs(C); }
GR_HD uint32_t kc_window(int C, int c) { return (210u * (uint32_t)C * (uint32_t)c) & ~15u; }
GR_HD uint32_t kc_s16(int C, int c) { return (210u * (uint32_t)C * (uint32_t)c) & 15u; }
GR_HD int kc_instr(int wave, int waves, int k, int C) {
  const int i = wave + waves * k, n = kc_instrs(C);
  return i < n ? i : n - 1;
}
// byte offset of the unit lane `lane` of instruction i loads, from row 0's window start
GR_HD uint32_t kc_src(int i, int lane, int C, uint32_t row_bytes) {
  const int S = kc_stride(C), U = kc_units(C);
  int L = 64 * i + lane;
  if (L > 16 * S - 1) L = 16 * S - 1;
  const int r = L / S;
  int col = L - r * S;
  if (col > U - 1) col = U - 1;
  return (uint32_t)r * row_bytes + 16u * (uint32_t)col;
}
GR_HD uint32_t kc_lds(int i, int lane) { return 1024u * (uint32_t)i + 16u * (uint32_t)lane; }
GR_HD uint32_t kc_lds_byte(int r, uint32_t b, int C) { return 16u * (uint32_t)kc_stride(C) * (uint32_t)r + b; }

GR_HD uint32_t q4_lds(int lane, int i) { return 1024u * (uint32_t)i + 16u * (uint32_t)lane; }
GR_HD uint32_t q6_lds(int lane, int i) { return 1024u * (uint32_t)i + 16u * (uint32_t)lane; }

}  // namespace addr
}  // namespace gr

#endif  // GR_GEMM_ADDR_H_
