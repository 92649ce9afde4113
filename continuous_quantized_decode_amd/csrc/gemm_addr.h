// gemm_addr.h -- address arithmetic of the GEMM's weight staging loads.
//
// Pure integer functions shared by the kernel (gemm.hip) and a host-side bounds check
// that enumerates every lane, instruction, super-block and tile shape (the check is
// compiled with a plain C++ compiler, so this header needs no HIP).
//
// A stage holds one super-block of the tile's 16 rows.  Load instruction i of lane l
// handles unit c = l + 64 i of the stage: the stage is the 16 row blocks one after the
// other, cut into units (16-byte chunks for Q4_K, dwords for Q6_K), so each
// instruction reads a few long contiguous runs.  Units past the stage's last one
// repeat the last unit (their LDS destinations are padding).
//
// Q4_K (144-byte blocks, 16-byte aligned): 9 chunks per row, 144 per stage; chunk c
// is row c / 9, bytes 16 (c % 9) of its block; LDS byte 16 c.
//
// Q6_K (210-byte blocks, 2-byte aligned): let A be a row block's address and s16 =
// A % 16 (even).  The row's window is the 224 bytes [A - s16, A - s16 + 224), i.e. 14
// whole 16-byte units: block byte b sits at window byte s16 + b, so the whole block
// (quants, scales and d) is inside.  Every unit is 16-byte aligned and starts inside the
// matrix (A - s16 >= the matrix start, which is 16-byte aligned), so a unit running past
// the matrix's end stays within the aligned 16 bytes holding that end (no page is
// crossed) and lies beyond the buffer descriptor's size.  Unit c of a stage is row
// c / 14, window unit c % 14; LDS byte 16 c.
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

constexpr int kQ4Instr = 3;   // 16-byte loads per lane and stage (144 chunks)
constexpr int kQ6Instr = 4;   // 16-byte loads per lane and stage (224 units)
constexpr int kQ4Units = 144;
constexpr int kQ6RowUnits = 14;  // 16-byte units per Q6_K row window
constexpr int kQ6Units = 16 * kQ6RowUnits;

// Byte offset from the tile's first row of tile row r: a ragged last tile (nvalid < 16
// rows inside the matrix) repeats its last row.
GR_HD uint32_t row_off(int r, int nvalid, uint32_t row_bytes) {
  return (uint32_t)(r < nvalid - 1 ? r : nvalid - 1) * row_bytes;
}

// Unit handled by lane `lane` in instruction i (clamped to the stage's last unit).
GR_HD int q4_unit(int lane, int i) { const int c = lane + 64 * i; return c < kQ4Units ? c : kQ4Units - 1; }
GR_HD int q6_unit(int lane, int i) { const int c = lane + 64 * i; return c < kQ6Units ? c : kQ6Units - 1; }

GR_HD int q4_row(int c) { return c / 9; }
GR_HD uint32_t q4_in_block(int c) { return 16u * (uint32_t)(c % 9); }  // byte offset in the row block

GR_HD int q6_row(int c) { return c / kQ6RowUnits; }

// Q6_K: s16 of a row block starting at an address with low 32 bits `addr_lo`.
GR_HD uint32_t q6_s16(uint32_t addr_lo) { return addr_lo & 15u; }

// Q6_K: per-lane constant of a unit: its offset from (the row's block address - s16),
// measured from the tile's block address.
GR_HD uint32_t q6_pre(uint32_t row_offset, int c) { return row_offset + 16u * (uint32_t)(c % kQ6RowUnits); }

// Q6_K, rows of a multiple of 16 bytes (every row block has the tile's s16): the load
// address is (tile block address - s16) + pre.
// Q6_K, general rows: the load address is (tile block address - 16) + q6_rel(pre, s16),
// s16 that of the unit's row.
GR_HD uint32_t q6_rel(uint32_t pre, uint32_t s16) { return pre + 16u - s16; }

// Q6_K: LDS byte offset, within a stage, of block byte b of row r.
GR_HD uint32_t q6_lds_byte(int r, uint32_t b, uint32_t s16) { return 224u * (uint32_t)r + s16 + b; }

// LDS byte offset, within a stage, where lane `lane`'s load of instruction i lands.
GR_HD uint32_t q4_lds(int lane, int i) { return 1024u * (uint32_t)i + 16u * (uint32_t)lane; }
GR_HD uint32_t q6_lds(int lane, int i) { return 1024u * (uint32_t)i + 16u * (uint32_t)lane; }

}  // namespace addr
}  // namespace gr

#endif  // GR_GEMM_ADDR_H_
