"""Host-side check of the GEMM kernel's weight-staging addresses (CPU only).

The kernel computes every direct-to-LDS load address with the integer functions of
continuous_quantized_decode_amd/csrc/gemm_addr.h.  This test compiles that header
into a small C++ program that enumerates every tile shape, ragged last tile,
super-block, lane and load instruction and checks that:
  * every load lies inside the weight matrix (no read before its start or past its end);
  * Q4_K, Q5_K and Q8_0 loads are 16-byte chunks inside their row block (Q5_K: 176 B,
    Q8_0: eight 34-byte blocks, 272 B, per 256 weights);
  * Q6_K loads are 16-byte aligned units starting inside [block - s16, block + 210); a
    unit may end past the matrix only inside the aligned 16 bytes that hold its end (no
    page is crossed);
  * no LDS write leaves the stage;
  * every LDS byte the compute reads (all bytes of row r's Q4_K / Q6_K block, at
    gemm_addr.h's q4_lds_byte / q6_lds_byte) holds the right byte of the matrix after
    the stage's loads, and Q8_0's three-dword reads around 2-byte aligned offsets stay
    inside the stage.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "continuous_quantized_decode_amd", "csrc", "gemm_addr.h")

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "gemm_addr.h"
using namespace gr::addr;

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { if (fails++ < 20) { std::printf(__VA_ARGS__); std::printf("\n"); } } } while (0)

int main() {
  const int nsbs[] = {1, 2, 3, 4, 5, 7, 12, 16, 48, 56, 57};
  const int rows[] = {1, 2, 15, 16, 17, 31, 33, 48};
  // 0: Q4_K, 1: Q6_K, 2: Q5_K, 3: Q8_0
  for (int wt = 0; wt < 4; ++wt) {
    const uint32_t bb = wt == 0 ? 144 : wt == 1 ? 210 : wt == 2 ? 176 : 272;
    const int ni = wt == 0 ? kQ4Instr : wt == 1 ? kQ6Instr : wt == 2 ? kQ5Instr : kQ8Instr;
    const int ru = wt == 2 ? kQ5RowUnits : kQ8RowUnits;
    const int stage = ni * 64 * 16;
    for (int nsb : nsbs) for (int N : rows) {
      const uint32_t row_bytes = bb * nsb;
      const uint64_t total = (uint64_t)N * row_bytes;  // the matrix starts 16-byte aligned, at 0
      for (int row0 = 0; row0 < N; row0 += 16) {
        const int nvalid = N - row0 < 16 ? N - row0 : 16;
        const uint64_t tile = (uint64_t)row0 * row_bytes;
        for (int sb = 0; sb < nsb; ++sb) {
          std::vector<int64_t> held(stage, -1);  // global byte address held by each LDS byte
          for (int lane = 0; lane < 64; ++lane) {
            for (int i = 0; i < ni; ++i) {
              uint64_t a; uint32_t len, lds;
              bool ok_end = false;  // a Q6_K unit may end past the matrix inside its last aligned 16 bytes
              if (wt == 0) {
                const int c = q4_unit(lane, i);
                const uint64_t blk = tile + row_off(q4_row(c), nvalid, row_bytes) + (uint64_t)sb * bb;
                a = blk + q4_in_block(c); len = 16; lds = q4_lds(lane, i);
                CHECK(a >= blk && a + len <= blk + bb, "q4 load leaves its row block");
              } else if (wt >= 2) {
                const int c = al_unit(lane, i, ru);
                const uint64_t blk = tile + row_off(al_row(c, ru), nvalid, row_bytes) + (uint64_t)sb * bb;
                a = blk + al_in_block(c, ru); len = 16; lds = al_lds(lane, i);
                CHECK(a >= blk && a + len <= blk + bb, "aligned-format load leaves its row block");
              } else {
                // exactly the kernel's arithmetic: a per-lane constant and the tile's
                // block address, with s16 from the tile (rows of a multiple of 16 bytes)
                // or from the unit's row (general)
                const int c = q6_unit(lane, i);
                const uint32_t pre = q6_pre(row_off(q6_row(c), nvalid, row_bytes), c);
                const uint64_t tblk = tile + (uint64_t)sb * bb;
                const uint64_t blk = tile + row_off(q6_row(c), nvalid, row_bytes) + (uint64_t)sb * bb;
                const uint32_t s16 = q6_s16((uint32_t)blk);
                if (row_bytes % 16 == 0) {
                  const uint32_t t16 = q6_s16((uint32_t)tblk);
                  CHECK(t16 == s16, "tile s16 differs from the row's");
                  a = tblk - t16 + pre;
                } else {
                  CHECK(q6_s16((uint32_t)tblk + pre) == s16, "row s16 from the lane constant is wrong");
                  a = tblk - 16 + q6_rel(pre, q6_s16((uint32_t)tblk + pre));
                }
                len = 16; lds = q6_lds(lane, i);
                CHECK(a % 16 == 0 && a + s16 >= blk && a < blk + 210, "q6 unit does not start in [blk - s16, blk + 210)");
                // past the matrix end only inside the aligned 16 bytes holding the end
                ok_end = a % 16 == 0 && a < total;
              }
              CHECK(a < total && (a + len <= total || ok_end), "wt %d nsb %d N %d row0 %d sb %d lane %d i %d: [%llu,+%u) outside %llu",
                    wt, nsb, N, row0, sb, lane, i, (unsigned long long)a, len, (unsigned long long)total);
              CHECK(lds + len <= (uint32_t)stage, "LDS write past the stage");
              for (uint32_t k = 0; k < len && lds + k < (uint32_t)stage; ++k)
                held[lds + k] = a + k < total ? (int64_t)(a + k) : -2;  // bytes past the matrix read as garbage
            }
          }
          // every byte the compute reads holds the right global byte
          for (int r = 0; r < 16; ++r) {
            const uint64_t blk = tile + row_off(r, nvalid, row_bytes) + (uint64_t)sb * bb;
            if (wt >= 2) {
              for (uint32_t b = 0; b < bb; ++b)
                CHECK(held[al_lds_byte(r, b, ru)] == (int64_t)(blk + b), "wt %d nsb %d N %d row0 %d sb %d row %d byte %u",
                      wt, nsb, N, row0, sb, r, b);
              if (wt == 3)  // d at 34 j, codes at 34 j + 2 + 8 kg: dwords [off & ~3, +12)
                for (int j = 0; j < 8; ++j)
                  for (int kg = 0; kg < 4; ++kg) {
                    const uint32_t off = 34 * j + 2 + 8 * kg;
                    CHECK(off % 2 == 0 && al_lds_byte(r, (off & ~3u) + 12, ru) <= (uint32_t)stage, "q8 read past the stage");
                  }
            } else if (wt == 0) {
              for (int b = 0; b < 144; ++b)
                CHECK(held[q4_lds_byte(r, b)] == (int64_t)(blk + b), "q4 nsb %d N %d row0 %d sb %d row %d byte %d", nsb, N,
                      row0, sb, r, b);
            } else {
              const uint32_t s16 = q6_s16((uint32_t)blk);
              for (uint32_t b = 0; b < 210; ++b)
                CHECK(held[q6_lds_byte(r, b, s16)] == (int64_t)(blk + b), "q6 nsb %d N %d row0 %d sb %d row %d byte %u s16 %u",
                      nsb, N, row0, sb, r, b, s16);
            }
          }
        }
      }
    }
  }
  std::printf("%s (%d failures)\n", fails ? "FAIL" : "ok", fails);
  return fails ? 1 : 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_gemm_staging_loads_stay_in_bounds_and_land_where_read():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "check.cpp")
        exe = os.path.join(d, "check")
        with open(src, "w") as f:
            f.write(PROGRAM)
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.dirname(HDR), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        print(out.stdout)
        assert out.returncode == 0, out.stdout


WHOLE_TILE_PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "gemm_addr.h"
using namespace gr::addr;

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { if (fails++ < 20) { std::printf(__VA_ARGS__); std::printf("\n"); } } } while (0)

// Whole-tile staging of Q4_K tiles: every wave's kWtInstr instructions, every lane.
int main() {
  const int rows[] = {1, 2, 15, 16, 17, 31, 33, 48};
  for (int nsb = 1; nsb <= 16; ++nsb) {
    // the kernel: one wave per super-block, kwi loads per wave and tile
    const int waves = nsb, U = wt_units(nsb), kwi = (wt_instrs(nsb) + waves - 1) / waves;
    const uint32_t row_bytes = 144u * nsb, slot = wt_slot_bytes(nsb);
    CHECK(16u * (uint32_t)U == row_bytes, "units per row");
    CHECK(kwi <= kWtInstr, "nsb %d: %d loads per wave", nsb, kwi);
    for (int N : rows) {
      const uint64_t total = (uint64_t)N * row_bytes;  // the matrix starts at 0
      for (int row0 = 0; row0 < N; row0 += 16) {
        const int nvalid = N - row0 < 16 ? N - row0 : 16;
        const uint64_t tile = (uint64_t)row0 * row_bytes;
        const uint64_t desc = (uint64_t)nvalid * row_bytes;  // the descriptor's size: rows past the matrix read 0
        std::vector<int64_t> held(slot, -1);
        for (int w = 0; w < waves; ++w)
          for (int k = 0; k < kwi; ++k) {
            const int i = wt_instr(w, waves, k, nsb);
            for (int lane = 0; lane < 64; ++lane) {
              const uint32_t off = wt_src(i, lane, nsb), lds = wt_lds(i, lane);
              CHECK(off % 16 == 0 && off + 16 <= 16u * row_bytes, "nsb %d: unit outside the 16 rows", nsb);
              CHECK(lds + 16 <= slot, "nsb %d: LDS write past the slot", nsb);
              CHECK(off >= desc || tile + off + 16 <= total, "nsb %d N %d: in-descriptor unit past the matrix", nsb, N);
              for (int b = 0; b < 16; ++b) {
                const int64_t v = off + b < desc ? (int64_t)(tile + off + b) : -2;  // -2: reads as zero
                // two loads of one LDS byte must agree (duplicate units and instructions)
                CHECK(held[lds + b] == -1 || held[lds + b] == v, "nsb %d: LDS byte %u loaded twice differently", nsb,
                      lds + b);
                held[lds + b] = v;
              }
            }
          }
        for (int r = 0; r < nvalid; ++r)
          for (uint32_t b = 0; b < row_bytes; ++b)
            CHECK(held[wt_lds_byte(r, b, nsb)] == (int64_t)(tile + (uint64_t)r * row_bytes + b),
                  "nsb %d N %d row0 %d row %d byte %u", nsb, N, row0, r, b);
      }
    }
    // reads of one unit column by the 16 rows (64 banks of 4 bytes): distinct banks when
    // 16 divides U (K = 4096: the rotation's wrap moves a row by a multiple of 64 dwords),
    // at most four rows per bank otherwise (small K, where the rotation wraps)
    for (int c = 0; c < U; ++c) {
      std::vector<int> bank_used(64, 0);
      for (int r = 0; r < 16; ++r) {
        const uint32_t dw = wt_lds_byte(r, 16u * c, nsb) / 4;
        for (int q = 0; q < 4; ++q) bank_used[(dw + q) % 64]++;
      }
      const int most = U % 16 == 0 ? 1 : 4;
      for (int q = 0; q < 64; ++q)
        CHECK(bank_used[q] <= most, "nsb %d column %d: bank %d used %d times", nsb, c, q, bank_used[q]);
    }
  }
  std::printf("%s (%d failures)\n", fails ? "FAIL" : "ok", fails);
  return fails ? 1 : 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_whole_tile_staging_in_bounds_and_conflict_free():
    """The whole-tile staging map (the tile loop's Q4_K gate/up pairs): every wave's
    loads stay inside the tile's 16 rows and the LDS slot, units past the matrix fall
    outside the buffer descriptor (they read zeros), every byte of every valid row lands
    where the compute reads it, and one unit column of the 16 rows sits on 64 distinct
    LDS banks at K = 4096 (four rows per bank at most otherwise)."""
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "check_wt.cpp")
        exe = os.path.join(d, "check_wt")
        with open(src, "w") as f:
            f.write(WHOLE_TILE_PROGRAM)
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.dirname(HDR), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        print(out.stdout)
        assert out.returncode == 0, out.stdout


KCHUNK_PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "gemm_addr.h"
using namespace gr::addr;

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { if (fails++ < 20) { std::printf(__VA_ARGS__); std::printf("\n"); } } } while (0)

// K-chunk staging of Q6_K tiles (rows of a multiple of 16 bytes): every wave's loads of
// every chunk, every lane, and the bytes the compute reads (dword pairs around each
// 2-byte aligned field of each block).
int main() {
  const int nsbs[] = {8, 16, 24, 48, 56};
  const int rows[] = {1, 15, 16, 17, 33};
  for (int nsb : nsbs)
    for (int C = 1; C <= 16; ++C) {
      if (nsb % C) continue;
      const int waves = C, nch = nsb / C, kwi = (kc_instrs(C) + waves - 1) / waves;
      const uint32_t row_bytes = 210u * nsb, slot = kc_slot_bytes(C);
      CHECK(row_bytes % 16 == 0, "rows of 16 bytes");
      CHECK(kwi <= 5, "C %d: %d loads per wave", C, kwi);
      CHECK(kc_stride(C) % 2 == 1 && kc_stride(C) >= kc_units(C), "stride");
      for (int N : rows)
        for (int row0 = 0; row0 < N; row0 += 16) {
          const int nvalid = N - row0 < 16 ? N - row0 : 16;
          const uint64_t total = (uint64_t)N * row_bytes, tile = (uint64_t)row0 * row_bytes;
          for (int c = 0; c < nch; ++c) {
            const uint64_t base = tile + kc_window(C, c);
            const uint64_t desc = (uint64_t)nvalid * row_bytes - kc_window(C, c);  // descriptor size from base
            std::vector<int64_t> held(slot, -1);
            for (int w = 0; w < waves; ++w)
              for (int k = 0; k < kwi; ++k) {
                const int i = kc_instr(w, waves, k, C);
                for (int lane = 0; lane < 64; ++lane) {
                  const uint32_t off = kc_src(i, lane, C, row_bytes), lds = kc_lds(i, lane);
                  CHECK(off % 16 == 0, "aligned unit");
                  CHECK(lds + 16 <= slot, "C %d: LDS write past the slot", C);
                  CHECK(off >= desc || base + off + 16 <= total, "nsb %d C %d N %d: in-descriptor unit past the matrix",
                        nsb, C, N);
                  for (int b = 0; b < 16; ++b) {
                    const int64_t v = off + b < desc ? (int64_t)(base + off + b) : -2;
                    CHECK(held[lds + b] == -1 || held[lds + b] == v, "C %d: LDS byte loaded twice differently", C);
                    held[lds + b] = v;
                  }
                }
              }
            const uint32_t s16 = kc_s16(C, c);
            for (int r = 0; r < nvalid; ++r)
              for (int j = 0; j < C; ++j) {
                const uint32_t x0 = s16 + 210u * j;  // the block's first byte in the window
                for (uint32_t b = 0; b < 210; ++b)
                  CHECK(held[kc_lds_byte(r, x0 + b, C)] == (int64_t)(tile + (uint64_t)r * row_bytes + 210u * (C * c + j) + b),
                        "nsb %d C %d N %d row0 %d chunk %d row %d block %d byte %u", nsb, C, N, row0, c, r, j, b);
                // the dword pairs the compute loads around each field stay inside the slot
                for (uint32_t f = 0; f < 212; f += 4)
                  CHECK(kc_lds_byte(r, ((x0 + f) & ~3u) + 8, C) <= slot, "C %d: read past the slot", C);
              }
          }
        }
      // one byte column of the 16 rows: 16 distinct banks
      for (uint32_t b = 0; b < 16u * kc_units(C); b += 4) {
        std::vector<int> used(64, 0);
        for (int r = 0; r < 16; ++r) used[(kc_lds_byte(r, b, C) / 4) % 64]++;
        for (int q = 0; q < 64; ++q) CHECK(used[q] <= 1, "C %d column %u: bank %d used %d times", C, b, q, used[q]);
      }
    }
  std::printf("%s (%d failures)\n", fails ? "FAIL" : "ok", fails);
  return fails ? 1 : 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_k_chunk_staging_in_bounds_and_conflict_free():
    """The K-chunk staging map (the Q6_K down GEMM): every wave's loads of every chunk stay
    inside the LDS slot and, inside the buffer descriptor, inside the matrix; every byte of
    every block of every valid row lands where the compute reads it, the dword pairs read
    around each field stay in the slot, and one byte column of 16 rows sits on 16 banks."""
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "check_kc.cpp")
        exe = os.path.join(d, "check_kc")
        with open(src, "w") as f:
            f.write(KCHUNK_PROGRAM)
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.dirname(HDR), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        print(out.stdout)
        assert out.returncode == 0, out.stdout


KRANGE_PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "gemm_addr.h"
using namespace gr::addr;

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { if (fails++ < 20) { std::printf(__VA_ARGS__); std::printf("\n"); } } } while (0)

// Whole-tile staging of K ranges (Q4_K): the matrix's rows are nsb super-blocks long, a
// range is W = nsb / nkr of them; every wave's loads of every range, every lane.
int main() {
  const int rows[] = {1, 15, 16, 17, 33, 48};
  const int shapes[][2] = {{4, 1}, {5, 1}, {8, 1}, {8, 2}, {12, 2}, {16, 2}, {16, 4}, {20, 4}, {24, 3}, {32, 4}, {56, 7}};
  for (const auto& sh : shapes) {
    const int nsb = sh[0], nkr = sh[1], W = nsb / nkr;
    const int U = wt_units(W), kwi = (wt_instrs(W) + W - 1) / W;
    const uint32_t row_bytes = 144u * nsb, slot = wt_slot_bytes(W), span = 16u * (uint32_t)U;
    CHECK(kwi <= kWtInstr, "W %d: %d loads per wave", W, kwi);
    for (int N : rows) {
      const uint64_t total = (uint64_t)N * row_bytes;  // the matrix starts at 0
      for (int row0 = 0; row0 < N; row0 += 16)
        for (int kr = 0; kr < nkr; ++kr) {
          const int nvalid = N - row0 < 16 ? N - row0 : 16;
          const uint64_t base = (uint64_t)row0 * row_bytes + 144u * (uint64_t)(kr * W);
          // the descriptor ends with the range of the last valid row: rows past the matrix read 0
          const uint64_t desc = (uint64_t)(nvalid - 1) * row_bytes + span;
          std::vector<int64_t> held(slot, -1);
          for (int w = 0; w < W; ++w)
            for (int k = 0; k < kwi; ++k) {
              const int i = wt_instr(w, W, k, W);
              for (int lane = 0; lane < 64; ++lane) {
                const uint32_t off = wt_src_rows(i, lane, W, row_bytes), lds = wt_lds(i, lane);
                CHECK(off % 16 == 0, "unaligned unit");
                CHECK(off % row_bytes + 16 <= span && off / row_bytes < 16, "nsb %d W %d: unit outside the range", nsb, W);
                CHECK(lds + 16 <= slot, "W %d: LDS write past the slot", W);
                CHECK(off >= desc || base + off + 16 <= total, "nsb %d N %d: in-descriptor unit past the matrix", nsb, N);
                CHECK(off >= desc || (int)(off / row_bytes) < nvalid, "in-descriptor unit of a row past the matrix");
                for (int b = 0; b < 16; ++b) {
                  const int64_t v = off + b < desc ? (int64_t)(base + off + b) : -2;  // -2: reads as zero
                  CHECK(held[lds + b] == -1 || held[lds + b] == v, "W %d: LDS byte %u loaded twice differently", W,
                        lds + b);
                  held[lds + b] = v;
                }
              }
            }
          for (int r = 0; r < nvalid; ++r)
            for (uint32_t b = 0; b < span; ++b)
              CHECK(held[wt_lds_byte(r, b, W)] == (int64_t)(base + (uint64_t)r * row_bytes + b),
                    "nsb %d W %d N %d row0 %d kr %d row %d byte %u", nsb, W, N, row0, kr, r, b);
        }
    }
  }
  std::printf("%s (%d failures)\n", fails ? "FAIL" : "ok", fails);
  return fails ? 1 : 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_k_range_staging_in_bounds():
    """Whole-tile staging of a K range (the many-row-block kernel: a tile's 16 rows over
    W super-blocks of a longer row): every wave's loads stay inside the range of the 16
    rows and inside the LDS slot, units of rows past the matrix fall outside the buffer
    descriptor (they read zeros), and every byte of every valid row's range lands where
    the compute reads it."""
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "check_kr.cpp")
        exe = os.path.join(d, "check_kr")
        with open(src, "w") as f:
            f.write(KRANGE_PROGRAM)
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.dirname(HDR), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        print(out.stdout)
        assert out.returncode == 0, out.stdout
