// gemm.hip -- fused-dequant skinny GEMM for GGUF Q4_K / Q6_K weights on gfx950.
//
// y[b][n] = sum_k W[n][k] x[b][k] for the B active decode rows sharing one pass over
// the weights (Leone, intro: active decode rows share matrix operations).  Every
// weight byte is read from HBM exactly once per call.
//
// Layout of the work (gfx950):
//  * One workgroup per output tile of 16 weight rows (SwiGLU: 16 gate rows + the 16
//    up rows of the same FFN columns) and all B rows; its waves split K into
//    contiguous super-block ranges and reduce their partial sums through LDS, so the
//    epilogue sees complete outputs (no atomics, no second pass).
//  * Quants are expanded in registers into exact bf16 integers (128 + q via an OR
//    with the exponent bits) and fed as the B operand of v_mfma_f32_16x16x32_bf16
//    (Q4_K: one 32-weight sub-block per MFMA) or v_mfma_f32_16x16x16_bf16 (Q6_K: one
//    16-weight sub-block).  The A operand is the activation tile in bf16 hi/lo rows
//    (actpack), so the products are exact and sums are fp32.
//  * A second MFMA of the same A against a ones vector gives, in the same output
//    layout, the activation sums S of the sub-block, so each MFMA result is scaled in
//    fp32 without any extra data:
//      Q4_K: acc += d*sc * D - (128*d*sc + dmin*m) * S
//      Q6_K: acc += d*sc * (D - 160 * S)
//  * The weights and activation fragments of super-block sb+1 are loaded before the
//    MFMAs of sb.
#include "gr_internal.h"
#include "quant.h"
#include "gemm_addr.h"

namespace gr {

constexpr u32 kOnesBf16 = 0x3F803F80u;  // two bf16 1.0

// ---------------------------------------------------------------------------------
// LDS staging of weights
//
// A wave streams the 16 rows of its tile one super-block at a time into a two-slot
// LDS ring with direct global->LDS loads (lane i of a load lands at slot + size*i),
// so every load instruction reads contiguous bytes; the MFMA operands are then read
// from LDS.  Activation fragments (already contiguous per instruction) go to
// registers.  An explicit vmcnt wait guards each slot before it is read.

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

constexpr int kQ4LoadInstr = addr::kQ4Instr;  // 16-byte loads per lane and stage
constexpr int kQ6LoadInstr = addr::kQ6Instr;  // 16-byte loads per lane and stage
// Every lane of every load instruction loads (lanes past the tile's data re-read a
// valid chunk into the padding), so each stage is exactly kQ*LoadInstr VMEM
// instructions on every path and the vmcnt waits below are exact.
constexpr int kQ4Stage = kQ4LoadInstr * 64 * 16;  // 3072 B (2304 used)
constexpr int kQ6Stage = kQ6LoadInstr * 64 * 16;  // 4096 B (3840 used)
constexpr int kQ5Stage = addr::kQ5Instr * 64 * 16;  // 3072 B (2816 used)
constexpr int kQ8Stage = addr::kQ8Instr * 64 * 16;  // 5120 B (4352 used)

constexpr int stage_bytes(int wtype) {
  return wtype == 12 ? kQ4Stage : wtype == 13 ? kQ5Stage : wtype == 8 ? kQ8Stage : kQ6Stage;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
GR_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// The same for a count known at run time (0..15), through a switch of constant waits.
GR_DEV void wait_vmcnt_n(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<15>(); break;
  }
}

// The 16 rows of a tile: `base` is its first row (wave-uniform, 16-byte aligned);
// row r reads matrix row min(r, nvalid - 1) of the tile, so a ragged last tile
// repeats its last row (results of such rows are never stored).
struct TileRows {
  const uint8_t* base;
  int nvalid;
  u32 row_bytes;
  GR_DEV u32 off(int r) const { return addr::row_off(r, nvalid, row_bytes); }
  GR_DEV const uint8_t* end() const { return base + (size_t)nvalid * row_bytes; }  // past its last row
};

// Staging loads (unit mapping, address arithmetic and LDS row strides: gemm_addr.h).  The loads are buffer
// loads into LDS: the wave-uniform part of the address (the tile's super-block) lives
// in the buffer descriptor, rebuilt per stage with scalar instructions, and each lane
// keeps its offsets within the tile, computed once.  The descriptor's size ends at the
// tile's last row, so a stray offset would read zeros rather than fault.
constexpr int kBufDword3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9)

GR_DEV __amdgpu_buffer_rsrc_t stage_rsrc(const uint8_t* base, const TileRows& tr, const uint8_t* tile_end) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)(u32)(tile_end - base), kBufDword3);
}

struct Q4Lane {
  u32 p[kQ4LoadInstr];  // byte offset of this lane's chunk from the tile's block address
};
GR_DEV Q4Lane q4_lane(const TileRows& tr, int lane) {
  Q4Lane l;
#pragma unroll
  for (int i = 0; i < kQ4LoadInstr; ++i) {
    const int c = addr::q4_unit(lane, i);
    l.p[i] = tr.off(addr::q4_row(c)) + addr::q4_in_block(c);
  }
  return l;
}
GR_DEV void q4_issue(const TileRows& tr, const Q4Lane& ln, int sb, lds_u8* slot) {
  const uint8_t* blk = tr.base + (size_t)sb * kQ4KBytes;  // wave-uniform
  const __amdgpu_buffer_rsrc_t rs = stage_rsrc(blk, tr, tr.end());
#pragma unroll
  for (int i = 0; i < kQ4LoadInstr; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(slot + 1024 * i), 16, ln.p[i], 0, 0, 0);
}

// Q5_K and Q8_0: the aligned-format staging (gemm_addr.h), NI loads of RU units per row.
template <int NI, int RU>
struct AlLane {
  u32 p[NI];  // byte offset of this lane's chunk from the tile's block address
};
template <int NI, int RU>
GR_DEV AlLane<NI, RU> al_lane(const TileRows& tr, int lane) {
  AlLane<NI, RU> l;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = addr::al_unit(lane, i, RU);
    l.p[i] = tr.off(addr::al_row(c, RU)) + addr::al_in_block(c, RU);
  }
  return l;
}
// One load instruction of the aligned-format staging: 16 bytes per lane into slot + 1024 i.
GR_DEV void al_issue1(const TileRows& tr, u32 p, int sb, int row_bytes, lds_u8* slot) {
  const uint8_t* blk = tr.base + (size_t)sb * row_bytes;  // wave-uniform
  const __amdgpu_buffer_rsrc_t rs = stage_rsrc(blk, tr, tr.end());
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)slot, 16, p, 0, 0, 0);
}

struct Q6Lane {
  u32 pre[kQ6LoadInstr];  // addr::q6_pre of this lane's unit per instruction
};
GR_DEV Q6Lane q6_lane(const TileRows& tr, int lane) {
  Q6Lane l;
#pragma unroll
  for (int i = 0; i < kQ6LoadInstr; ++i) {
    const int c = addr::q6_unit(lane, i);
    l.pre[i] = addr::q6_pre(tr.off(addr::q6_row(c)), c);
  }
  return l;
}
// ALIGNED: every row of the matrix is a multiple of 16 bytes, so all rows of a stage
// share the tile's s16, which folds into the descriptor's base; otherwise each lane
// finds its row's.
template <bool ALIGNED>
GR_DEV void q6_issue(const TileRows& tr, const Q6Lane& ln, int sb, lds_u8* slot) {
  const uint8_t* blk = tr.base + (size_t)sb * kQ6KBytes;  // wave-uniform
  if constexpr (ALIGNED) {
    const __amdgpu_buffer_rsrc_t rs = stage_rsrc(blk - addr::q6_s16((u32)(uintptr_t)blk), tr, tr.end());
#pragma unroll
    for (int i = 0; i < kQ6LoadInstr; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(slot + 1024 * i), 16, ln.pre[i], 0, 0, 0);
  } else {
    const __amdgpu_buffer_rsrc_t rs = stage_rsrc(blk - 16, tr, tr.end());
#pragma unroll
    for (int i = 0; i < kQ6LoadInstr; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lptr_t)(slot + 1024 * i), 16, addr::q6_rel(ln.pre[i], addr::q6_s16((u32)(uintptr_t)blk + ln.pre[i])), 0,
          0, 0);
  }
}

// 4 bytes at (lo dword, hi dword) shifted right by sh bytes.
GR_DEV u32 lds_pair(const lds_u8* lo, const lds_u8* hi, u32 sh) {
  return __builtin_amdgcn_alignbyte(*(const __attribute__((address_space(3))) u32*)hi,
                                    *(const __attribute__((address_space(3))) u32*)lo, sh);
}

// ---------------------------------------------------------------------------------
// The per-wave stream over super-blocks [s0, s1): weights run D - 1 stages ahead in a
// D-slot LDS ring, activation fragments one stage ahead in two register buffers (the
// loop is unrolled by two so the buffers are named statically).  Before stage i's
// math, the only memory instructions allowed outstanding are the ones issued after
// stage i's activations (the weights of stage i + D - 1 and the activations of stage
// i + 1, when issued), so every wait below is exact on each path.
constexpr int kRing = 2;  // D (slots of the LDS ring; D - 1 stages of weights in flight)

template <int KW, int KA, class Buf, class IssueW, class IssueA, class Step>
GR_DEV void pipeline_ring(int s0, int s1, Buf& b0, Buf& b1, IssueW&& issue_w, IssueA&& issue_a, Step&& step) {
  if (s1 - s0 >= kRing) {
#pragma unroll
    for (int d = 0; d < kRing - 1; ++d) issue_w(s0 + d);
  } else {
#pragma unroll
    for (int d = 0; d < kRing - 1; ++d)
      if (s0 + d < s1) issue_w(s0 + d);
  }
  issue_a(b0, s0);
  int i = s0;
  // steady state, no branches: both stages of a pair issue their successors' loads
  for (; i + kRing < s1; i += 2) {
    issue_w(i + kRing - 1);
    issue_a(b1, i + 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<KW + KA>();
    __builtin_amdgcn_sched_barrier(0);
    step(b0, i);
    __builtin_amdgcn_sched_barrier(0);
    issue_w(i + kRing);
    issue_a(b0, i + 2);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<KW + KA>();
    __builtin_amdgcn_sched_barrier(0);
    step(b1, i + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the last (at most kRing) stages
  auto one = [&](Buf& cur, Buf& nxt, int j) {
    const bool w_next = j + kRing - 1 < s1;
    const bool a_next = j + 1 < s1;
    if (w_next) issue_w(j + kRing - 1);
    if (a_next) issue_a(nxt, j + 1);
    __builtin_amdgcn_sched_barrier(0);
    if (w_next)
      wait_vmcnt<KW + KA>();
    else if (a_next)
      wait_vmcnt<KA>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    step(cur, j);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (; i < s1; i += 2) {
    one(b0, b1, i);
    if (i + 1 < s1) one(b1, b0, i + 1);
  }
}

// ---------------------------------------------------------------------------------
// wave bodies: accumulate rows 8bt+2g and 8bt+2g+1 of output column n (lane (n, g))
// of tile t over super-blocks [sb0, sb1).  acc[t][b][e] holds MFMA row 4g + e, i.e.
// batch row 8b + 2g + (e >> 1), bf16 hi (e even) or lo (e odd) part.

// One super-block of Q4_K for NT tiles, weights from LDS slots, activations `ca`.
template <int NT, int BTN>
GR_DEV void q4_step(const GemmArgs& a, lds_u8* const (&slot)[NT], const u32x4* ca, int sb, int lane,
                    float (&acc)[NT][BTN][4]) {
  const u32x4* xp = (const u32x4*)a.xpack;
  const u32x4 ones = {kOnesBf16, kOnesBf16, kOnesBf16, kOnesBf16};
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, kg = lane >> 4;
  const u32 M = vconst(0x43004300u);
  Q4Regs w[NT];
  float sd[NT][8], mm[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const lds_u8* rp = slot[t] + addr::q4_lds_byte(n, 0);  // row n's block
    w[t].hdr = *(const __attribute__((address_space(3))) u32x4*)rp;
#pragma unroll
    for (int c = 0; c < 4; ++c) w[t].qs[c] = *(const __attribute__((address_space(3))) u32x2*)(rp + 16 + 32 * c + 8 * kg);
    q4_scales(w[t].hdr, sd[t], mm[t]);
#pragma unroll
    for (int j = 0; j < 8; ++j) mm[t][j] = __builtin_fmaf(128.0f, sd[t][j], mm[t][j]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 av[BTN];
    f32x4 sv[BTN];
#pragma unroll
    for (int b = 0; b < BTN; ++b) {
      if constexpr (BTN == 1)
        av[b] = ca[j];
      else
        av[b] = xp[(((size_t)b * a.nslices) + (size_t)sb * 8 + j) * 64 + lane];
      sv[b] = mfma_bf16_k32(av[b], ones, z4);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 bq = q4_expand(w[t].qs[j >> 1], (j & 1) != 0, M);
#pragma unroll
      for (int b = 0; b < BTN; ++b) {
        const f32x4 dd = mfma_bf16_k32(av[b], bq, z4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[t][b][e] = __builtin_fmaf(sd[t][j], dd[e], __builtin_fmaf(-mm[t][j], sv[b][e], acc[t][b][e]));
      }
    }
  }
}

template <int NA>
struct ABuf {
  u32x4 a[NA];  // activation fragments of one super-block
};

template <int NT, int BTN>
GR_DEV void q4_wave(const GemmArgs& a, const TileRows (&tr)[NT], lds_u8* ring, int sb0, int sb1, int lane,
                    float (&acc)[NT][BTN][4]) {
  constexpr int NA = BTN == 1 ? 8 : 1;
  constexpr int KW = NT * kQ4LoadInstr, KA = BTN == 1 ? 8 : 0;  // VMEM instructions per issue
  Q4Lane ln[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) ln[t] = q4_lane(tr[t], lane);
  auto slot_of = [&](int sb, int t) { return ring + (((sb - sb0) & (kRing - 1)) * NT + t) * kQ4Stage; };
  ABuf<NA> b0, b1;
  auto issue_w = [&](int sb) {
#pragma unroll
    for (int t = 0; t < NT; ++t) q4_issue(tr[t], ln[t], sb, slot_of(sb, t));
  };
  auto issue_a = [&](ABuf<NA>& b, int sb) {
    if constexpr (BTN == 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) b.a[j] = ((const u32x4*)a.xpack)[((size_t)sb * 8 + j) * 64 + lane];
    }
  };
  auto step = [&](ABuf<NA>& b, int sb) {
    lds_u8* slots[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) slots[t] = slot_of(sb, t);
    q4_step<NT, BTN>(a, slots, b.a, sb, lane, acc);
  };
  pipeline_ring<KW, KA>(sb0, sb1, b0, b1, issue_w, issue_a, step);
}

// One super-block of Q5_K: Q4_K's header and nibbles with a fifth bit per weight (bit
// 2c + high of high-bit byte l); 128 + q (q < 32) is still an exact bf16, so the sums
// and scales are Q4_K's.
template <int NT, int BTN>
GR_DEV void q5_step(const GemmArgs& a, lds_u8* const (&slot)[NT], const u32x4* ca, int sb, int lane,
                    float (&acc)[NT][BTN][4]) {
  const u32x4* xp = (const u32x4*)a.xpack;
  const u32x4 ones = {kOnesBf16, kOnesBf16, kOnesBf16, kOnesBf16};
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, kg = lane >> 4;
  const u32 M = vconst(0x43004300u);
  u32x4 hdr[NT];
  u32x2 qs[NT][4], qh[NT];
  float sd[NT][8], mm[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const lds_u8* rp = slot[t] + addr::al_lds_byte(n, 0, addr::kQ5RowUnits);  // row n's block
    hdr[t] = *(const __attribute__((address_space(3))) u32x4*)rp;
    qh[t] = *(const __attribute__((address_space(3))) u32x2*)(rp + 16 + 8 * kg);
#pragma unroll
    for (int c = 0; c < 4; ++c) qs[t][c] = *(const __attribute__((address_space(3))) u32x2*)(rp + 48 + 32 * c + 8 * kg);
    q4_scales(hdr[t], sd[t], mm[t]);
#pragma unroll
    for (int j = 0; j < 8; ++j) mm[t][j] = __builtin_fmaf(128.0f, sd[t][j], mm[t][j]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 av[BTN];
    f32x4 sv[BTN];
#pragma unroll
    for (int b = 0; b < BTN; ++b) {
      if constexpr (BTN == 1)
        av[b] = ca[j];
      else
        av[b] = xp[(((size_t)b * a.nslices) + (size_t)sb * 8 + j) * 64 + lane];
      sv[b] = mfma_bf16_k32(av[b], ones, z4);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 bq = q5_expand(qs[t][j >> 1], qh[t], j, M);
#pragma unroll
      for (int b = 0; b < BTN; ++b) {
        const f32x4 dd = mfma_bf16_k32(av[b], bq, z4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[t][b][e] = __builtin_fmaf(sd[t][j], dd[e], __builtin_fmaf(-mm[t][j], sv[b][e], acc[t][b][e]));
      }
    }
  }
}

// Four bytes of row n's stage from byte offset `off` (any 2-byte-aligned offset) as one
// dword, and the next four.
GR_DEV u32x2 lds_8bytes(const lds_u8* row, u32 off) {
  const u32 al = off & ~3u, sh = off & 3u;
  const u32 d0 = *(const __attribute__((address_space(3))) u32*)(row + al);
  const u32 d1 = *(const __attribute__((address_space(3))) u32*)(row + al + 4);
  const u32 d2 = *(const __attribute__((address_space(3))) u32*)(row + al + 8);
  return u32x2{__builtin_amdgcn_alignbyte(d1, d0, sh), __builtin_amdgcn_alignbyte(d2, d1, sh)};
}

constexpr u32 kNeg2304Bf16 = 0xC510C510u;  // two bf16 -2304.0

// One super-block of Q8_0 (eight 34-byte blocks: fp16 d, 32 int8 codes).  A code q is
// u - 128 with u = q ^ 0x80 = 16 h + l; the MFMA chain C = A x (-2304), then B = 128 + l,
// then B = 2048 + 16 h (both exact bf16) returns sum a * (16 h + l - 128) = sum a * q.
template <int NT, int BTN>
GR_DEV void q8_step(const GemmArgs& a, lds_u8* const (&slot)[NT], const u32x4* ca, int sb, int lane,
                    float (&acc)[NT][BTN][4]) {
  const u32x4* xp = (const u32x4*)a.xpack;
  const u32x4 neg = {kNeg2304Bf16, kNeg2304Bf16, kNeg2304Bf16, kNeg2304Bf16};
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, kg = lane >> 4;
  const u32 NIB = 0x000F000Fu;
  const u32 ML = vconst(0x43004300u), MH = vconst(0x45004500u);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 av[BTN];
    f32x4 c0[BTN];
#pragma unroll
    for (int b = 0; b < BTN; ++b) {
      if constexpr (BTN == 1)
        av[b] = ca[j];
      else
        av[b] = xp[(((size_t)b * a.nslices) + (size_t)sb * 8 + j) * 64 + lane];
      c0[b] = mfma_bf16_k32(av[b], neg, z4);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const lds_u8* rp = slot[t] + addr::al_lds_byte(n, 0, addr::kQ8RowUnits);  // row n's 272 bytes
      const float d = h2f(*(const __attribute__((address_space(3))) u16*)(rp + 34 * j));
      const u32x2 q = lds_8bytes(rp, 34 * j + 2 + 8 * kg);
      const u32 u0 = q.x ^ 0x80808080u, u1 = q.y ^ 0x80808080u;
      const u32x4 bl = {(u0 & NIB) | ML, ((u0 >> 8) & NIB) | ML, (u1 & NIB) | ML, ((u1 >> 8) & NIB) | ML};
      const u32x4 bh = {((u0 >> 4) & NIB) | MH, ((u0 >> 12) & NIB) | MH, ((u1 >> 4) & NIB) | MH,
                        ((u1 >> 12) & NIB) | MH};
#pragma unroll
      for (int b = 0; b < BTN; ++b) {
        const f32x4 dd = mfma_bf16_k32(av[b], bh, mfma_bf16_k32(av[b], bl, c0[b]));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][b][e] = __builtin_fmaf(d, dd[e], acc[t][b][e]);
      }
    }
  }
}

// The per-wave stream of the aligned formats (WT 13: Q5_K, 8: Q8_0).
template <int WT, int NT, int BTN>
GR_DEV void al_wave(const GemmArgs& a, const TileRows (&tr)[NT], lds_u8* ring, int sb0, int sb1, int lane,
                    float (&acc)[NT][BTN][4]) {
  constexpr int NI = WT == 13 ? addr::kQ5Instr : addr::kQ8Instr;
  constexpr int RU = WT == 13 ? addr::kQ5RowUnits : addr::kQ8RowUnits;
  constexpr int kStg = stage_bytes(WT);
  constexpr int NA = BTN == 1 ? 8 : 1;
  constexpr int KW = NT * NI, KA = BTN == 1 ? 8 : 0;  // VMEM instructions per issue
  AlLane<NI, RU> ln[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) ln[t] = al_lane<NI, RU>(tr[t], lane);
  auto slot_of = [&](int sb, int t) { return ring + (((sb - sb0) & (kRing - 1)) * NT + t) * kStg; };
  ABuf<NA> b0, b1;
  auto issue_w = [&](int sb) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < NI; ++i) al_issue1(tr[t], ln[t].p[i], sb, 16 * RU, slot_of(sb, t) + 1024 * i);
    }
  };
  auto issue_a = [&](ABuf<NA>& b, int sb) {
    if constexpr (BTN == 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) b.a[j] = ((const u32x4*)a.xpack)[((size_t)sb * 8 + j) * 64 + lane];
    }
  };
  auto step = [&](ABuf<NA>& b, int sb) {
    lds_u8* slots[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) slots[t] = slot_of(sb, t);
    if constexpr (WT == 13)
      q5_step<NT, BTN>(a, slots, b.a, sb, lane, acc);
    else
      q8_step<NT, BTN>(a, slots, b.a, sb, lane, acc);
  };
  pipeline_ring<KW, KA>(sb0, sb1, b0, b1, issue_w, issue_a, step);
}

constexpr u32 kNeg160Bf16 = 0xC320C320u;  // two bf16 -160.0

// Row n's Q6_K super-block from a staged window (lane group kg's quant dwords, the
// scales and d).  The window holds block byte b at q6_lds_byte(n, b, s16): the field at
// block byte C (a multiple of 4) is the dword pair at q6_lds_byte(n, C, s16 & 12)
// shifted right by s16 & 3 bytes.
GR_DEV void q6_load_at(const lds_u8* rs, u32 sh, int kg, Q6Regs& w);
GR_DEV void q6_load_lds(const lds_u8* slot, u32 s16, int n, int kg, Q6Regs& w) {
  // shift in bytes (alignbyte's shift operand counts bytes)
  q6_load_at(slot + addr::q6_lds_byte(n, 0, s16 & 12u), s16 & 3u, kg, w);
}
// A row's block whose byte 0 sits sh bytes past the 4-byte aligned LDS address rs.
GR_DEV void q6_load_at(const lds_u8* rs, u32 sh, int kg, Q6Regs& w) {
  const lds_u8* rp = rs + 4 * kg;
#pragma unroll
  for (int hu = 0; hu < 4; ++hu) {
    const int h = hu >> 1, u = hu & 1;
    const int ca = 64 * h + 16 * u, cb = ca + 32, cq = 128 + 32 * h + 16 * u;
    w.part[hu].a = lds_pair(rp + ca, rp + ca + 4, sh);
    w.part[hu].b = lds_pair(rp + cb, rp + cb + 4, sh);
    w.part[hu].q = lds_pair(rp + cq, rp + cq + 4, sh);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) w.sc[i] = lds_pair(rs + 192 + 4 * i, rs + 196 + 4 * i, sh);
  w.d = (u16)(lds_pair(rs + 208, rs + 212, sh) & 0xFFFFu);
}

// One super-block of Q6_K.  Per 16-weight sub-block: C = A x (-160) gives -160 * S
// (S the activation sums), and the quant MFMA accumulates onto it, so the MFMA returns
// D - 160 S = sum a * (q - 32) with no vector work; the scale is one FMA per row.
// REG: the activation fragments come from registers, ca[b * 8 + pair] (the tile-loop
// kernel; the split-K kernel's single batch tile); otherwise from the pack in memory.
template <int NT, int BTN, bool REG = (BTN == 1)>
GR_DEV void q6_step(const GemmArgs& a, lds_u8* const (&slot)[NT], const u32 (&s16reg)[NT], const u32x4* ca, int sb,
                    int lane, float (&acc)[NT][BTN][4]) {
  const u32x4* xp = (const u32x4*)a.xpack;
  const u32x2 neg160 = {kNeg160Bf16, kNeg160Bf16};
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, kg = lane >> 4;
  const u32 E = vconst(0x43434343u);
  Q6Regs w[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) q6_load_lds(slot[t], s16reg[t], n, kg, w[t]);
  float dsc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) dsc[t] = h2f(w[t].d);
#pragma unroll
  for (int hu = 0; hu < 4; ++hu) {
    const int h = hu >> 1, u = hu & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sub = 8 * h + 2 * r + u;  // 16-weight sub-block within the super-block
      u32x2 av[BTN];
      f32x4 cs[BTN];
#pragma unroll
      for (int b = 0; b < BTN; ++b) {
        u32x4 pr;
        if constexpr (REG)
          pr = ca[b * 8 + (sub >> 1)];
        else
          pr = xp[(((size_t)b * (a.nslices >> 1)) + (size_t)sb * 8 + (sub >> 1)) * 64 + lane];
        av[b] = (sub & 1) ? u32x2{pr.z, pr.w} : u32x2{pr.x, pr.y};
        cs[b] = mfma_bf16_k16(av[b], neg160, z4);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x2 bq = q6_expand(w[t].part[hu], r, E);
        const float sd = dsc[t] * (float)(int)(int8_t)((w[t].sc[sub >> 2] >> (8 * (sub & 3))) & 0xFF);
#pragma unroll
        for (int b = 0; b < BTN; ++b) {
          const f32x4 dd = mfma_bf16_k16(av[b], bq, cs[b]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][b][e] = __builtin_fmaf(sd, dd[e], acc[t][b][e]);
        }
      }
    }
    // keep the scheduler from hoisting all sixteen sub-blocks' MFMAs at once
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One Q6_K super-block of one tile at one activation tile, its block already in
// registers (q6_step's arithmetic; ca: the activation fragments of the super-block).
GR_DEV void q6_step_w(const Q6Regs& w, const u32x4* ca, float (&acc)[4]) {
  const u32x2 neg160 = {kNeg160Bf16, kNeg160Bf16};
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const u32 E = vconst(0x43434343u);
  const float dsc = h2f(w.d);
#pragma unroll
  for (int hu = 0; hu < 4; ++hu) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sub = 8 * (hu >> 1) + 2 * r + (hu & 1);
      const u32x4 pr = ca[sub >> 1];
      const u32x2 av = (sub & 1) ? u32x2{pr.z, pr.w} : u32x2{pr.x, pr.y};
      const f32x4 cs = mfma_bf16_k16(av, neg160, z4);
      const u32x2 bq = q6_expand(w.part[hu], r, E);
      const float sd = dsc * (float)(int)(int8_t)((w.sc[sub >> 2] >> (8 * (sub & 3))) & 0xFF);
      const f32x4 dd = mfma_bf16_k16(av, bq, cs);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(sd, dd[e], acc[e]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NT, int BTN, bool ALIGNED>
GR_DEV void q6_wave(const GemmArgs& a, const TileRows (&tr)[NT], lds_u8* ring, int sb0, int sb1, int lane,
                    float (&acc)[NT][BTN][4]) {
  constexpr int NA = BTN == 1 ? 8 : 1;
  constexpr int KW = NT * kQ6LoadInstr, KA = BTN == 1 ? 8 : 0;
  const int n = lane & 15;
  Q6Lane ln[NT];
  u32 on[NT];  // byte offset of row n (block 0) from the tile base
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    ln[t] = q6_lane(tr[t], lane);
    on[t] = tr[t].off(n);
  }
  auto slot_of = [&](int sb, int t) { return ring + (((sb - sb0) & (kRing - 1)) * NT + t) * kQ6Stage; };
  ABuf<NA> b0, b1;
  auto issue_w = [&](int sb) {
#pragma unroll
    for (int t = 0; t < NT; ++t) q6_issue<ALIGNED>(tr[t], ln[t], sb, slot_of(sb, t));
  };
  auto issue_a = [&](ABuf<NA>& b, int sb) {
    if constexpr (BTN == 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) b.a[j] = ((const u32x4*)a.xpack)[((size_t)sb * 8 + j) * 64 + lane];
    }
  };
  auto step = [&](ABuf<NA>& b, int sb) {
    lds_u8* slots[NT];
    u32 s16[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      slots[t] = slot_of(sb, t);
      s16[t] = addr::q6_s16((u32)(uintptr_t)(tr[t].base + (size_t)sb * kQ6KBytes) + on[t]);
    }
    q6_step<NT, BTN>(a, slots, s16, b.a, sb, lane, acc);
  };
  pipeline_ring<KW, KA>(sb0, sb1, b0, b1, issue_w, issue_a, step);
}

// ---------------------------------------------------------------------------------
// the kernel: waves split K, LDS reduction, epilogue

// ALIGNED (Q6_K only): every weight row is a multiple of 16 bytes (a multiple of 8
// super-blocks per row).
template <int WT, int NT, int BTN, int MAXT, bool ALIGNED>
__global__ __launch_bounds__(MAXT) void gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // staging rings, then the reduction
  float* red = (float*)lds;  // [waves][NT][BTN][64 lanes][2]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  const int tile = blockIdx.x;
  const int n = lane & 15;

  if (a.zero_ptr && tile == 0)
    for (int i = threadIdx.x; i < a.zero_n; i += blockDim.x) a.zero_ptr[i] = 0.0;

  // rows of the tile(s).  SwiGLU: tile t of the pair is the same 16 columns of gate
  // (t = 0) and up (t = 1).  Otherwise the workgroup's group of NT consecutive tiles of
  // one matrix; a tile past the matrix's rows (odd tile count) re-reads the previous
  // tile's rows and stores nothing.
  int seg = 0, local = tile;
  if (a.epi != kEpiSwiGLU) {
    while (seg + 1 < a.nseg && tile >= a.seg_tile_off[seg + 1]) ++seg;
    local = tile - a.seg_tile_off[seg];
  }
  TileRows tr[NT];
  int rows_n = a.seg_rows[seg];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int s = a.epi == kEpiSwiGLU ? t : seg;
    int lt = a.epi == kEpiSwiGLU ? local : local * NT + t;  // tile index within matrix s
    if (lt * 16 >= a.seg_rows[s]) lt = (a.seg_rows[s] - 1) / 16;
    tr[t] = TileRows{a.w[s] + (size_t)lt * 16 * a.row_bytes, a.seg_rows[s] - lt * 16, (u32)a.row_bytes};
  }
  // The input rows' RMSNorm partial sums (ss_slots * B <= kSsCap values) are parked in
  // LDS beside the reduction for the epilogue: one value per thread is loaded before the
  // main loop (one register through it), any rest (workgroups of fewer threads than
  // values) after it.
  const int n_ss = a.ss ? a.ss_slots * a.B : 0;
  const double ssp = (int)threadIdx.x < n_ss ? a.ss[threadIdx.x] : 0.0;
  // Epilogue element e = (t, bt, lane', k2) (a SwiGLU pair handles both tiles at once).
  // Its other operands that do not depend on the GEMM (the residual and the next norm
  // gain) are loaded before the main loop, for the first kPre elements of each thread,
  // so the epilogue waits on no memory.
  constexpr int kPer = NT * BTN * 128;
  const int n_elem = a.epi == kEpiSwiGLU ? BTN * 128 : kPer;
  struct Elem {
    bool in, live;
    int t, rem, bt, nn, brow, col;
  };
  auto elem = [&](int e) {
    Elem m;
    m.in = e < n_elem;
    m.t = a.epi == kEpiSwiGLU ? 0 : (m.in ? e / (BTN * 128) : 0);
    m.rem = e % (BTN * 128);
    m.bt = m.rem / 128;
    const int lp = (m.rem % 128) >> 1, k2 = m.rem & 1;
    m.nn = lp & 15;
    m.brow = 8 * m.bt + 2 * (lp >> 4) + k2;
    const int lt = a.epi == kEpiSwiGLU ? local : local * NT + m.t;  // output tile within the matrix
    m.live = m.in && m.brow < a.B && lt * 16 + m.nn < rows_n;
    m.col = (a.epi == kEpiSwiGLU ? 0 : a.seg_col_off[seg]) + lt * 16 + m.nn;
    return m;
  };
  constexpr int kPre = BTN > 2 ? 0 : ((kPer + 63) / 64 < 4 ? (kPer + 63) / 64 : 4);
  float pre_x[kPre > 0 ? kPre : 1], pre_g[kPre > 0 ? kPre : 1];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const Elem m = elem(threadIdx.x + k * blockDim.x);
    pre_x[k] = (m.live && a.epi == kEpiResidual) ? a.y[(size_t)m.brow * a.ldy + m.col] : 0.f;
    pre_g[k] = (m.live && a.epi == kEpiResidual && a.gain) ? a.gain[m.col] : 1.f;
  }

  float acc[NT][BTN][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < BTN; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][b][e] = 0.f;

  const int sb0 = wave * a.sb_per_wave;
  const int sb1 = min(a.nsb, sb0 + a.sb_per_wave);
  constexpr int kStage = stage_bytes(WT);
  lds_u8* ring = (lds_u8*)lds + wave * (kRing * NT * kStage);
  if (sb0 < sb1) {
    if constexpr (WT == 12)
      q4_wave<NT, BTN>(a, tr, ring, sb0, sb1, lane, acc);
    else if constexpr (WT == 13 || WT == 8)
      al_wave<WT, NT, BTN>(a, tr, ring, sb0, sb1, lane, acc);
    else
      q6_wave<NT, BTN, ALIGNED>(a, tr, ring, sb0, sb1, lane, acc);
  }
  __syncthreads();  // the reduction buffer reuses the staging area

  // reduce over waves: red[((w*NT + t)*BTN + b)*128 + lane*2 + e]
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < BTN; ++b) {
      float* r = red + (((size_t)wave * NT + t) * BTN + b) * 128 + lane * 2;
      r[0] = acc[t][b][0] + acc[t][b][1];  // hi + lo parts of batch row 8b + 2g
      r[1] = acc[t][b][2] + acc[t][b][3];  // and of row 8b + 2g + 1
    }
  double* s_ss = (double*)(red + (size_t)nwaves * NT * BTN * 128);  // [ss_slots][B]
  if ((int)threadIdx.x < n_ss) s_ss[threadIdx.x] = ssp;
  for (int i = threadIdx.x + blockDim.x; i < n_ss; i += blockDim.x) s_ss[i] = a.ss[i];
  __syncthreads();

  // epilogue
  const float inv_k = a.inv_k, eps = a.eps;
  int k = 0;
  for (int e = threadIdx.x; e < ((n_elem + 63) & ~63); e += blockDim.x, ++k) {
    // every lane of the wave reaches the shuffles below
    const Elem m = elem(e);
    float v = 0.f, v2 = 0.f;
    if (m.in) {
      // the waves' sums in wave order, each tile's reads issued at once (a loop over the
      // run-time wave count waited for each read before the next)
      constexpr int MW = MAXT / 64;
      const size_t ws = (size_t)NT * BTN * 128;  // from one wave's sums to the next
      float x[MW];
      const float* r0 = red + ((size_t)m.t * BTN + m.bt) * 128 + (m.rem % 128);
#pragma unroll
      for (int w = 0; w < MW; ++w) x[w] = r0[(size_t)min(w, nwaves - 1) * ws];
#pragma unroll
      for (int w = 0; w < MW; ++w) v += w < nwaves ? x[w] : 0.f;
      if (a.epi == kEpiSwiGLU) {
        const float* r1 = red + ((size_t)1 * BTN + m.bt) * 128 + (m.rem % 128);
#pragma unroll
        for (int w = 0; w < MW; ++w) x[w] = r1[(size_t)min(w, nwaves - 1) * ws];
#pragma unroll
        for (int w = 0; w < MW; ++w) v2 += w < nwaves ? x[w] : 0.f;
      }
    }
    double ssv = 0.0;
    float xv = 0.f, gv_ = 1.f;
    if (m.live && a.ss)
      for (int s = 0; s < a.ss_slots; ++s) ssv += s_ss[s * a.B + m.brow];
    if (k < kPre) {
#pragma unroll
      for (int q = 0; q < kPre; ++q)
        if (q == k) {
          xv = pre_x[q];
          gv_ = pre_g[q];
        }
    } else if (m.live) {
      if (a.epi == kEpiResidual) {
        xv = a.y[(size_t)m.brow * a.ldy + m.col];
        gv_ = a.gain ? a.gain[m.col] : 1.f;
      }
    }
    const float rs = m.live ? (a.ss ? 1.0f / sqrtf((float)ssv * inv_k + eps) : 1.0f) : 0.f;
    if (a.epi == kEpiStore) {
      if (m.live) a.y[(size_t)m.brow * a.ldy + m.col] = rs * v;
    } else if (a.epi == kEpiSwiGLU) {
      if (m.live) {
        const float gv = rs * v, uv = rs * v2;
        actpack_put(a.pack_out, a.pack_kind, a.pack_nslices, m.brow, m.col, gv / (1.0f + expf(-gv)) * uv);
      }
    } else {
      float xn = 0.f;
      if (m.live) {
        xn = xv + rs * v;
        a.y[(size_t)m.brow * a.ldy + m.col] = xn;
        const float pv = xn * gv_;
        if (a.pack_out) actpack_put(a.pack_out, a.pack_kind, a.pack_nslices, m.brow, m.col, pv);
        if (a.pack_out2) actpack_put(a.pack_out2, a.pack_kind2, a.pack_nslices2, m.brow, m.col, pv);
      }
      // sum of squares over the tile's 16 columns of each batch row: lanes with the
      // same (g, k2) differ in nn, which is bits 1..4 of the thread index
      float sq = xn * xn;
#pragma unroll
      for (int o = 2; o <= 16; o <<= 1) sq += __shfl_xor(sq, o, 64);
      if (m.in && m.nn == 0 && m.brow < a.B && a.ss_out)
        atomicAdd(a.ss_out + (size_t)(tile % a.ss_slots) * a.B + m.brow, (double)sq);
    }
  }
}

// ---------------------------------------------------------------------------------
// Tile-loop kernel for matrices with many tiles (one activation tile, K <= 2 super-
// blocks per wave).  Each wave owns a fixed K slice of at most two super-blocks and
// keeps that slice's activation fragments in registers for the whole launch; the
// workgroup walks a contiguous run of tile groups, its waves streaming the weights of
// their slice of each group through a kTlRing-slot LDS ring (prefetch crossing group
// boundaries), and after each group the waves' partial sums meet in one of two LDS
// reduction buffers for the group's epilogue.  Activations are read once per
// workgroup instead of once per group, which leaves the texture path to the weights.
//
// Waits: every weight stage is NT * kQ*LoadInstr LDS-DMA loads; the activation loads
// are issued before any of them.  Loads complete in order, so before stage q only the
// stages issued after it may be outstanding.  Epilogue stores that are younger than a
// waited-for load only make a wait longer (a pending older load keeps every younger
// load pending), never shorter.

constexpr u32 kNeg128Bf16 = 0xC300C300u;  // two bf16 -128.0

// bf16 of a small non-negative integer value v (exact), in both halves of a dword.
GR_DEV u32 bf16_dup(float v) {
  const u32 b = f2u(v);
  return (b >> 16) | (b & 0xFFFF0000u);
}

// Row n's Q4_K super-block from its staged bytes (rp): the quants of lane group kg, the
// scales sd[j] = d sc_j, dmin, and the mins m_2kg, m_2kg+1 as the B operand of a K = 16
// MFMA (each repeated for a bf16 hi / lo pair of the A operand).
GR_DEV void q4_decode_tl(const Q4Regs& w, int kg, float (&sd)[8], float& dmin, u32x2& bm);
GR_DEV void q4_load_tl(const lds_u8* rp, int kg, Q4Regs& w, float (&sd)[8], float& dmin, u32x2& bm) {
  w.hdr = *(const __attribute__((address_space(3))) u32x4*)rp;
#pragma unroll
  for (int c = 0; c < 4; ++c) w.qs[c] = *(const __attribute__((address_space(3))) u32x2*)(rp + 16 + 32 * c + 8 * kg);
  q4_decode_tl(w, kg, sd, dmin, bm);
}
// The same from a whole-tile slot: unit j of the row's block sits at unit (c0 + j) mod U
// of the row (rowp), c0 = the block's first unit plus the row's rotation.
GR_DEV void q4_load_tlw(const lds_u8* rowp, int c0, int U, int kg, Q4Regs& w, float (&sd)[8], float& dmin,
                        u32x2& bm) {
  auto unit = [&](int j) {
    const int u = c0 + j;
    return rowp + 16 * (u >= U ? u - U : u);
  };
  w.hdr = *(const __attribute__((address_space(3))) u32x4*)unit(0);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    w.qs[c] = *(const __attribute__((address_space(3))) u32x2*)(unit(1 + 2 * c + (kg >> 1)) + 8 * (kg & 1));
  q4_decode_tl(w, kg, sd, dmin, bm);
}
GR_DEV void q4_decode_tl(const Q4Regs& w, int kg, float (&sd)[8], float& dmin, u32x2& bm) {
  const u32 h0 = w.hdr.x, s0 = w.hdr.y, s1 = w.hdr.z, s2 = w.hdr.w;
  const float d = h2f((u16)(h0 & 0xFFFF));
  dmin = h2f((u16)(h0 >> 16));
  const u32 sc_lo = s0 & 0x3F3F3F3Fu, sc_hi = (s2 & 0x0F0F0F0Fu) | ((s0 >> 2) & 0x30303030u);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sd[j] = d * (float)((sc_lo >> (8 * j)) & 0xFF);
    sd[j + 4] = d * (float)((sc_hi >> (8 * j)) & 0xFF);
  }
  // mins m_2kg and m_2kg+1: bytes 2(kg & 1) and 2(kg & 1) + 1 of the low (j < 4) or
  // high (j >= 4) mins word
  const u32 m_lo = s1 & 0x3F3F3F3Fu, m_hi = ((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u);
  const u32 mw = (kg < 2 ? m_lo : m_hi) >> (16 * (kg & 1));
  bm = u32x2{bf16_dup((float)(mw & 0xFF)), bf16_dup((float)((mw >> 8) & 0xFF))};
}

// One Q4_K super-block in the tile-loop kernel.  The wave's activation slice is fixed,
// so the sums S_j of its 32-weight sub-blocks come precomputed (aS: the K = 16 MFMA
// A operand holding S_2g and S_2g+1 of row l % 16 as bf16 hi/lo pairs).  Each
// sub-block's quant MFMA starts from C_j = A_j x (-128) = -128 S_j, so it returns
// sum a q with no vector work (as the Q6_K path), and the mins term is one MFMA per
// tile (B: the mins m_j as exact bf16, repeated for the hi and lo parts of S_j):
//   acc += sum_j d sc_j (D_j - 128 S_j) - dmin sum_j m_j S_j
template <int NT, int BTN>
GR_DEV void q4_step_tl(lds_u8* const (&slot)[NT], const u32x4 (&ca)[BTN][8], const u32x2 (&aS)[BTN], int lane,
                       float (&acc)[NT][BTN][4]) {
  const u32x4 neg128 = {kNeg128Bf16, kNeg128Bf16, kNeg128Bf16, kNeg128Bf16};
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, kg = lane >> 4;
  const u32 M = vconst(0x43004300u);
  Q4Regs w[NT];
  float sd[NT][8], dmin[NT];
  u32x2 bm[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) q4_load_tl(slot[t] + addr::q4_lds_byte(n, 0), kg, w[t], sd[t], dmin[t], bm[t]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f32x4 cj[BTN];
#pragma unroll
    for (int b = 0; b < BTN; ++b) cj[b] = mfma_bf16_k32(ca[b][j], neg128, z4);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 bq = q4_expand(w[t].qs[j >> 1], (j & 1) != 0, M);
#pragma unroll
      for (int b = 0; b < BTN; ++b) {
        const f32x4 dd = mfma_bf16_k32(ca[b][j], bq, cj[b]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][b][e] = __builtin_fmaf(sd[t][j], dd[e], acc[t][b][e]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < BTN; ++b) {
      const f32x4 corr = mfma_bf16_k16(aS[b], bm[t], z4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][b][e] = __builtin_fmaf(-dmin[t], corr[e], acc[t][b][e]);
    }
}

// One Q4_K super-block of one tile from a whole-tile slot (q4_step_tl's arithmetic).
template <int BTN>
GR_DEV void q4_step_tlw(const lds_u8* rowp, int c0, int U, const u32x4 (&ca)[BTN][8], const u32x2 (&aS)[BTN],
                        int lane, float (&acc)[BTN][4]) {
  const u32x4 neg128 = {kNeg128Bf16, kNeg128Bf16, kNeg128Bf16, kNeg128Bf16};
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int kg = lane >> 4;
  const u32 M = vconst(0x43004300u);
  Q4Regs w;
  float sd[8], dmin;
  u32x2 bm;
  q4_load_tlw(rowp, c0, U, kg, w, sd, dmin, bm);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 bq = q4_expand(w.qs[j >> 1], (j & 1) != 0, M);
#pragma unroll
    for (int b = 0; b < BTN; ++b) {
      const f32x4 dd = mfma_bf16_k32(ca[b][j], bq, mfma_bf16_k32(ca[b][j], neg128, z4));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[b][e] = __builtin_fmaf(sd[j], dd[e], acc[b][e]);
    }
  }
#pragma unroll
  for (int b = 0; b < BTN; ++b) {
    const f32x4 corr = mfma_bf16_k16(aS[b], bm, z4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[b][e] = __builtin_fmaf(-dmin, corr[e], acc[b][e]);
  }
}

// Workgroup barrier for LDS written with ds_write only: the weight loads in flight
// (LDS-DMA into ring slots that no other wave reads) must not be drained at every
// group, which a fence would do (LDS-DMA completion is counted by vmcnt).  The wave's
// own LDS writes complete (lgkmcnt) before the barrier; the memory clobber keeps the
// compiler from moving memory accesses across it.
GR_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int WT, int NT, bool ALIGNED, int D, int BTN>
__global__ __launch_bounds__(512) void gemm_tl_kernel(GemmArgs a) {
  static_assert(D >= 2 && D <= 4, "ring depth");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int kStage = WT == 12 ? kQ4Stage : kQ6Stage;
  constexpr int KW = NT * (WT == 12 ? kQ4LoadInstr : kQ6LoadInstr);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  const int n = lane & 15;
  lds_u8* ring = (lds_u8*)lds + wave * (D * NT * kStage);
  float* red = (float*)(lds + (size_t)nwaves * D * NT * kStage);  // [2][waves][NT][BTN][128]

  if (a.zero_ptr && blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.zero_n; i += blockDim.x) a.zero_ptr[i] = 0.0;

  // this workgroup's tile groups and this wave's K slice
  const int g0 = blockIdx.x * a.tl_groups_per_wg;
  const int ng = min(a.tl_groups, g0 + a.tl_groups_per_wg) - g0;
  const int sb0 = wave * a.sb_per_wave;
  const int nst = max(0, min(a.nsb, sb0 + a.sb_per_wave) - sb0);  // 1 or 2 (0: idle wave)
  const int nq = ng * nst;

  // epilogue element of this thread (fixed): e < n_elem, e = (t, batch tile, 128 outputs)
  const int n_elem = (a.epi == kEpiSwiGLU ? 128 : NT * 128) * BTN;
  const int e = threadIdx.x;
  const int e_t = a.epi == kEpiSwiGLU ? 0 : (e < n_elem ? e / (128 * BTN) : 0);
  const int e_b = (e >> 7) % BTN;
  const int e_rem = e & 127;
  const int e_lp = e_rem >> 1;
  const int e_nn = e_lp & 15;
  const int e_brow = 8 * e_b + 2 * (e_lp >> 4) + (e_rem & 1);
  // rows of group gi: as in gemm_kernel (SwiGLU pairs, or NT consecutive tiles of one
  // matrix with a phantom tile re-reading the last one).  The segment table (at most
  // three matrices) is read into scalar registers once, so that finding a group's rows
  // costs no memory access inside the loops.
  const int nseg = a.nseg;
  const int off1 = a.seg_tile_off[1], off2 = a.seg_tile_off[2];
  const int rows0 = a.seg_rows[0], rows1 = a.seg_rows[1], rows2 = a.seg_rows[2];
  const uint8_t* const w0 = a.w[0];
  const uint8_t* const w1 = a.w[1];
  const uint8_t* const w2 = a.w[2];
  const int col1 = a.seg_col_off[1], col2 = a.seg_col_off[2];
  auto seg_of = [&](int gi) { return (nseg > 1 && gi >= off1 ? 1 : 0) + (nseg > 2 && gi >= off2 ? 1 : 0); };
  auto rows_of = [&](int sg) { return sg == 0 ? rows0 : sg == 1 ? rows1 : rows2; };
  auto w_of = [&](int sg) { return sg == 0 ? w0 : sg == 1 ? w1 : w2; };
  auto col_of = [&](int sg) { return sg == 0 ? 0 : sg == 1 ? col1 : col2; };
  auto group_rows = [&](int gi, TileRows (&tr)[NT], int& seg, int& local) {
    seg = a.epi == kEpiSwiGLU ? 0 : seg_of(gi);
    local = gi - (seg == 0 ? 0 : seg == 1 ? off1 : off2);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int sg = a.epi == kEpiSwiGLU ? t : seg;
      const int rows = rows_of(sg);
      int lt = a.epi == kEpiSwiGLU ? local : local * NT + t;
      if (lt * 16 >= rows) lt = (rows - 1) / 16;
      tr[t] = TileRows{w_of(sg) + (size_t)lt * 16 * a.row_bytes, rows - lt * 16, (u32)a.row_bytes};
    }
  };
  // per-lane load offsets of a full tile (a ragged tile recomputes its own)
  const TileRows full{w0, 16, (u32)a.row_bytes};
  auto slot_of = [&](int q, int t) { return ring + ((q % D) * NT + t) * kStage; };
  auto issue = [&](int q) {
    const int gl = nst == 2 ? q >> 1 : q;
    const int s = q - gl * nst;
    TileRows tr[NT];
    int seg, local;
    group_rows(g0 + gl, tr, seg, local);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (WT == 12) {
        const Q4Lane ln = q4_lane(tr[t].nvalid == 16 ? full : tr[t], lane);
        q4_issue(tr[t], ln, sb0 + s, slot_of(q, t));
      } else {
        const Q6Lane ln = q6_lane(tr[t].nvalid == 16 ? full : tr[t], lane);
        q6_issue<ALIGNED>(tr[t], ln, sb0 + s, slot_of(q, t));
      }
    }
  };

  float acc[NT][BTN][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < BTN; ++b)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[t][b][k] = 0.f;

  // Issue order: the RMSNorm partial sums, the slice's activation fragments (8 per
  // super-block, loaded once; a one-super-block slice loads its block twice), then the
  // first D - 1 weight stages (unconditionally: a workgroup with fewer stages repeats
  // its last one into slots it never reads).  So the first step waits for stage 0 and
  // what is older than it, not for the whole prologue.
  double sv[16];  // B <= 16: ss_slots(B) = 16; every lane loads (a valid row), uniformly
  if (a.ss) {
    const int row = min(e_brow, a.B - 1);
#pragma unroll
    for (int s = 0; s < 16; ++s) sv[s] = a.ss[s * a.B + row];
  }
  // activation tile b starts K / 32 fragments of 1 KB after tile b - 1 (both pack kinds)
  const size_t tile_frags = (size_t)a.nsb * 8;
  u32x4 act[2][BTN][8];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int sb = min(sb0 + s, a.nsb - 1);
#pragma unroll
    for (int b = 0; b < BTN; ++b)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        act[s][b][j] = ((const u32x4*)a.xpack)[((size_t)b * tile_frags + (size_t)sb * 8 + j) * 64 + lane];
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d) issue(d < nq ? d : nq - 1);
  // everything but the prologue's stages has landed (so the loop starts with no
  // register load pending, and the compiler adds no wait of its own before it)
  wait_vmcnt<(D - 1) * KW>();
  // Q4_K: the slice's sub-block sums S_j as the mins MFMA's A operand (row l % 16,
  // j = 2kg and 2kg + 1, bf16 hi/lo), transposed through this wave's part of the
  // reduction buffers before any group uses them
  u32x2 aS[2][BTN];
  if constexpr (WT == 12) {
    const u32x4 ones = {kOnesBf16, kOnesBf16, kOnesBf16, kOnesBf16};
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int b = 0; b < BTN; ++b) {
      // 128 floats of the wave's part of buffer s per batch tile, each written once and
      // read once: a location reused for the next tile would let the compiler keep, for
      // the lanes that do not write it, the value they loaded for the previous tile
      float* scr = red + (((size_t)s * nwaves + wave) * NT * BTN + b) * 128;  // [j][row]
      f32x4 sj[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) sj[j] = mfma_bf16_k32(act[s][b][j], ones, z4);
      if (m == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) scr[j * 16 + 4 * g + q] = sj[j][q];
      }
      asm volatile("" ::: "memory");  // the reads below see the other lanes' writes
      u16 h0, l0, h1, l1;
      split_bf16(scr[(2 * g) * 16 + m], h0, l0);
      split_bf16(scr[(2 * g + 1) * 16 + m], h1, l1);
      aS[s][b] = u32x2{(u32)h0 | ((u32)l0 << 16), (u32)h1 | ((u32)l1 << 16)};
    }
  }
  float rs = 1.0f;  // 1 / rms of the input row
  if (a.ss && e < n_elem && e_brow < a.B) {
    // (the empty asm keeps the sum from being hoisted above the prologue's loads)
#pragma unroll
    for (int s = 0; s < 16; ++s) asm volatile("" : "+v"(sv[s]));
    double ssv = 0.0;
#pragma unroll
    for (int s = 0; s < 16; ++s) ssv += sv[s];
    rs = 1.0f / sqrtf((float)ssv * a.inv_k + a.eps);
  }

  for (int gl = 0; gl < ng; ++gl) {
    TileRows tr[NT];
    int seg, local;
    group_rows(g0 + gl, tr, seg, local);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < nst) {
        const int q = gl * nst + s;
        if (q + D - 1 < nq) issue(q + D - 1);
        __builtin_amdgcn_sched_barrier(0);
        const int younger = min(D - 1, nq - 1 - q);
        if (younger >= D - 1)
          wait_vmcnt<(D - 1) * KW>();
        else if (D > 2 && younger == 1)
          wait_vmcnt<KW>();
        else if (D > 3 && younger == 2)
          wait_vmcnt<2 * KW>();
        else
          wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
        lds_u8* slots[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) slots[t] = slot_of(q, t);
        if constexpr (WT == 12) {
          q4_step_tl<NT, BTN>(slots, act[s], aS[s], lane, acc);
        } else {
          u32 s16[NT];
#pragma unroll
          for (int t = 0; t < NT; ++t)
            s16[t] = addr::q6_s16((u32)(uintptr_t)(tr[t].base + (size_t)(sb0 + s) * kQ6KBytes) + tr[t].off(n));
          q6_step<NT, BTN, true>(a, slots, s16, &act[s][0][0], sb0 + s, lane, acc);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the group's partial sums: red[gl & 1][wave][t][b][lane * 2 + k]
    float* rb = red + (size_t)(gl & 1) * nwaves * NT * BTN * 128;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int b = 0; b < BTN; ++b) {
        float* r = rb + (((size_t)wave * NT + t) * BTN + b) * 128 + lane * 2;
        r[0] = acc[t][b][0] + acc[t][b][1];
        r[1] = acc[t][b][2] + acc[t][b][3];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[t][b][k] = 0.f;
      }
    lds_barrier();
    if (e < n_elem) {
      float v = 0.f, v2 = 0.f;
      {  // the waves' sums in wave order, each tile's reads issued at once
        constexpr int MW = 512 / 64;
        const size_t ws = (size_t)NT * BTN * 128;
        float x[MW];
        const float* r0 = rb + ((size_t)e_t * BTN + e_b) * 128 + e_rem;
#pragma unroll
        for (int w = 0; w < MW; ++w) x[w] = r0[(size_t)min(w, nwaves - 1) * ws];
#pragma unroll
        for (int w = 0; w < MW; ++w) v += w < nwaves ? x[w] : 0.f;
        if (a.epi == kEpiSwiGLU) {
          const float* r1 = rb + ((size_t)1 * BTN + e_b) * 128 + e_rem;
#pragma unroll
          for (int w = 0; w < MW; ++w) x[w] = r1[(size_t)min(w, nwaves - 1) * ws];
#pragma unroll
          for (int w = 0; w < MW; ++w) v2 += w < nwaves ? x[w] : 0.f;
        }
      }
      const int lt = a.epi == kEpiSwiGLU ? local : local * NT + e_t;
      const bool live = e_brow < a.B && lt * 16 + e_nn < rows_of(seg);
      if (live) {
        if (a.epi == kEpiSwiGLU) {
          const float gv = rs * v, uv = rs * v2;
          actpack_put(a.pack_out, a.pack_kind, a.pack_nslices, e_brow, lt * 16 + e_nn, gv / (1.0f + expf(-gv)) * uv);
        } else {
          a.y[(size_t)e_brow * a.ldy + col_of(seg) + lt * 16 + e_nn] = rs * v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Tile loop with whole-tile staging: the Q4_K gate/up pairs (the SwiGLU GEMM) at one
// activation tile.  The per-wave K slices above load 16 rows x 144 bytes per
// instruction, many short runs; here the workgroup's waves load each weight tile
// together, a tile being 16 rows of K / 256 consecutive super-blocks, consecutive in
// memory, so every 1 KB instruction reads a few long runs (gemm_addr.h: wt_*; each row
// is rotated in LDS so that one column of 16 rows falls on different banks).  One
// workgroup per CU, one wave per super-block of K (its activation fragments held in
// registers for the whole launch), a three-slot ring of whole tiles: two tiles in
// flight while one is computed.  Stage q is tile q of the workgroup's run (gate and up
// of pair q / 2); the pairs are split over the grid in proportion (the first
// workgroups take one more when they do not divide).
//
// Step q: wait for this wave's loads of stage q (those of stage q + 1 may stay in
// flight), then a workgroup barrier (every wave's loads of stage q have landed, and
// every wave is done reading the slot of stage q - 1), then (even q) the previous
// pair's epilogue from the reduction buffer, then the loads of stage q + 2 into the
// freed slot, then stage q's math; after the up tile (odd q) each wave writes its two
// tiles' partial sums to the reduction buffer, which the next step's barrier publishes.
// One barrier per tile.  The epilogue's stores go out before the next loads, so waiting
// for those loads does not wait for stores issued after them.
constexpr int kTlwSlots = 3;  // four (three tiles in flight, all 160 KB) measured slower: gate/up 22.2 against 21.3 us
constexpr int kTlwStore = 0, kTlwResidual = 1, kTlwPair = 2;

inline int tlw_waves(int nsb) { return nsb; }
inline size_t tlw_lds_bytes(int nsb) {
  return (size_t)kTlwSlots * addr::wt_slot_bytes(nsb) + (size_t)2 * tlw_waves(nsb) * 128 * sizeof(float);
}

// One whole-tile staging load (16 bytes per lane into dst + 16 lane).
GR_DEV void issue_wt(__amdgpu_buffer_rsrc_t rs, lds_u8* dst, u32 voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)dst, 16, voff, 0, 0, 0);
}

// MODE: kTlwStore (plain store), kTlwResidual (x += ..., the next input's packs and
// sum of squares), kTlwPair (gate/up pairs with SwiGLU)
template <int MODE>
__global__ __launch_bounds__(1024) void gemm_tlw_kernel(GemmArgs a) {
  constexpr bool PAIR = MODE == kTlwPair;
  constexpr int SPG = PAIR ? 2 : 1;  // stages (tiles) per group
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int KWI = addr::kWtInstr;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;  // = nsb: wave w computes super-block w
  const int n = lane & 15;
  const int nsb = a.nsb;
  const int U = addr::wt_units(nsb);
  const u32 slot_bytes = addr::wt_slot_bytes(nsb);
  const int kwi = (addr::wt_instrs(nsb) + nwaves - 1) / nwaves;  // loads per wave and tile (<= KWI)
  lds_u8* const slots = (lds_u8*)lds;
  // reduction buffer [2][waves][128]: the two tiles of a pair, or (single tiles) two
  // groups in turn, so a group's partial sums never overwrite ones still being read
  float* const red = (float*)(lds + kTlwSlots * (size_t)slot_bytes);

  if (a.zero_ptr && blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.zero_n; i += blockDim.x) a.zero_ptr[i] = 0.0;

  const int g0 = (int)(((long long)blockIdx.x * a.tl_groups) / gridDim.x);
  const int ng = (int)(((long long)(blockIdx.x + 1) * a.tl_groups) / gridDim.x) - g0;
  if (ng <= 0) return;  // workgroup-uniform, before any barrier
  const int nq = SPG * ng;
  // the matrices (at most three; SwiGLU: gate, up) and the group -> (matrix, tile) map
  const int off1 = a.seg_tile_off[1], off2 = a.seg_tile_off[2], nseg = a.nseg;
  auto seg_of = [&](int gi) { return PAIR ? 0 : (nseg > 1 && gi >= off1 ? 1 : 0) + (nseg > 2 && gi >= off2 ? 1 : 0); };
  auto seg_off = [&](int sg) { return sg == 0 ? 0 : sg == 1 ? off1 : off2; };
  // this lane's source offsets of its loads (the same for every tile; a ragged tile's
  // descriptor ends at its last row, so the rest read 0)
  u32 voff[KWI];
#pragma unroll
  for (int k = 0; k < KWI; ++k) voff[k] = addr::wt_src(addr::wt_instr(wave, nwaves, k, nsb), lane, nsb);
  auto issue = [&](int q) {
    const int gi = g0 + q / SPG;
    const int sg = PAIR ? (q & 1) : seg_of(gi);          // the matrix
    const int lt = PAIR ? gi : gi - seg_off(sg);         // tile within it
    const uint8_t* base = (sg == 0 ? a.w[0] : sg == 1 ? a.w[1] : a.w[2]) + (size_t)lt * 16 * a.row_bytes;
    const int nvalid = min(16, (sg == 0 ? a.seg_rows[0] : sg == 1 ? a.seg_rows[1] : a.seg_rows[2]) - lt * 16);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)(u32)((size_t)nvalid * a.row_bytes), kBufDword3);
    lds_u8* slot = slots + (q % kTlwSlots) * slot_bytes;
#pragma unroll
    for (int k = 0; k < KWI; ++k)
      if (k < kwi) issue_wt(rs, slot + 1024u * (u32)addr::wt_instr(wave, nwaves, k, nsb), voff[k]);
  };
  // the loads of one stage are kwi instructions: a wait that leaves the y younger stages
  // in flight allows exactly y kwi outstanding
  auto wait_younger = [&](int y) { wait_vmcnt_n(y * kwi); };

  // prologue: RMSNorm partial sums, this wave's activation fragments, then stages 0, 1
  const int e = threadIdx.x;
  const int e_brow = 2 * ((e & 127) >> 5) + (e & 1);  // the epilogue element's batch row
  double sv[16];
  if (a.ss && wave < 2) {  // the epilogue's threads (e < 128)
    const int row = min(e_brow, a.B - 1);
#pragma unroll
    for (int q = 0; q < 16; ++q) sv[q] = a.ss[q * a.B + row];
  }
  u32x4 act[1][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) act[0][j] = ((const u32x4*)a.xpack)[((size_t)wave * 8 + j) * 64 + lane];
  // residual update: the first group's residual and gain (before the stages, so that
  // the waits below count the stages only)
  float pre_x = 0.f, pre_g = 1.f;
  if (MODE == kTlwResidual && e < 128 && ng > 0) {
    const int sg = seg_of(g0), lt = g0 - seg_off(sg);
    const int r = lt * 16 + ((e >> 1) & 15);
    const int rows_s = sg == 0 ? a.seg_rows[0] : sg == 1 ? a.seg_rows[1] : a.seg_rows[2];
    const int col_s = sg == 0 ? a.seg_col_off[0] : sg == 1 ? a.seg_col_off[1] : a.seg_col_off[2];
    if (e_brow < a.B && r < rows_s) {
      pre_x = a.y[(size_t)e_brow * a.ldy + col_s + r];
      pre_g = a.gain ? a.gain[col_s + r] : 1.f;
    }
  }
  const int pro = min(kTlwSlots - 1, nq);  // stages in flight from the start
  for (int q = 0; q < pro; ++q) issue(q);
  wait_younger(pro);  // the loads above (older than the stages) have landed
  float rs = 1.0f;  // 1 / rms of the input row (first, so that the partial sums die early)
  if (a.ss && e < 128 && e_brow < a.B) {
    double ssv = 0.0;
#pragma unroll
    for (int q = 0; q < 16; ++q) ssv += sv[q];
    rs = 1.0f / sqrtf((float)ssv * a.inv_k + a.eps);
  }
  // sub-block sums of the wave's super-block, through its scratch in the last slot (not
  // loaded before step 0's barrier)
  u32x2 aS[1];
  {
    const u32x4 ones = {kOnesBf16, kOnesBf16, kOnesBf16, kOnesBf16};
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const int m = lane & 15, g = lane >> 4;
    float* scr = (float*)(slots + (kTlwSlots - 1) * (size_t)slot_bytes) + (size_t)wave * 128;  // [j][row], once
    f32x4 sj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sj[j] = mfma_bf16_k32(act[0][j], ones, z4);
    if (m == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) scr[j * 16 + 4 * g + t] = sj[j][t];
    }
    asm volatile("" ::: "memory");  // the reads below see the other lanes' writes
    u16 h0, l0, h1, l1;
    split_bf16(scr[(2 * g) * 16 + m], h0, l0);
    split_bf16(scr[(2 * g + 1) * 16 + m], h1, l1);
    aS[0] = u32x2{(u32)h0 | ((u32)l0 << 16), (u32)h1 | ((u32)l1 << 16)};
  }

  // row n of a slot, and the unit column of this wave's super-block in that row
  const int c0 = [&] {
    const int c = 9 * wave + addr::wt_rot(n, U);
    return c >= U ? c - U : c;
  }();
  auto epilogue = [&](int pr) {  // group g0 + pr, from the reduction buffer
    // the element's indices are recomputed here from an opaque copy of the thread index,
    // so that they are not held in registers across the main loop
    int ee = threadIdx.x;
    asm volatile("" : "+v"(ee));
    if (ee < 128) {
      const int erem = ee & 127, elp = erem >> 1;
      const int brow = 2 * (elp >> 4) + (erem & 1);
      const int gi = g0 + pr;
      const float* r0 = red + (size_t)(PAIR ? 0 : (pr & 1)) * nwaves * 128;
      float v = 0.f, v2 = 0.f;
      for (int w = 0; w < nwaves; ++w) {
        v += r0[(size_t)w * 128 + erem];
        if (PAIR) v2 += red[((size_t)nwaves + w) * 128 + erem];
      }
      if (PAIR) {
        const int col = gi * 16 + (elp & 15);
        if (brow < a.B && col < a.seg_rows[0]) {
          const float gv = rs * v, uv = rs * v2;
          actpack_put(a.pack_out, a.pack_kind, a.pack_nslices, brow, col, gv / (1.0f + expf(-gv)) * uv);
        }
      } else {
        const int sg = seg_of(gi), lt = gi - seg_off(sg);
        const int rows_s = sg == 0 ? a.seg_rows[0] : sg == 1 ? a.seg_rows[1] : a.seg_rows[2];
        const int col_s = sg == 0 ? a.seg_col_off[0] : sg == 1 ? a.seg_col_off[1] : a.seg_col_off[2];
        const int r = lt * 16 + (elp & 15);
        const bool live = brow < a.B && r < rows_s;
        const size_t yi = (size_t)brow * a.ldy + col_s + r;
        if (MODE == kTlwStore) {
          if (live) a.y[yi] = rs * v;
        } else {  // residual update: x += rs v, the next input's packs and sum of squares
          float xn = 0.f;
          if (live) {
            const float xv = pr == 0 ? pre_x : a.y[yi];
            const float gv = pr == 0 ? pre_g : (a.gain ? a.gain[col_s + r] : 1.f);
            xn = xv + rs * v;
            a.y[yi] = xn;
            const float pv = xn * gv;
            if (a.pack_out) actpack_put(a.pack_out, a.pack_kind, a.pack_nslices, brow, col_s + r, pv);
            if (a.pack_out2) actpack_put(a.pack_out2, a.pack_kind2, a.pack_nslices2, brow, col_s + r, pv);
          }
          // over the tile's 16 columns of each batch row: lanes with the same (row pair,
          // k2) differ in nn, bits 1..4 of the thread index (waves 0 and 1 whole here)
          float sq = xn * xn;
#pragma unroll
          for (int o = 2; o <= 16; o <<= 1) sq += __shfl_xor(sq, o, 64);
          if ((elp & 15) == 0 && brow < a.B && a.ss_out)
            atomicAdd(a.ss_out + (size_t)(gi % a.ss_slots) * a.B + brow, (double)sq);
        }
      }
    }
  };

  float acc[SPG][1][4];
#pragma unroll
  for (int t = 0; t < SPG; ++t)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[t][0][k] = 0.f;

  for (int pr = 0; pr < ng; ++pr) {
#pragma unroll
    for (int t = 0; t < SPG; ++t) {
      const int q = SPG * pr + t;
      wait_younger(min(kTlwSlots - 2, nq - 1 - q));  // stage q has landed
      lds_barrier();
      if (t == 0 && pr > 0) epilogue(pr - 1);
      if (q + kTlwSlots - 1 < nq) issue(q + kTlwSlots - 1);
      __builtin_amdgcn_sched_barrier(0);
      const lds_u8* rowp = slots + (q % kTlwSlots) * slot_bytes + (size_t)n * U * 16;
      q4_step_tlw<1>(rowp, c0, U, act, aS, lane, acc[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the group's partial sums: red[t or pr & 1][wave][lane * 2 + k]
#pragma unroll
    for (int t = 0; t < SPG; ++t) {
      float* r = red + ((size_t)(PAIR ? t : (pr & 1)) * nwaves + wave) * 128 + lane * 2;
      r[0] = acc[t][0][0] + acc[t][0][1];
      r[1] = acc[t][0][2] + acc[t][0][3];
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[t][0][k] = 0.f;
    }
  }
  lds_barrier();
  epilogue(ng - 1);
}

// ---------------------------------------------------------------------------------
// Row-block kernel: the Q4_K gate/up pairs (SwiGLU) at 17 to 32 rows (four activation
// tiles: a 32-row decode step, a four-token verification step).  The split-K kernel's
// waves read every row's activation fragments from L2 for each weight tile, which at 32
// rows is 14 times the tile's own bytes.  Here each wave holds the fragments of the four
// activation tiles for
// one super-block in registers (128 VGPRs, two waves per SIMD) for the whole launch, so a
// workgroup of W waves covers a K range of W super-blocks and nkr = K / 256 / W
// workgroups cover K.  Weight tiles stream as in the whole-tile kernel: the 16 rows of
// the range, loaded together by the waves (gemm_addr.h: wt_src_rows) into a three-slot
// LDS ring, two in flight; each expanded weight fragment feeds the four activation
// tiles' MFMAs.  Per pair the waves' sums meet in LDS as the range's partial sums, which
// go to memory (agent scope) after the loop.  Then a workgroup counts its arrival on each
// of its pairs (one agent-scope counter per pair, zero between launches) and, where it
// arrives last, adds the nkr partials in range order (so the result does not depend on
// which range came last), applies the SwiGLU epilogue and resets the counter.  With one
// range (K of at most 8 super-blocks) the epilogue runs straight from LDS.  Measured at
// Qwen3-8B (32 rows, 768 pairs, K = 4096 in two ranges): 46 us against the split-K
// kernel's 49 us; it is bound by its math (41 us with the weight loads removed: 68 MFMAs
// and about 350 other vector instructions per wave and tile at two waves per SIMD), so
// for QKV and Wo (two or three tiles per workgroup, whose prologue loads 256 KB of
// activation fragments) it was slower (20.0 and 18.7 us against 18.6 and 14.0).
// Agent-scope (device-wide) store and load: past the per-XCD L2 (the partial sums of
// one tile are written and read on different XCDs).
GR_DEV void gst_agent(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
GR_DEV float gld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kRbBT = 4;          // activation tiles
constexpr int kRbSlots = 3;       // ring slots: two tiles in flight while one is computed
constexpr int kRbMaxWaves = 8;    // super-blocks per range (128 activation VGPRs per wave)
constexpr int kRbMaxRanges = 8;
constexpr int kRbMaxGroups = 64;  // tile groups per workgroup
constexpr int kRbElems = kRbBT * 128;  // outputs of one tile: 16 columns x 32 rows

int rb_ranges(int nsb) {
  for (int nkr = (nsb + kRbMaxWaves - 1) / kRbMaxWaves; nkr <= nsb / 4 && nkr <= kRbMaxRanges; ++nkr)
    if (nkr >= 1 && nsb % nkr == 0) return nkr;
  return 0;
}
// reduction buffers: [2 (pr & 1)][2 (gate, up)][W][BT][128] floats, then (several ranges)
// the workgroup's partial sums [ngm][SPG][kRbElems] until they are stored at the end
inline size_t rb_lds_bytes(int W, int ngm, int spg) {
  return (size_t)kRbSlots * addr::wt_slot_bytes(W) + (size_t)4 * W * kRbBT * 128 * sizeof(float) +
         (size_t)ngm * spg * kRbElems * sizeof(float);
}
constexpr size_t kRbStaticLds = kSsCap * sizeof(double) + kRbMaxGroups * sizeof(uint32_t);

template <int NK>
GR_DEV float rb_sum(const float* p, size_t stride) {
  float v[NK];
#pragma unroll
  for (int q = 0; q < NK; ++q) v[q] = gld_agent(p + (size_t)q * stride);
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < NK; ++q) s += v[q];
  return s;
}
// the nk partials p[0], p[stride], ... added in order (all loads issued at once)
GR_DEV float rb_sum_n(const float* p, size_t stride, int nk) {
  switch (nk) {
    case 1: return rb_sum<1>(p, stride);
    case 2: return rb_sum<2>(p, stride);
    case 3: return rb_sum<3>(p, stride);
    case 4: return rb_sum<4>(p, stride);
    case 5: return rb_sum<5>(p, stride);
    case 6: return rb_sum<6>(p, stride);
    case 7: return rb_sum<7>(p, stride);
    default: return rb_sum<8>(p, stride);
  }
}

// Grid: nkr workgroups per slot, workgroup i takes range i % nkr and the (i / nkr)-th
// share of the gate/up pairs.
__global__ __launch_bounds__(kRbMaxWaves * 64) void gemm_rb_kernel(GemmArgs a) {
  constexpr int SPG = 2;  // stages (tiles) per pair: gate, up
  constexpr int BT = kRbBT, NE = kRbElems;
  constexpr int KWI = addr::kWtInstr;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ double s_ss[kSsCap];         // the input rows' RMSNorm partial sums
  __shared__ uint32_t s_last[kRbMaxGroups];  // this workgroup arrived last on group g0 + t
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int W = nthr >> 6;  // super-blocks of the range: wave w computes super-block kr W + w
  const int n = lane & 15;
  const int nkr = a.nsb / W;
  const int kr = (int)blockIdx.x % nkr;
  const int U = addr::wt_units(W);
  const u32 slot_bytes = addr::wt_slot_bytes(W);
  const int kwi = (addr::wt_instrs(W) + W - 1) / W;  // loads per wave and tile (<= KWI)
  lds_u8* const slots = (lds_u8*)lds;
  // reduction buffers red[buf][wave][b][128]: buf = 2 (pr & 1) + t, tile t (gate / up, or
  // the single tile) of group pr, so a group's sums never overwrite ones still being read
  float* const red = (float*)(lds + kRbSlots * (size_t)slot_bytes);
  auto red_buf = [&](int pr, int t) { return red + (size_t)(2 * (pr & 1) + t) * W * BT * 128; };
  float* const outb = red + (size_t)4 * W * BT * 128;  // [ng][SPG][NE]: this range's partials

  if (a.zero_ptr && blockIdx.x == 0)
    for (int i = tid; i < a.zero_n; i += nthr) a.zero_ptr[i] = 0.0;

  const int G = a.tl_groups, per = (int)gridDim.x / nkr, wi = (int)blockIdx.x / nkr;
  const int g0 = (int)(((long long)wi * G) / per);
  const int ng = (int)(((long long)(wi + 1) * G) / per) - g0;
  if (ng <= 0) return;  // workgroup-uniform, before any barrier
  const int nq = SPG * ng;
  const int sbr = kr * W;  // the range's first super-block
  const u32 rbytes = (u32)a.row_bytes;
  u32 voff[KWI];
#pragma unroll
  for (int k = 0; k < KWI; ++k) voff[k] = addr::wt_src_rows(addr::wt_instr(wave, W, k, W), lane, W, rbytes);
  auto issue = [&](int q) {  // stage q: tile (gate q even, up q odd) of pair g0 + q / 2
    const int gi = g0 + q / SPG;
    const uint8_t* base = ((q & 1) ? a.w[1] : a.w[0]) + (size_t)gi * 16 * a.row_bytes + (size_t)sbr * kQ4KBytes;
    const int nvalid = min(16, a.seg_rows[0] - gi * 16);
    // the descriptor ends with the last valid row's range: the rows past it read 0
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)base, 0, (int)((u32)(nvalid - 1) * rbytes + 16u * (u32)U), kBufDword3);
    lds_u8* slot = slots + (q % kRbSlots) * slot_bytes;
#pragma unroll
    for (int k = 0; k < KWI; ++k)
      if (k < kwi) issue_wt(rs, slot + 1024u * (u32)addr::wt_instr(wave, W, k, W), voff[k]);
  };
  auto wait_younger = [&](int y) { wait_vmcnt_n(y * kwi); };

  // prologue: the RMSNorm partial sums, this wave's activation fragments, then stages 0, 1
  const int n_ss = a.ss ? a.ss_slots * a.B : 0;  // <= kSsCap <= nthr
  const double ssp = tid < n_ss ? a.ss[tid] : 0.0;
  const size_t tile_frags = (size_t)a.nsb * 8;
  u32x4 act[BT][8];
#pragma unroll
  for (int b = 0; b < BT; ++b)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      act[b][j] = ((const u32x4*)a.xpack)[((size_t)b * tile_frags + (size_t)(sbr + wave) * 8 + j) * 64 + lane];
  const int pro = min(kRbSlots - 1, nq);
  for (int q = 0; q < pro; ++q) issue(q);
  wait_younger(pro);  // the loads above (older than the stages) have landed
  if (tid < n_ss) s_ss[tid] = ssp;  // published by step 0's barrier
  // sub-block sums of the wave's super-block per activation tile, through the wave's part
  // of the reduction buffer (first written after step 0's barrier)
  u32x2 aS[BT];
  {
    const u32x4 ones = {kOnesBf16, kOnesBf16, kOnesBf16, kOnesBf16};
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      float* scr = red + ((size_t)wave * BT + b) * 128;  // [j][row], each written and read once
      f32x4 sj[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) sj[j] = mfma_bf16_k32(act[b][j], ones, z4);
      if (m == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int t = 0; t < 4; ++t) scr[j * 16 + 4 * g + t] = sj[j][t];
      }
      asm volatile("" ::: "memory");  // the reads below see the other lanes' writes
      u16 h0, l0, h1, l1;
      split_bf16(scr[(2 * g) * 16 + m], h0, l0);
      split_bf16(scr[(2 * g + 1) * 16 + m], h1, l1);
      aS[b] = u32x2{(u32)h0 | ((u32)l0 << 16), (u32)h1 | ((u32)l1 << 16)};
    }
  }
  const int c0 = [&] {
    const int c = 9 * wave + addr::wt_rot(n, U);
    return c >= U ? c - U : c;
  }();

  // The SwiGLU epilogue of pair gi on the finished sums of element e (gate v, up v2).
  auto finish = [&](int gi, int e, bool in, float v, float v2) {
    const int rem = e & 127, lp = rem >> 1;
    const int brow = 8 * (e >> 7) + 2 * (lp >> 4) + (rem & 1), col = gi * 16 + (lp & 15);
    if (in && brow < a.B && col < a.seg_rows[0]) {
      float rs = 1.0f;  // 1 / rms of the input row
      if (n_ss) {
        double ssv = 0.0;
        for (int s = 0; s < a.ss_slots; ++s) ssv += s_ss[s * a.B + brow];
        rs = 1.0f / sqrtf((float)ssv * a.inv_k + a.eps);
      }
      const float gv = rs * v, uv = rs * v2;
      actpack_put(a.pack_out, a.pack_kind, a.pack_nslices, brow, col, gv / (1.0f + expf(-gv)) * uv);
    }
  };
  // group pr's sums from the reduction buffer: kept in LDS as this range's partials (stored
  // after the loop, so that no stage's wait waits for them), or (one range) finished at once
  auto publish = [&](int pr) {
    const int gi = g0 + pr;
    for (int e0 = 0; e0 < NE; e0 += nthr) {
      const int e = e0 + tid;
      const bool in = e < NE;
      const int ee = in ? e : 0;
      const int b = ee >> 7, rem = ee & 127;
      float v[SPG];
#pragma unroll
      for (int t = 0; t < SPG; ++t) {
        const float* r0 = red_buf(pr, t) + (size_t)b * 128 + rem;  // [wave][b][128]
        // the W waves' sums in wave order, all eight reads issued at once (a loop over
        // the run-time W waited for each read before the next)
        float x[kRbMaxWaves];
#pragma unroll
        for (int w = 0; w < kRbMaxWaves; ++w) x[w] = r0[(size_t)min(w, W - 1) * BT * 128];
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kRbMaxWaves; ++w) s += w < W ? x[w] : 0.f;
        v[t] = s;
      }
      if (nkr == 1) {
        finish(gi, ee, in, v[0], v[1]);
      } else if (in) {
#pragma unroll
        for (int t = 0; t < SPG; ++t) outb[((size_t)pr * SPG + t) * NE + e] = v[t];
      }
    }
  };

  float acc[BT][4];  // one tile's sums: stored to its reduction buffer after its step
#pragma unroll
  for (int b = 0; b < BT; ++b)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[b][k] = 0.f;

  for (int pr = 0; pr < ng; ++pr) {
#pragma unroll
    for (int t = 0; t < SPG; ++t) {
      const int q = SPG * pr + t;
      wait_younger(min(kRbSlots - 2, nq - 1 - q));  // stage q has landed
      lds_barrier();
      if (t == 0 && pr > 0) publish(pr - 1);
      if (q + kRbSlots - 1 < nq) issue(q + kRbSlots - 1);
      __builtin_amdgcn_sched_barrier(0);
      const lds_u8* rowp = slots + (q % kRbSlots) * slot_bytes + (size_t)n * U * 16;
      q4_step_tlw<BT>(rowp, c0, U, act, aS, lane, acc);
      __builtin_amdgcn_sched_barrier(0);
      // the tile's partial sums: red_buf(pr, t)[wave][b][lane * 2 + k]
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        float* r = red_buf(pr, t) + ((size_t)wave * BT + b) * 128 + lane * 2;
        r[0] = acc[b][0] + acc[b][1];
        r[1] = acc[b][2] + acc[b][3];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[b][k] = 0.f;
      }
    }
  }
  lds_barrier();
  publish(ng - 1);
  if (nkr == 1) return;

  // ---- the partials to memory, all at once; they are stored before any arrival is
  // counted, and the last arriver on a group adds its ranges' partials
  __syncthreads();
  for (int i = tid; i < ng * SPG * NE; i += nthr)
    gst_agent(a.part + ((size_t)kr * G + g0) * SPG * NE + i, outb[i]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid < ng)
    s_last[tid] = __hip_atomic_fetch_add(a.rb_cnt + g0 + tid, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (uint32_t)(nkr - 1);
  __syncthreads();
  for (int t = 0; t < ng; ++t) {
    if (!s_last[t]) continue;  // workgroup-uniform
    const int gi = g0 + t;
    const size_t stride = (size_t)G * SPG * NE;  // from one range's partial to the next
    for (int e0 = 0; e0 < NE; e0 += nthr) {
      const int e = e0 + tid;
      const bool in = e < NE;
      const int ee = in ? e : 0;
      const float* p0 = a.part + ((size_t)gi * SPG) * NE + ee;
      finish(gi, ee, in, rb_sum_n(p0, stride, nkr), rb_sum_n(p0 + NE, stride, nkr));
    }
    if (tid == 0) __hip_atomic_store(a.rb_cnt + gi, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------------
// K-chunk staging: the Q6_K residual GEMM (down) at one activation tile, rows of a
// multiple of 16 bytes.  One 16-row tile per workgroup, C waves; stage c is super-blocks
// [C c, C c + C) of the tile's 16 rows (gemm_addr.h: kc_*), loaded by all waves
// together as runs of consecutive bytes per row into a three-slot LDS ring; wave w
// computes super-block C c + w of stage c with its activation fragments one stage ahead
// in registers.  Load order: a(0), w(0), w(1), then at step c (after the barrier) a(c + 1)
// and w(c + 2); so before step c's math the loads younger than a(c) and w(c) are exactly
// w(c + 1) when it exists, and one wait count (one stage) covers every step but the last.
// The waves' sums meet in LDS for the residual epilogue of gemm_kernel.
constexpr int kKcwSlots = 3;

inline size_t kcw_lds_bytes(int C) {
  const size_t ring = (size_t)kKcwSlots * addr::kc_slot_bytes(C);
  const size_t red = (size_t)C * 128 * sizeof(float) + kSsCap * sizeof(double);
  return ring > red ? ring : red;
}
// Waves (= super-blocks per stage) for K / 256 = nsb: the most, up to 16, that divide
// nsb and whose three stages fit the LDS; 0 if none (or fewer than two).
int kcw_waves(int nsb) {
  for (int c = 16; c >= 2; --c)
    if (nsb % c == 0 && kcw_lds_bytes(c) <= (size_t)kGemmLds) return c;
  return 0;
}

struct KcwAct {
  u32x4 a[8];
};

__global__ __launch_bounds__(1024) void gemm_kcw_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int C = blockDim.x >> 6;  // waves = super-blocks per stage
  const int nch = a.nsb / C;      // stages
  const int n = lane & 15, kg = lane >> 4;
  const int tile = blockIdx.x;
  const u32 slot_bytes = addr::kc_slot_bytes(C);
  const int stride = addr::kc_stride(C);
  const int kwi = (addr::kc_instrs(C) + C - 1) / C;  // loads per wave and stage (<= 5)
  lds_u8* const slots = (lds_u8*)lds;

  if (a.zero_ptr && tile == 0)
    for (int i = threadIdx.x; i < a.zero_n; i += blockDim.x) a.zero_ptr[i] = 0.0;

  const int rows_n = a.seg_rows[0];
  const int nvalid = min(16, rows_n - tile * 16);
  const uint8_t* const tbase = a.w[0] + (size_t)tile * 16 * a.row_bytes;
  u32 voff[addr::kWtInstr];
#pragma unroll
  for (int k = 0; k < addr::kWtInstr; ++k)
    voff[k] = addr::kc_src(addr::kc_instr(wave, C, k, C), lane, C, (u32)a.row_bytes);
  auto issue = [&](int c) {
    const u32 ws = addr::kc_window(C, c);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(tbase + ws), 0, (int)(u32)((size_t)nvalid * a.row_bytes - ws), kBufDword3);
    lds_u8* slot = slots + (c % kKcwSlots) * slot_bytes;
#pragma unroll
    for (int k = 0; k < addr::kWtInstr; ++k)
      if (k < kwi) issue_wt(rs, slot + 1024u * (u32)addr::kc_instr(wave, C, k, C), voff[k]);
  };
  auto load_act = [&](KcwAct& b, int c) {
    const int sb = c * C + wave;
#pragma unroll
    for (int j = 0; j < 8; ++j) b.a[j] = ((const u32x4*)a.xpack)[((size_t)sb * 8 + j) * 64 + lane];
  };
  auto wait_stage = [&]() {  // leaves one stage's loads in flight
    if (kwi == 5)
      wait_vmcnt<5>();
    else if (kwi == 4)
      wait_vmcnt<4>();
    else if (kwi == 3)
      wait_vmcnt<3>();
    else if (kwi == 2)
      wait_vmcnt<2>();
    else
      wait_vmcnt<1>();
  };

  // the epilogue element of this thread (threads < 128): output row brow, column col
  const int e = threadIdx.x;
  const int e_nn = (e >> 1) & 15, e_brow = 2 * (e >> 5) + (e & 1);
  const bool e_live = e < 128 && e_brow < a.B && tile * 16 + e_nn < rows_n;
  const int e_col = a.seg_col_off[0] + tile * 16 + e_nn;
  // operands of the epilogue that do not depend on the GEMM, loaded first
  const double ssp = (a.ss && (int)threadIdx.x < a.ss_slots * a.B) ? a.ss[threadIdx.x] : 0.0;
  const float pre_x = (e_live && a.epi == kEpiResidual) ? a.y[(size_t)e_brow * a.ldy + e_col] : 0.f;
  const float pre_g = (e_live && a.epi == kEpiResidual && a.gain) ? a.gain[e_col] : 1.f;

  KcwAct b0, b1;
  load_act(b0, 0);
  issue(0);
  if (nch > 1) issue(1);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto step = [&](int c, const KcwAct& cur, KcwAct& nxt) {
    if (c + 1 < nch)
      wait_stage();
    else
      wait_vmcnt<0>();
    lds_barrier();
    if (c + 1 < nch) load_act(nxt, c + 1);
    if (c + 2 < nch) issue(c + 2);
    __builtin_amdgcn_sched_barrier(0);
    const u32 x0 = addr::kc_s16(C, c) + 210u * (u32)wave;  // the block's first byte in the window
    const lds_u8* rs = slots + (c % kKcwSlots) * slot_bytes + addr::kc_lds_byte(n, x0 & ~3u, C);
    Q6Regs w;
    q6_load_at(rs, x0 & 3u, kg, w);
    q6_step_w(w, cur.a, acc);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int c = 0; c < nch; c += 2) {
    step(c, b0, b1);
    if (c + 1 < nch) step(c + 1, b1, b0);
  }
  (void)stride;

  // the waves' sums (hi + lo parts of each batch row) through LDS, then the epilogue
  lds_barrier();  // every wave is done with the ring
  float* red = (float*)lds;  // [waves][128]
  red[(size_t)wave * 128 + lane * 2] = acc[0] + acc[1];
  red[(size_t)wave * 128 + lane * 2 + 1] = acc[2] + acc[3];
  double* s_ss = (double*)(red + (size_t)C * 128);
  if (a.ss && (int)threadIdx.x < a.ss_slots * a.B) s_ss[threadIdx.x] = ssp;
  __syncthreads();
  if (e < 128) {  // waves 0 and 1, whole: the shuffles below see every lane
    float v = 0.f;
    for (int w2 = 0; w2 < C; ++w2) v += red[(size_t)w2 * 128 + e];
    double ssv = 0.0;
    if (e_live && a.ss)
      for (int q = 0; q < a.ss_slots; ++q) ssv += s_ss[q * a.B + e_brow];
    const float rsn = e_live ? (a.ss ? 1.0f / sqrtf((float)ssv * a.inv_k + a.eps) : 1.0f) : 0.f;
    if (a.epi == kEpiStore) {
      if (e_live) a.y[(size_t)e_brow * a.ldy + e_col] = rsn * v;
    } else {
      float xn = 0.f;
      if (e_live) {
        xn = pre_x + rsn * v;
        a.y[(size_t)e_brow * a.ldy + e_col] = xn;
        const float pv = xn * pre_g;
        if (a.pack_out) actpack_put(a.pack_out, a.pack_kind, a.pack_nslices, e_brow, e_col, pv);
        if (a.pack_out2) actpack_put(a.pack_out2, a.pack_kind2, a.pack_nslices2, e_brow, e_col, pv);
      }
      // sum of squares over the tile's 16 columns of each batch row: lanes with the same
      // (row pair, k2) differ in nn, bits 1..4 of the thread index
      float sq = xn * xn;
#pragma unroll
      for (int o = 2; o <= 16; o <<= 1) sq += __shfl_xor(sq, o, 64);
      if (e_nn == 0 && e_brow < a.B && a.ss_out)
        atomicAdd(a.ss_out + (size_t)(tile % a.ss_slots) * a.B + e_brow, (double)sq);
    }
  }
}

// Which GEMMs take it: Q6_K with a residual update or a plain store, one activation
// tile, rows of a multiple of 16 bytes (K a multiple of 8 super-blocks), one matrix.
bool use_kcw(int wtype, int K, int B, int nmat) {
  const int nsb = K / kQK;
  return wtype == 14 && B <= 8 && nmat == 1 && K % kQK == 0 && nsb % 8 == 0 && kcw_waves(nsb) >= 2;
}

hipError_t launch_gemm_kcw(int tiles, GemmArgs a, hipStream_t st) {
  const int C = kcw_waves(a.nsb);
  if (tiles <= 0) return hipSuccess;
  if (C < 2 || a.nsb % C || a.B > 8 || a.nseg != 1 || a.row_bytes % 16 || (a.epi != kEpiResidual && a.epi != kEpiStore) ||
      (a.ss && a.ss_slots * a.B > C * 64) || (a.ss && a.ss_slots * a.B > kSsCap))
    return hipErrorInvalidValue;
  static const bool lds_set = [] {
    (void)hipFuncSetAttribute((const void*)gemm_kcw_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    (void)hipGetLastError();
    return true;
  }();
  (void)lds_set;
  void* kargs[] = {&a};
  const hipError_t e = launch_fn((const void*)gemm_kcw_kernel, dim3(tiles), dim3(C * 64), kcw_lds_bytes(C), st, kargs);
  return e != hipSuccess ? e : hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Many-row kernel (more than 64 rows: prompt chunks, long verification runs).  The
// skinny kernels above read every activation fragment once per weight tile, which is
// cheap for a few rows and dominates for hundreds.  Here a workgroup owns a 2-D output
// tile: MB activation tiles (8 rows each) x 16 weight tiles (16 rows each), with 8
// waves; wave w owns weight tiles 2w and 2w + 1 (SwiGLU: gate and up tile w) for all MB
// activation tiles, so each activation fragment read from LDS feeds two MFMAs and each
// expanded weight fragment feeds MB.  Per super-block the MB tiles' activation
// fragments are staged in LDS once for all waves (one workgroup barrier per
// super-block), and each wave streams its own two weight tiles through a private
// two-slot ring.  The whole K accumulates in registers (no split-K, no reduction).
//
// Q4_K arithmetic is the tile-loop kernel's: C_j = A_j x (-128) starts each sub-block's
// quant MFMA, so it returns sum a q; the mins term is one K = 16 MFMA per tile pair and
// super-block, its A operand the sub-block sums of each MFMA row, which an MFMA of a
// ones matrix against the activation fragment (passed as the B operand: the two
// operand layouts hold the same registers) returns already indexed by row.
// Q6_K arithmetic is q6_step's.

constexpr int kMmWaves = 8, kMmNT = 2;
constexpr int mm_mb(int wtype) { return wtype == 12 ? 4 : 2; }  // activation tiles per workgroup
constexpr int mm_wstage(int wtype) { return wtype == 12 ? kQ4Stage : kQ6Stage; }
// LDS: two activation stages (MB tiles x 8 fragments of 1 KB) and every wave's
// two-slot ring of its two weight tiles (Q4_K: 64 + 96 KB; Q6_K: 32 + 128 KB)
constexpr size_t mm_lds(int wtype) {
  return (size_t)2 * mm_mb(wtype) * 8 * 1024 + (size_t)kMmWaves * 2 * kMmNT * mm_wstage(wtype);
}
static_assert(mm_lds(12) <= (size_t)kGemmLds && mm_lds(14) <= (size_t)kGemmLds, "many-row LDS");

template <int BT>
GR_DEV void q4_step_mm(const lds_u8* as, lds_u8* const (&slot)[kMmNT], int lane, float (&acc)[kMmNT][BT][4]) {
  constexpr int NT = kMmNT;
  const u32x4 neg128 = {kNeg128Bf16, kNeg128Bf16, kNeg128Bf16, kNeg128Bf16};
  const u32x4 ones = {kOnesBf16, kOnesBf16, kOnesBf16, kOnesBf16};
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, kg = lane >> 4;
  const u32 M = vconst(0x43004300u);
  Q4Regs w[NT];
  float sd[NT][8], dmin[NT];
  u32x2 bm[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) q4_load_tl(slot[t] + addr::q4_lds_byte(n, 0), kg, w[t], sd[t], dmin[t], bm[t]);
  float se[BT], so[BT];  // S_2kg and S_2kg+1 of MFMA row l % 16
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 av[BT];
    f32x4 cj[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      av[b] = *(const __attribute__((address_space(3))) u32x4*)(as + (b * 8 + j) * 1024 + lane * 16);
      cj[b] = mfma_bf16_k32(av[b], neg128, z4);
      const f32x4 st = mfma_bf16_k32(ones, av[b], z4);  // every element: S_j of row l % 16
      if (j == 2 * kg) se[b] = st[0];
      if (j == 2 * kg + 1) so[b] = st[0];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 bq = q4_expand(w[t].qs[j >> 1], (j & 1) != 0, M);
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const f32x4 dd = mfma_bf16_k32(av[b], bq, cj[b]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][b][e] = __builtin_fmaf(sd[t][j], dd[e], acc[t][b][e]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    u16 h0, l0, h1, l1;
    split_bf16(se[b], h0, l0);
    split_bf16(so[b], h1, l1);
    const u32x2 aS = {(u32)h0 | ((u32)l0 << 16), (u32)h1 | ((u32)l1 << 16)};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 corr = mfma_bf16_k16(aS, bm[t], z4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][b][e] = __builtin_fmaf(-dmin[t], corr[e], acc[t][b][e]);
    }
  }
}

template <int BT>
GR_DEV void q6_step_mm(const lds_u8* as, lds_u8* const (&slot)[kMmNT], const u32 (&s16)[kMmNT], int lane,
                       float (&acc)[kMmNT][BT][4]) {
  constexpr int NT = kMmNT;
  const u32x2 neg160 = {kNeg160Bf16, kNeg160Bf16};
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, kg = lane >> 4;
  const u32 E = vconst(0x43434343u);
  Q6Regs w[NT];
  float dsc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    q6_load_lds(slot[t], s16[t], n, kg, w[t]);
    dsc[t] = h2f(w[t].d);
  }
#pragma unroll
  for (int hu = 0; hu < 4; ++hu) {
    const int h = hu >> 1, u = hu & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sub = 8 * h + 2 * r + u;  // 16-weight sub-block within the super-block
      u32x2 av[BT];
      f32x4 cs[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const u32x4 pr = *(const __attribute__((address_space(3))) u32x4*)(as + (b * 8 + (sub >> 1)) * 1024 + lane * 16);
        av[b] = (sub & 1) ? u32x2{pr.z, pr.w} : u32x2{pr.x, pr.y};
        cs[b] = mfma_bf16_k16(av[b], neg160, z4);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x2 bq = q6_expand(w[t].part[hu], r, E);
        const float sd = dsc[t] * (float)(int)(int8_t)((w[t].sc[sub >> 2] >> (8 * (sub & 3))) & 0xFF);
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          const f32x4 dd = mfma_bf16_k16(av[b], bq, cs[b]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][b][e] = __builtin_fmaf(sd, dd[e], acc[t][b][e]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Grid: mtiles * groups workgroups per K range (a.mm_mtiles = activation tiles / MB;
// a.mm_groups: groups of 16 weight tiles per matrix segment, or of 8 gate/up tile
// pairs), 512 threads.  a.seg_tile_off counts groups.
template <int WT, bool ALIGNED>
__global__ __launch_bounds__(512) void gemm_mm_kernel(GemmArgs a) {
  constexpr int MB = mm_mb(WT), BT = MB, NT = kMmNT;
  constexpr int kW = mm_wstage(WT);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  lds_u8* abuf = (lds_u8*)lds;                                                   // [2][MB * 8][1 KB]
  lds_u8* ring = (lds_u8*)lds + 2 * MB * 8 * 1024 + wave * (2 * NT * kW);         // [2][NT][kW]

  if (a.zero_ptr && blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.zero_n; i += blockDim.x) a.zero_ptr[i] = 0.0;

  // workgroup -> (activation tile group, weight tile group); on a grid that is a
  // multiple of 8, consecutive groups of weight tiles go to one XCD (workgroups are
  // dealt to the 8 XCDs round-robin), so the activation tiles sharing a weight tile
  // meet in that XCD's L2
  const int G = gridDim.x, bid = blockIdx.x;
  const int lg = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int mtiles = a.mm_mtiles, per_split = mtiles * a.mm_groups;
  const int ks = lg / per_split, rem = lg - ks * per_split;
  const int mt = rem % mtiles, ng = rem / mtiles;
  const int nsplit = a.part ? G / per_split : 1;
  const int sb_lo = ks * a.nsb / nsplit, sb_hi = (ks + 1) * a.nsb / nsplit;  // this workgroup's K range
  int seg = 0;
  if (a.epi != kEpiSwiGLU)
    while (seg + 1 < a.nseg && ng >= a.seg_tile_off[seg + 1]) ++seg;
  const int local = ng - (a.epi == kEpiSwiGLU ? 0 : a.seg_tile_off[seg]);
  // this wave's tiles: SwiGLU tile t = 0 gate, 1 up, both at column tile local * 8 + wave
  int lt[NT];
  TileRows tr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int sg = a.epi == kEpiSwiGLU ? t : seg;
    lt[t] = a.epi == kEpiSwiGLU ? local * kMmWaves + wave : local * (kMmWaves * NT) + wave * NT + t;
    int ltc = lt[t];
    if (ltc * 16 >= a.seg_rows[sg]) ltc = (a.seg_rows[sg] - 1) / 16;  // past the matrix: re-read, store nothing
    tr[t] = TileRows{a.w[sg] + (size_t)ltc * 16 * a.row_bytes, a.seg_rows[sg] - ltc * 16, (u32)a.row_bytes};
  }

  // activation staging: fragment f = b * 8 + j (1 KB) of stage sb is tile (mt * MB + b),
  // slice 8 sb + j; wave w loads fragments w, w + 8, ...
  const int tile_kb = a.nsb * 8;  // KB per activation tile (K / 32 fragments of 1 KB)
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)a.xpack + (size_t)mt * MB * tile_kb * 1024), 0, MB * tile_kb * 1024, kBufDword3);
  Q4Lane l4[NT];
  Q6Lane l6[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if constexpr (WT == 12)
      l4[t] = q4_lane(tr[t], lane);
    else
      l6[t] = q6_lane(tr[t], lane);
  }
  auto issue = [&](int sb) {
    lds_u8* as = abuf + (sb & 1) * (MB * 8 * 1024);
#pragma unroll
    for (int f = wave; f < MB * 8; f += kMmWaves) {
      const int b = f >> 3, j = f & 7;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lptr_t)(as + f * 1024), 16,
                                               (u32)((b * tile_kb + sb * 8 + j) * 1024 + lane * 16), 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      lds_u8* slot = ring + ((sb & 1) * NT + t) * kW;
      if constexpr (WT == 12)
        q4_issue(tr[t], l4[t], sb, slot);
      else
        q6_issue<ALIGNED>(tr[t], l6[t], sb, slot);
    }
  };

  float acc[NT][BT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < BT; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][b][e] = 0.f;

  issue(sb_lo);
  for (int sb = sb_lo; sb < sb_hi; ++sb) {
    // only stage sb's loads are outstanding: once every wave has seen its own land, the
    // stage is complete, and every wave is done with stage sb - 1, whose slots the next
    // issue reuses
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (sb + 1 < sb_hi) issue(sb + 1);
    __builtin_amdgcn_sched_barrier(0);
    lds_u8* slots[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) slots[t] = ring + ((sb & 1) * NT + t) * kW;
    const lds_u8* as = abuf + (sb & 1) * (MB * 8 * 1024);
    if constexpr (WT == 12) {
      q4_step_mm<BT>(as, slots, lane, acc);
    } else {
      u32 s16[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        s16[t] = addr::q6_s16((u32)(uintptr_t)(tr[t].base + (size_t)sb * kQ6KBytes) + tr[t].off(n));
      q6_step_mm<BT>(as, slots, s16, lane, acc);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // epilogue: lane (n, g) holds rows 8 b' + 2 g and 8 b' + 2 g + 1 (b' the activation
  // tile) of column n of each of its tiles
  const int rows0 = a.seg_rows[a.epi == kEpiSwiGLU ? 0 : seg];
  const int col0 = a.epi == kEpiSwiGLU ? 0 : a.seg_col_off[seg];
  if (a.part) {  // split K: raw partial sums, finished by gemm_mm_finish_kernel
#pragma unroll
    for (int b = 0; b < BT; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * (mt * MB + b) + 2 * g + h;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int c = lt[t] * 16 + n;
          if (row < a.B && c < rows0)
            a.part[((size_t)ks * a.B + row) * a.ldp + (col0 - a.pcol0) + c] = acc[t][b][2 * h] + acc[t][b][2 * h + 1];
        }
      }
    return;
  }
#pragma unroll
  for (int b = 0; b < BT; ++b) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * (mt * MB + b) + 2 * g + h;
      const bool row_ok = row < a.B;
      float rs = 1.0f;
      if (a.ss && row_ok) {
        double ssv = 0.0;
        for (int s = 0; s < a.ss_slots; ++s) ssv += a.ss[s * a.B + row];
        rs = 1.0f / sqrtf((float)ssv * a.inv_k + a.eps);
      }
      if (a.epi == kEpiSwiGLU) {
        const int col = lt[0] * 16 + n;
        if (row_ok && col < rows0) {
          const float gv = rs * (acc[0][b][2 * h] + acc[0][b][2 * h + 1]);
          const float uv = rs * (acc[1][b][2 * h] + acc[1][b][2 * h + 1]);
          actpack_put(a.pack_out, a.pack_kind, a.pack_nslices, row, col, gv / (1.0f + expf(-gv)) * uv);
        }
      } else if (a.epi == kEpiStore) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int c = lt[t] * 16 + n;
          if (row_ok && c < rows0) a.y[(size_t)row * a.ldy + col0 + c] = rs * (acc[t][b][2 * h] + acc[t][b][2 * h + 1]);
        }
      } else {
        float sq = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int c = lt[t] * 16 + n;
          if (row_ok && c < rows0) {
            float* yp = a.y + (size_t)row * a.ldy + col0 + c;
            const float xn = *yp + rs * (acc[t][b][2 * h] + acc[t][b][2 * h + 1]);
            *yp = xn;
            const float pv = xn * (a.gain ? a.gain[col0 + c] : 1.f);
            if (a.pack_out) actpack_put(a.pack_out, a.pack_kind, a.pack_nslices, row, col0 + c, pv);
            if (a.pack_out2) actpack_put(a.pack_out2, a.pack_kind2, a.pack_nslices2, row, col0 + c, pv);
            sq = __builtin_fmaf(xn, xn, sq);
          }
        }
        // the row's sum over the wave's 32 columns: lanes with the same g differ in n
#pragma unroll
        for (int o = 1; o <= 8; o <<= 1) sq += __shfl_xor(sq, o, 64);
        if (n == 0 && row_ok && a.ss_out)
          atomicAdd(a.ss_out + (size_t)(bid % a.ss_slots) * a.B + row, (double)sq);
      }
    }
  }
}

// Second pass of a K-split many-row launch: the sum of the partial sums, then the store
// or residual epilogue.  Grid (ceil(ldp / 256), B), 256 threads: thread = one column.
__global__ __launch_bounds__(256) void gemm_mm_finish_kernel(GemmArgs a, int nsplit) {
  __shared__ float red[4];
  const int row = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  const bool live = c < a.ldp;
  float v = 0.f;
  if (live)
    for (int s = 0; s < nsplit; ++s) v += a.part[((size_t)s * a.B + row) * a.ldp + c];
  float rs = 1.0f;
  if (a.ss) {
    double ssv = 0.0;
    for (int s = 0; s < a.ss_slots; ++s) ssv += a.ss[s * a.B + row];
    rs = 1.0f / sqrtf((float)ssv * a.inv_k + a.eps);
  }
  const int col = a.pcol0 + c;
  if (a.epi == kEpiStore) {
    if (live) a.y[(size_t)row * a.ldy + col] = rs * v;
    return;
  }
  float sq = 0.f;
  if (live) {
    float* yp = a.y + (size_t)row * a.ldy + col;
    const float xn = *yp + rs * v;
    *yp = xn;
    const float pv = xn * (a.gain ? a.gain[col] : 1.f);
    if (a.pack_out) actpack_put(a.pack_out, a.pack_kind, a.pack_nslices, row, col, pv);
    if (a.pack_out2) actpack_put(a.pack_out2, a.pack_kind2, a.pack_nslices2, row, col, pv);
    sq = xn * xn;
  }
  sq = wave_sum(sq);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sq;
  __syncthreads();
  if (threadIdx.x == 0 && a.ss_out)
    atomicAdd(a.ss_out + (size_t)(blockIdx.x % a.ss_slots) * a.B + row, (double)(red[0] + red[1] + red[2] + red[3]));
}

// ---------------------------------------------------------------------------------
// plan and launch

// Kernel variants by (NT, BTN): those whose registers fit four waves per SIMD (one tile
// with up to four batch tiles, two tiles with up to two) take up to 16 waves, the
// others up to 4.
struct GemmVariant {
  const void* fn = nullptr;
  int maxt = 0;
  int waves_per_cu = 0;  // resident waves per CU that the kernel's registers allow
};

// Workgroup size of a variant: 1024 threads where the kernel fits 128 VGPRs without
// spilling (Q5_K's NT 2 x BTN 2 does not), else 256.
constexpr int variant_maxt(int wt, int nt, int btn) {
  return (nt == 1 && btn <= 4) || (nt == 2 && btn == 2 && wt != 13) ? 1024 : 256;
}

template <int WT, bool AL>
const void* variant_fn(int nt, int btn) {
  switch (nt * 100 + btn) {
    case 101: return (const void*)gemm_kernel<WT, 1, 1, variant_maxt(WT, 1, 1), AL>;
    case 102: return (const void*)gemm_kernel<WT, 1, 2, variant_maxt(WT, 1, 2), AL>;
    case 104: return (const void*)gemm_kernel<WT, 1, 4, variant_maxt(WT, 1, 4), AL>;
    case 108: return (const void*)gemm_kernel<WT, 1, 8, variant_maxt(WT, 1, 8), AL>;
    case 201: return (const void*)gemm_kernel<WT, 2, 1, variant_maxt(WT, 2, 1), AL>;
    case 202: return (const void*)gemm_kernel<WT, 2, 2, variant_maxt(WT, 2, 2), AL>;
    case 204: return (const void*)gemm_kernel<WT, 2, 4, variant_maxt(WT, 2, 4), AL>;
    case 208: return (const void*)gemm_kernel<WT, 2, 8, variant_maxt(WT, 2, 8), AL>;
    default: return nullptr;
  }
}

struct VariantTable {
  GemmVariant v[5][2][4];  // (Q4_K, Q6_K aligned, Q6_K unaligned, Q5_K, Q8_0) x NT x log2 BTN
  int cus = 256;
  VariantTable() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                hipSuccess && n > 0)
      cus = n;
    for (int ty = 0; ty < 5; ++ty)
      for (int nt = 1; nt <= 2; ++nt)
        for (int lb = 0; lb < 4; ++lb) {
          const int btn = 1 << lb;
          GemmVariant& g = v[ty][nt - 1][lb];
          g.fn = ty == 0   ? variant_fn<12, true>(nt, btn)
                 : ty == 1 ? variant_fn<14, true>(nt, btn)
                 : ty == 2 ? variant_fn<14, false>(nt, btn)
                 : ty == 3 ? variant_fn<13, true>(nt, btn)
                           : variant_fn<8, true>(nt, btn);
          g.maxt = variant_maxt(ty == 0 ? 12 : ty == 3 ? 13 : ty == 4 ? 8 : 14, nt, btn);
          // registers per lane -> waves per SIMD (512 VGPRs, granule 8); without a device
          // to ask, assume the 128 that a 1024-thread workgroup requires
          int regs = 128;
          hipFuncAttributes at{};
          if (hipFuncGetAttributes(&at, g.fn) == hipSuccess && at.numRegs > 0) regs = at.numRegs;
          const int per_simd = 512 / ((regs + 7) & ~7);
          g.waves_per_cu = 4 * (per_simd < 8 ? per_simd : 8);
          (void)hipFuncSetAttribute(g.fn, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
        }
    (void)hipGetLastError();  // a missing device leaves an error behind; it is not this call's
  }
};

const VariantTable& variants() {
  static const VariantTable t;  // built once, thread-safe
  return t;
}

int log2_btn(int btn) { return btn == 1 ? 0 : btn == 2 ? 1 : btn == 4 ? 2 : 3; }

const GemmVariant& gemm_variant(int wtype, bool aligned, int nt, int btn) {
  const int ty = wtype == 12 ? 0 : wtype == 13 ? 3 : wtype == 8 ? 4 : aligned ? 1 : 2;
  return variants().v[ty][nt - 1][log2_btn(btn)];
}

// Q6_K rows are a multiple of 16 bytes when K is a multiple of 8 super-blocks.
bool q6_aligned(int K) { return (K / kQK) % 8 == 0; }

GemmPlan plan_gemm(int wtype, int total_tiles, int K, int B, int nt) {
  GemmPlan pl{};
  pl.nt = nt;
  pl.btn = actpack_tiles(B);
  pl.tiles = total_tiles;
  const int nsb = K / kQK;
  const GemmVariant& v = gemm_variant(wtype, wtype != 14 || q6_aligned(K), nt, pl.btn);
  pl.maxt = v.maxt;
  const int max_waves = min(pl.maxt / 64, nsb);
  // LDS: staging rings (waves * NT * kRing slots) and the reduction (waves * NT * BTN *
  // 512 B, then the RMSNorm partial sums) share one allocation of at most kGemmLds
  const int stage = stage_bytes(wtype);
  auto lds_need = [&](int w) {
    return max(w * pl.nt * kRing * stage, w * pl.nt * pl.btn * 512 + kSsCap * (int)sizeof(double));
  };
  auto waves_for = [&](int w) {  // waves actually used when splitting nsb over w
    const int spw = (nsb + w - 1) / w;
    return (nsb + spw - 1) / spw;
  };
  // The most waves per workgroup that still lets every workgroup be resident at once
  // (one round: no tail of workgroups that start late); when no choice does, about
  // 4096 waves in flight.
  int pick = 0;
  for (int w = max_waves; w >= 1 && !pick; --w) {
    const int wu = waves_for(w);
    if (lds_need(wu) > kGemmLds) continue;
    const int per_cu = min(v.waves_per_cu / wu, kGemmLds / lds_need(wu));
    if ((long long)per_cu * variants().cus >= total_tiles) pick = wu;
  }
  if (!pick) {
    int want = (4096 + total_tiles - 1) / total_tiles;
    if (want > max_waves) want = max_waves;
    while (want > 1 && lds_need(waves_for(want)) > kGemmLds) --want;
    pick = want < 1 ? 1 : want;
  }
  pl.sb_per_wave = (nsb + pick - 1) / pick;
  pl.waves = (nsb + pl.sb_per_wave - 1) / pl.sb_per_wave;
  pl.lds = (size_t)lds_need(pl.waves);
  return pl;
}

hipError_t launch_gemm(int wtype, const GemmPlan& pl, const GemmArgs& a, hipStream_t st) {
  if (pl.tiles <= 0) return hipSuccess;
  const bool aligned = wtype != 14 || a.row_bytes % 16 == 0;
  const GemmVariant& v = gemm_variant(wtype, aligned, pl.nt, pl.btn);
  if (!v.fn || v.maxt != pl.maxt || pl.waves * 64 > pl.maxt) return hipErrorInvalidValue;
  const dim3 grid(pl.tiles), block(pl.waves * 64);
  const size_t lds = pl.lds;
  const void* fn = v.fn;
  GemmArgs args = a;
  void* kargs[] = {&args};
  const hipError_t e = launch_fn(fn, grid, block, lds, st, kargs);
  return e != hipSuccess ? e : hipGetLastError();
}

// ---------------------------------------------------------------------------------
// tile-loop plan and launch

// ring depth by (type, NT): the deepest that fits kGemmLds with 8 waves
// ring depth by (type, NT, batch tiles): the deepest that fits kGemmLds with 8 waves
constexpr int tl_ring(int wtype, int nt, int btn) {
  return wtype == 12 ? (nt == 1 ? 4 : btn == 1 ? 3 : 2) : (nt == 1 ? 4 : 2);
}

// One or two activation tiles (at most 16 rows).  The epilogue gives each of a group's
// 128 outputs per batch tile (a tile, or a gate/up pair, of 8 rows) a thread of its own,
// so the workgroup needs two waves per batch tile: K of at least three super-blocks (one
// wave per two) for 8 rows, seven for 16.
bool use_tile_loop(int wtype, int groups, int K, int B) {
  const int nsb = K / kQK;
  return (wtype == 12 || wtype == 14) && B <= 16 && K % kQK == 0 && nsb >= (B <= 8 ? 3 : 7) && nsb <= 16 &&
         groups >= 2 * variants().cus;
}

// Whole-tile staging (Q4_K, one activation tile) from one group per CU.
bool use_tile_loop_whole(int wtype, int groups, int K, int B) {
  const int nsb = K / kQK;
  return wtype == 12 && B <= 8 && K % kQK == 0 && nsb >= 3 && nsb <= 16 && groups >= variants().cus;
}

TlPlan plan_gemm_tl(int wtype, int nt, int groups, int K, int B) {
  TlPlan pl{};
  const int nsb = K / kQK;
  const int btn = tl_btn(B);
  pl.waves = (nsb + 1) / 2;
  pl.ring = tl_ring(wtype, nt, btn);
  const int stage = wtype == 12 ? kQ4Stage : kQ6Stage;
  pl.whole = wtype == 12 && btn == 1 && nsb >= 3 && nsb <= 16;  // whole-tile staging (gemm_tlw_kernel)
  if (pl.whole) pl.waves = tlw_waves(nsb);
  pl.lds = pl.whole ? tlw_lds_bytes(nsb)
                    : (size_t)pl.waves * pl.ring * nt * stage + (size_t)2 * pl.waves * nt * btn * 128 * sizeof(float);
  const int per_cu = max(1, kGemmLds / (int)pl.lds);
  int wgs = min(groups, variants().cus * per_cu);
  pl.groups_per_wg = (groups + wgs - 1) / wgs;
  // whole-tile staging splits the groups over every resident workgroup in proportion
  pl.grid = pl.whole ? wgs : (groups + pl.groups_per_wg - 1) / pl.groups_per_wg;
  return pl;
}

template <int WT, bool AL>
const void* tl_fn(int nt, int btn) {
  if (btn == 1) {
    if (nt == 1) return (const void*)gemm_tl_kernel<WT, 1, AL, tl_ring(WT, 1, 1), 1>;
    return (const void*)gemm_tl_kernel<WT, 2, AL, tl_ring(WT, 2, 1), 1>;
  }
  if (nt == 1) return (const void*)gemm_tl_kernel<WT, 1, AL, tl_ring(WT, 1, 2), 2>;
  return (const void*)gemm_tl_kernel<WT, 2, AL, tl_ring(WT, 2, 2), 2>;
}

hipError_t launch_gemm_tl(int wtype, int nt, const TlPlan& pl, GemmArgs a, hipStream_t st) {
  if (pl.grid <= 0) return hipSuccess;
  const int btn = tl_btn(a.B);
  if ((nt != 1 && nt != 2) || pl.waves < 2 || pl.waves > (pl.whole ? 16 : 8) || pl.lds > (size_t)kGemmLds || a.B > 16 ||
      (a.ss && a.ss_slots != 16) || (a.epi == kEpiSwiGLU ? 1 : nt) * 128 * btn > pl.waves * 64)
    return hipErrorInvalidValue;
  const bool aligned = wtype == 12 || a.row_bytes % 16 == 0;
  if (!pl.whole && a.epi == kEpiResidual) return hipErrorInvalidValue;  // only the whole-tile kernel updates
  if (pl.whole && (wtype != 12 || btn != 1 || (nt == 2) != (a.epi == kEpiSwiGLU) || a.nsb > 16 ||
                   a.nsb < 2 || pl.waves != tlw_waves(a.nsb) || addr::kWtInstr * pl.waves < addr::wt_instrs(a.nsb) ||
                   pl.lds != tlw_lds_bytes(a.nsb)))
    return hipErrorInvalidValue;
  const void* fn = pl.whole      ? (nt == 2                  ? (const void*)gemm_tlw_kernel<kTlwPair>
                                    : a.epi == kEpiResidual ? (const void*)gemm_tlw_kernel<kTlwResidual>
                                                            : (const void*)gemm_tlw_kernel<kTlwStore>)
                   : wtype == 12 ? tl_fn<12, true>(nt, btn)
                   : aligned     ? tl_fn<14, true>(nt, btn)
                                 : tl_fn<14, false>(nt, btn);
  static const bool lds_set = [] {
    for (int b = 1; b <= 2; ++b)
      for (int t = 1; t <= 2; ++t) {
        const void* all[] = {tl_fn<12, true>(t, b), tl_fn<14, true>(t, b), tl_fn<14, false>(t, b)};
        for (const void* f : all) (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
      }
    for (const void* f : {(const void*)gemm_tlw_kernel<kTlwStore>, (const void*)gemm_tlw_kernel<kTlwResidual>,
                          (const void*)gemm_tlw_kernel<kTlwPair>})
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    (void)hipGetLastError();
    return true;
  }();
  (void)lds_set;
  a.sb_per_wave = 2;
  a.tl_groups_per_wg = pl.groups_per_wg;
  void* kargs[] = {&a};
  const hipError_t e = launch_fn(fn, dim3(pl.grid), dim3(pl.waves * 64), pl.lds, st, kargs);
  return e != hipSuccess ? e : hipGetLastError();
}

bool mm_required(int B) { return B > kSkinnyRows; }
bool use_mm(int wtype, int B) { return mm_supported(wtype) && B > kMmMinRows; }
// Wide plain-store GEMMs (the output head) from 9 rows: the many-row kernel streams each
// weight tile once per 16 (Q6_K) or 32 (Q4_K) rows instead of re-reading every row's
// activations per tile
bool use_mm_store(int wtype, int B, int cols) {
  return use_mm(wtype, B) ||
         (mm_supported(wtype) && cols > kMmSplitMaxCols && B > 8 && actpack_tiles(B) % mm_mb(wtype) == 0);
}
bool mm_supported(int wtype) { return wtype == 12 || wtype == 14; }
int mm_group_tiles(bool swiglu) { return swiglu ? kMmWaves : kMmWaves * kMmNT; }

// Few workgroups (narrow matrices: QKV, Wo, down at a few hundred rows): split K so the
// grid fills the CUs more than once; a second pass sums the ranges.
// One workgroup per CU at a time (its LDS), so a launch takes ceil(workgroups / CUs)
// rounds; n ranges make rounds of 1/n the work.  The split that minimizes rounds / n
// wins, a split paying 5 % for its finishing pass.
int mm_split(int wtype, int B, int cols, int nsb, int groups, int epi, size_t part_cap) {
  const int wgs = (actpack_tiles(B) / mm_mb(wtype)) * groups;
  if (epi == kEpiSwiGLU || cols > kMmSplitMaxCols) return 1;
  const int cus = variants().cus;
  int best = 1;
  double best_t = (double)((wgs + cus - 1) / cus);
  for (int n = 2; n <= kMmMaxSplit && n <= nsb / 2; ++n) {
    if ((size_t)n * B * cols > part_cap) break;
    const double t = (double)((wgs * n + cus - 1) / cus) / n + 0.05;
    if (t < best_t) {
      best_t = t;
      best = n;
    }
  }
  return best;
}

hipError_t launch_gemm_mm(int wtype, int groups, GemmArgs a, hipStream_t st) {
  if (groups <= 0) return hipSuccess;
  if (!mm_supported(wtype) || a.B <= 0 || a.ss_slots < 1) return hipErrorInvalidValue;
  const int mtiles = actpack_tiles(a.B) / mm_mb(wtype);
  if (mtiles * mm_mb(wtype) != actpack_tiles(a.B)) return hipErrorInvalidValue;
  const bool aligned = wtype == 12 || a.row_bytes % 16 == 0;
  const void* fn = wtype == 12 ? (const void*)gemm_mm_kernel<12, true>
                               : aligned ? (const void*)gemm_mm_kernel<14, true> : (const void*)gemm_mm_kernel<14, false>;
  static const bool lds_set = [] {
    const void* all[] = {(const void*)gemm_mm_kernel<12, true>, (const void*)gemm_mm_kernel<14, true>,
                         (const void*)gemm_mm_kernel<14, false>};
    for (const void* f : all) (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    (void)hipGetLastError();
    return true;
  }();
  (void)lds_set;
  a.mm_mtiles = mtiles;
  a.mm_groups = groups;
  const int nsplit = a.part ? mm_split(wtype, a.B, a.ldp, a.nsb, groups, a.epi, a.part_cap) : 1;
  if (nsplit <= 1) a.part = nullptr;
  void* kargs[] = {&a};
  hipError_t e = launch_fn(fn, dim3(mtiles * groups * nsplit), dim3(kMmWaves * 64), mm_lds(wtype), st, kargs);
  if (e != hipSuccess) return e;
  if ((e = hipGetLastError()) != hipSuccess || nsplit <= 1) return e;
  launch_kernel(gemm_mm_finish_kernel, dim3((a.ldp + 255) / 256, a.B), dim3(256), 0, st, a, nsplit);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// row-block plan and launch

// Which GEMMs take it: Q4_K gate/up pairs, 17 to 32 rows, K split into ranges of 4 to 8
// super-blocks.
bool use_rb(int wtype, int K, int B) {
  return wtype == 12 && B > 16 && B <= 32 && K % kQK == 0 && rb_ranges(K / kQK) > 0;
}
int rb_slots(int nsb) {
  const int nkr = rb_ranges(nsb);
  return nkr > 0 ? variants().cus / nkr : 0;
}
int rb_grid(int nsb) { return rb_slots(nsb) * rb_ranges(nsb); }
size_t rb_part_floats(int groups, int K, bool pair) {
  const int nkr = rb_ranges(K / kQK);
  return nkr > 1 ? (size_t)nkr * groups * (pair ? 2 : 1) * kRbElems : 0;
}
// groups of the workgroup with the most, and the dynamic LDS of a launch
int rb_ngm(int groups, int nsb) {
  const int per = rb_slots(nsb);
  return per > 0 ? (groups + per - 1) / per : 0;
}
size_t rb_lds(int groups, int nsb, bool pair) {
  const int nkr = rb_ranges(nsb);
  return rb_lds_bytes(nsb / nkr, nkr > 1 ? rb_ngm(groups, nsb) : 0, pair ? 2 : 1);
}
bool rb_fits(int groups, int K, bool pair, size_t part_cap, int cnt_n) {
  const int nsb = K / kQK, nkr = rb_ranges(nsb);
  if (nkr < 1) return false;
  const int ngm = rb_ngm(groups, nsb);
  if (ngm < 1 || ngm > kRbMaxGroups || rb_lds(groups, nsb, pair) + kRbStaticLds > (size_t)kGemmLds) return false;
  return nkr == 1 || (rb_part_floats(groups, K, pair) <= part_cap && groups <= cnt_n);
}

hipError_t launch_gemm_rb(int groups, GemmArgs a, hipStream_t st) {
  if (groups <= 0) return hipSuccess;
  const int nkr = rb_ranges(a.nsb);
  const bool pair = true;
  if (nkr < 1 || a.B > 32 || a.B < 1 || a.epi != kEpiSwiGLU || a.nseg != 2 || a.seg_rows[0] > groups * 16 ||
      (a.ss && (a.ss_slots * a.B > kSsCap || a.ss_slots < 1)) ||
      !rb_fits(groups, a.nsb * kQK, pair, a.part_cap, a.rb_cnt_n) || (nkr > 1 && (!a.part || !a.rb_cnt)))
    return hipErrorInvalidValue;
  const int W = a.nsb / nkr;
  if (W < 4 || W > kRbMaxWaves || addr::kWtInstr * W < addr::wt_instrs(W)) return hipErrorInvalidValue;
  static const bool lds_set = [] {
    (void)hipFuncSetAttribute((const void*)gemm_rb_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              kGemmLds - (int)kRbStaticLds);
    (void)hipGetLastError();
    return true;
  }();
  (void)lds_set;
  a.tl_groups = groups;
  const void* fn = (const void*)gemm_rb_kernel;
  void* kargs[] = {&a};
  const hipError_t e =
      launch_fn(fn, dim3(rb_grid(a.nsb)), dim3(W * 64), rb_lds(groups, a.nsb, pair), st, kargs);
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace gr
