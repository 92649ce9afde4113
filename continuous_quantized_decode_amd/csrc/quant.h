// quant.h -- register-level decoders of GGUF Q4_K / Q6_K super-blocks, shared by the
// fused-dequant GEMM and the bit-exactness dequant exports (so both run the same
// unpacking code).  Block layouts: the public GGUF formats (Leone, "What ships":
// Q4_K and Q6_K weights).
//
// Q4_K (144 B): d, dmin (fp16), 12 bytes of packed 6-bit scales/mins, 128 bytes of
// nibbles; byte 32c+l holds weight 64c+l (low nibble) and 64c+32+l (high nibble);
// w = d*sc[j]*q - dmin*m[j] for sub-block j (32 weights).
// Q6_K (210 B): ql[128], qh[64], int8 scales[16], d (fp16) last; weight
// 128h+l+32r (l < 32) takes its low 4 bits from ql[64h + l + 32(r&1)] (nibble r>>1)
// and its top 2 bits from bits 2r..2r+1 of qh[32h+l]; w = d*scale[i/16]*(q-32).
#pragma once

#include "gr_common.h"

namespace gr {

// ---------------------------------------------------------------------------------
// Q4_K

// Expand 8 bytes of Q4_K quants (two dwords) into the bf16 B operand of one
// sub-block: `high` selects the high nibbles (odd sub-block of the chunk).
// Keeps a constant in a VGPR, so that (x & mask) | c compiles to one three-input
// v_and_or_b32 (gfx9 VOP3 takes no literal and one scalar operand).
GR_DEV u32 vconst(u32 c) {
  asm volatile("" : "+v"(c));
  return c;
}

GR_DEV u32x4 q4_expand(u32x2 q, bool high, u32 M = 0x43004300u) {
  const u32 NIB = 0x000F000Fu;
  u32 w0 = high ? (q.x >> 4) : q.x;
  u32 w1 = high ? (q.y >> 4) : q.y;
  u32x4 r;
  r.x = (w0 & NIB) | M;
  r.y = ((w0 >> 8) & NIB) | M;
  r.z = (w1 & NIB) | M;
  r.w = ((w1 >> 8) & NIB) | M;
  return r;
}

// Q5_K: the Q4_K expansion with each weight's fifth bit (bit j of its high-bit byte for
// sub-block j) at value 16; 128 + q (q < 32) is an exact bf16.
GR_DEV u32x4 q5_expand(u32x2 q, u32x2 h, int j, u32 M = 0x43004300u) {
  const u32 NIB = 0x000F000Fu, B1 = 0x00010001u;
  const bool high = (j & 1) != 0;
  const u32 w0 = high ? (q.x >> 4) : q.x, w1 = high ? (q.y >> 4) : q.y;
  const u32 h0 = h.x >> j, h1 = h.y >> j;
  u32x4 r;
  r.x = (w0 & NIB) | ((h0 & B1) << 4) | M;
  r.y = ((w0 >> 8) & NIB) | (((h0 >> 8) & B1) << 4) | M;
  r.z = (w1 & NIB) | ((h1 & B1) << 4) | M;
  r.w = ((w1 >> 8) & NIB) | (((h1 >> 8) & B1) << 4) | M;
  return r;
}

// Scales of one Q4_K super-block header: sd[j] = d*sc[j] and dm[j] = dmin*m[j], both
// exact in fp32 (11-bit fp16 mantissa times a 6-bit integer).
GR_DEV void q4_scales(u32x4 hdr, float* sd, float* dm) {
  const float d = h2f((u16)(hdr.x & 0xFFFF)), dmin = h2f((u16)(hdr.x >> 16));
  const u32 s0 = hdr.y, s1 = hdr.z, s2 = hdr.w;
  const u32 sc_lo = s0 & 0x3F3F3F3Fu, m_lo = s1 & 0x3F3F3F3Fu;
  const u32 sc_hi = (s2 & 0x0F0F0F0Fu) | ((s0 >> 2) & 0x30303030u);
  const u32 m_hi = ((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sd[j] = d * (float)((sc_lo >> (8 * j)) & 0xFF);
    sd[j + 4] = d * (float)((sc_hi >> (8 * j)) & 0xFF);
    dm[j] = dmin * (float)((m_lo >> (8 * j)) & 0xFF);
    dm[j + 4] = dmin * (float)((m_hi >> (8 * j)) & 0xFF);
  }
}

struct Q4Regs {
  u32x4 hdr;
  u32x2 qs[4];
};

GR_DEV void q4_load(Q4Regs& r, const uint8_t* blk, int kg) {
  r.hdr = gr_ld((const u32x4*)blk);
#pragma unroll
  for (int c = 0; c < 4; ++c) r.qs[c] = gr_ld((const u32x2*)(blk + 16 + 32 * c + 8 * kg));
}

// ---------------------------------------------------------------------------------
// Q6_K

// One Q6_K half-chunk for lane group kg: dwords of ql (low nibbles of weights l and
// l+64), ql+32 (l+32, l+96) and qh (their top two bits), l = 16u + 4kg .. +3.
struct Q6Part {
  u32 a, b, q;
};
struct Q6Regs {
  Q6Part part[4];  // (h, u) = (0,0) (0,1) (1,0) (1,1)
  u32 sc[4];       // 16 int8 scales
  u16 d;
};

// 4 bytes at a 2-byte aligned address: one 8-byte load at the enclosing 4-byte
// aligned address, then a byte funnel shift.  The load covers [p-2, p+6) or [p, p+8),
// which must lie inside the buffer (callers keep at least 4 bytes after p + 4).
typedef u32 u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
GR_DEV u32 ld4_a2(const uint8_t* p) {
  const uintptr_t a = (uintptr_t)p;
  const u32x2_a4 w = gr_ld((const u32x2_a4*)(a & ~(uintptr_t)3));
  return __builtin_amdgcn_alignbyte(w.y, w.x, (u32)(a & 3));
}

GR_DEV void q6_load(Q6Regs& r, const uint8_t* blk, int kg) {
#pragma unroll
  for (int hu = 0; hu < 4; ++hu) {
    const int h = hu >> 1, u = hu & 1;
    r.part[hu].a = ld4_a2(blk + 64 * h + 16 * u + 4 * kg);
    r.part[hu].b = ld4_a2(blk + 64 * h + 32 + 16 * u + 4 * kg);
    r.part[hu].q = ld4_a2(blk + 128 + 32 * h + 16 * u + 4 * kg);
  }
  // scales [192, 208): aligned dwords covering them, funnel-shifted when the block is
  // 2 mod 4; the fifth dword is read only when needed (else the fourth again), so
  // the reads stay inside the block, and there is no branch.
  const uintptr_t a = (uintptr_t)(blk + 192);
  const u32 sh = (u32)(a & 3);
  const u32* base = (const u32*)(a & ~(uintptr_t)3);
  const u32 w0 = gr_ld(base), w1 = gr_ld(base + 1);
  const u32 w2 = gr_ld(base + 2), w3 = gr_ld(base + 3);
  const u32 w4 = gr_ld(base + (sh ? 4 : 3));
  r.sc[0] = __builtin_amdgcn_alignbyte(w1, w0, sh);
  r.sc[1] = __builtin_amdgcn_alignbyte(w2, w1, sh);
  r.sc[2] = __builtin_amdgcn_alignbyte(w3, w2, sh);
  r.sc[3] = __builtin_amdgcn_alignbyte(w4, w3, sh);
  r.d = gr_ld((const u16*)(blk + 208));
}

// Four bytes b0..b3 of v (each < 128) as the bf16 pairs (128 + b0, 128 + b2) and
// (128 + b1, 128 + b3): one byte permute each, the exponent byte 0x43 taken from E
// (0x43434343; v_perm_b32 selectors 0-3 pick bytes of its second operand, 4-7 of
// its first).
GR_DEV u32x2 bytes_to_bf16(u32 v, u32 E) {
  u32x2 o;
  o.x = __builtin_amdgcn_perm(E, v, 0x04020400u);
  o.y = __builtin_amdgcn_perm(E, v, 0x04030401u);
  return o;
}

// 6-bit quants of sub-block (h, 2r+u) as four bytes, then as the bf16 B operand.
GR_DEV u32x2 q6_expand(const Q6Part& pt, int r, u32 E = 0x43434343u) {
  u32 v;
  if (r == 0)
    v = (pt.a & 0x0F0F0F0Fu) | ((pt.q << 4) & 0x30303030u);
  else if (r == 1)
    v = (pt.b & 0x0F0F0F0Fu) | ((pt.q << 2) & 0x30303030u);
  else if (r == 2)
    v = ((pt.a >> 4) & 0x0F0F0F0Fu) | (pt.q & 0x30303030u);
  else
    v = ((pt.b >> 4) & 0x0F0F0F0Fu) | ((pt.q >> 2) & 0x30303030u);
  return bytes_to_bf16(v, E);
}

}  // namespace gr
