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
GR_DEV u32x4 q4_expand(u32x2 q, bool high) {
  const u32 M = 0x43004300u, NIB = 0x000F000Fu;
  u32 w0 = high ? (q.x >> 4) : q.x;
  u32 w1 = high ? (q.y >> 4) : q.y;
  u32x4 r;
  r.x = (w0 & NIB) | M;
  r.y = ((w0 >> 8) & NIB) | M;
  r.z = (w1 & NIB) | M;
  r.w = ((w1 >> 8) & NIB) | M;
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
  r.hdr = __builtin_nontemporal_load((const u32x4*)blk);
#pragma unroll
  for (int c = 0; c < 4; ++c) r.qs[c] = __builtin_nontemporal_load((const u32x2*)(blk + 16 + 32 * c + 8 * kg));
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

GR_DEV void q6_load(Q6Regs& r, const uint8_t* blk, int kg) {
#pragma unroll
  for (int hu = 0; hu < 4; ++hu) {
    const int h = hu >> 1, u = hu & 1;
    r.part[hu].a = load_u32_a2(blk + 64 * h + 16 * u + 4 * kg);
    r.part[hu].b = load_u32_a2(blk + 64 * h + 32 + 16 * u + 4 * kg);
    r.part[hu].q = load_u32_a2(blk + 128 + 32 * h + 16 * u + 4 * kg);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) r.sc[i] = load_u32_a2(blk + 192 + 4 * i);
  r.d = __builtin_nontemporal_load((const u16*)(blk + 208));
}

// 6-bit quants of sub-block (h, 2r+u) as four bytes, then as the bf16 B operand.
GR_DEV u32x2 q6_expand(const Q6Part& pt, int r) {
  u32 v;
  if (r == 0)
    v = (pt.a & 0x0F0F0F0Fu) | ((pt.q << 4) & 0x30303030u);
  else if (r == 1)
    v = (pt.b & 0x0F0F0F0Fu) | ((pt.q << 2) & 0x30303030u);
  else if (r == 2)
    v = ((pt.a >> 4) & 0x0F0F0F0Fu) | (pt.q & 0x30303030u);
  else
    v = ((pt.b >> 4) & 0x0F0F0F0Fu) | ((pt.q >> 2) & 0x30303030u);
  const u32 M = 0x43004300u;
  u32x2 o;
  o.x = (v & 0x00FF00FFu) | M;
  o.y = ((v >> 8) & 0x00FF00FFu) | M;
  return o;
}

}  // namespace gr
