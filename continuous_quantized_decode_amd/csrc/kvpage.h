// kvpage.h -- register-level access to one 16-token page of one KV head, shared by
// the split attention kernel and the page-gather export.
//
// Pool layout: page p holds every KV head; head g's block starts at g*HB.  K heads
// are token-major [16][D], V heads dim-major [D][16]; q8_0 heads hold the 16*D int8
// codes in that order, then fp16 scales [16 tokens][D/32].
#pragma once

#include "gr_common.h"
#include "attn_internal.h"

namespace gr {

// ------------------------------------------------------------------ operand loads
// K tile for slice sigma (32 dims): lane (n = token, kg) needs K[n][32 sigma + 8kg .. +7].
// V tile for d-tile dt (16 dims): lane (n = dim, kg) needs V[4kg .. 4kg+3][16 dt + n].

template <int KVDT, int D>
struct PageRegs;

template <int D>
struct PageRegs<KV_F16_T, D> {
  u32x4 k[D / 32];
  u32x2 v[D / 16];
};
template <int D>
struct PageRegs<KV_F32_T, D> {
  u32x4 k[D / 32][2];  // 8 floats
  u32x4 v[D / 16];     // 4 floats
};
template <int D>
struct PageRegs<KV_Q8_T, D> {
  u32x2 k[D / 32];  // 8 codes
  u32 v[D / 16];    // 4 codes
  u32 ksc[D / 64];  // this lane's token: D/32 fp16 scales (K)
  u32 vsc[D / 64];  // same for V
};

template <int KVDT, int D>
GR_DEV void load_page(PageRegs<KVDT, D>& r, const uint8_t* kh, const uint8_t* vh, int lane) {
  const int n = lane & 15, kg = lane >> 4;
  if constexpr (KVDT == KV_F16_T) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) r.k[s] = gr_ld((const u32x4*)(kh + (n * D + 32 * s + 8 * kg) * 2));
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      r.v[t] = gr_ld((const u32x2*)(vh + ((16 * t + n) * kPage + 4 * kg) * 2));
  } else if constexpr (KVDT == KV_F32_T) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      r.k[s][0] = gr_ld((const u32x4*)(kh + (n * D + 32 * s + 8 * kg) * 4));
      r.k[s][1] = gr_ld((const u32x4*)(kh + (n * D + 32 * s + 8 * kg + 4) * 4));
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      r.v[t] = gr_ld((const u32x4*)(vh + ((16 * t + n) * kPage + 4 * kg) * 4));
  } else {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) r.k[s] = gr_ld((const u32x2*)(kh + n * D + 32 * s + 8 * kg));
#pragma unroll
    for (int t = 0; t < D / 16; ++t) r.v[t] = gr_ld((const u32*)(vh + (16 * t + n) * kPage + 4 * kg));
    // scales of token n: [16][D/32] fp16 after the 16*D codes
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      r.ksc[i] = gr_ld((const u32*)(kh + kPage * D + (n * (D / 32) + 2 * i) * 2));
      r.vsc[i] = gr_ld((const u32*)(vh + kPage * D + (n * (D / 32) + 2 * i) * 2));
    }
  }
}

// Replace the new token's slot (token `slot` of this page) with the stored values
// kept in LDS (same byte format as the pool).
template <int KVDT, int D>
GR_DEV void patch_page(PageRegs<KVDT, D>& r, const uint8_t* knew, const uint8_t* vnew, int slot, int lane) {
  const int n = lane & 15, kg = lane >> 4;
  if (n == slot) {
    if constexpr (KVDT == KV_F16_T) {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) r.k[s] = *(const u32x4*)(knew + (32 * s + 8 * kg) * 2);
    } else if constexpr (KVDT == KV_F32_T) {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        r.k[s][0] = *(const u32x4*)(knew + (32 * s + 8 * kg) * 4);
        r.k[s][1] = *(const u32x4*)(knew + (32 * s + 8 * kg + 4) * 4);
      }
    } else {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) r.k[s] = *(const u32x2*)(knew + 32 * s + 8 * kg);
#pragma unroll
      for (int i = 0; i < D / 64; ++i) {
        r.ksc[i] = *(const u32*)(knew + D + 4 * i);
        r.vsc[i] = *(const u32*)(vnew + D + 4 * i);
      }
    }
  }
  // V: lane (dim n, kg) holds tokens 4kg..4kg+3 of its dims; replace token `slot`.
  if (kg == (slot >> 2)) {
    const int e = slot & 3;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const int d = 16 * t + n;
      if constexpr (KVDT == KV_F16_T) {
        const u32 hv = ((const u16*)vnew)[d];
        u32 w = e < 2 ? r.v[t].x : r.v[t].y;
        w = (e & 1) ? ((w & 0x0000FFFFu) | (hv << 16)) : ((w & 0xFFFF0000u) | hv);
        if (e < 2)
          r.v[t].x = w;
        else
          r.v[t].y = w;
      } else if constexpr (KVDT == KV_F32_T) {
        const u32 fv = ((const u32*)vnew)[d];
        if (e == 0) r.v[t].x = fv;
        if (e == 1) r.v[t].y = fv;
        if (e == 2) r.v[t].z = fv;
        if (e == 3) r.v[t].w = fv;
      } else {
        const u32 cv = vnew[d];
        r.v[t] = (r.v[t] & ~(0xFFu << (8 * e))) | (cv << (8 * e));
      }
    }
  }
}

// Zero V elements of tokens >= valid (lane (dim, kg) holds tokens 4kg..4kg+3).
template <int KVDT, int D>
GR_DEV void mask_v_tail(PageRegs<KVDT, D>& r, int valid, int lane) {
  const int kg = lane >> 4;
  if constexpr (KVDT == KV_F16_T) {
    u32 m0 = 0, m1 = 0;
    if (4 * kg + 0 < valid) m0 |= 0x0000FFFFu;
    if (4 * kg + 1 < valid) m0 |= 0xFFFF0000u;
    if (4 * kg + 2 < valid) m1 |= 0x0000FFFFu;
    if (4 * kg + 3 < valid) m1 |= 0xFFFF0000u;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      r.v[t].x &= m0;
      r.v[t].y &= m1;
    }
  } else if constexpr (KVDT == KV_F32_T) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      if (4 * kg + 0 >= valid) r.v[t].x = 0;
      if (4 * kg + 1 >= valid) r.v[t].y = 0;
      if (4 * kg + 2 >= valid) r.v[t].z = 0;
      if (4 * kg + 3 >= valid) r.v[t].w = 0;
    }
  }
}

// int8 codes (4 per dword) -> exact f16 values; order (0,2,1,3).
GR_DEV u32x2 q8_to_f16x4(u32 w) {
  const u32 x = w ^ 0x80808080u;
  u32 a = (x & 0x00FF00FFu) | 0x64006400u;          // 1024 + 128 + c
  u32 b = ((x >> 8) & 0x00FF00FFu) | 0x64006400u;
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const h2 ha = __builtin_bit_cast(h2, a) - off;     // exact: small integers
  const h2 hb = __builtin_bit_cast(h2, b) - off;
  return u32x2{__builtin_bit_cast(u32, ha), __builtin_bit_cast(u32, hb)};
}

// f32 x4 -> f16 hi pair and lo pair (natural order)
GR_DEV void f32_to_f16hl(u32x4 f, u32x2& hi, u32x2& lo) {
  u16 h[4], l[4];
  const float v[4] = {u2f(f.x), u2f(f.y), u2f(f.z), u2f(f.w)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f2h(v[i]);
    l[i] = f2h(v[i] - h2f(h[i]));
  }
  hi = u32x2{(u32)h[0] | ((u32)h[1] << 16), (u32)h[2] | ((u32)h[3] << 16)};
  lo = u32x2{(u32)l[0] | ((u32)l[1] << 16), (u32)l[2] | ((u32)l[3] << 16)};
}

}  // namespace gr
