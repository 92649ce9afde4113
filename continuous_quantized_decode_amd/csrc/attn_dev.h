// attn_dev.h -- device helpers shared by the attention kernels (attn.hip, attn_decode.hip):
// RoPE pair layout, the per-head QK-RMSNorm and rotation of the set-up, and the store of a
// token's K or V vector in the pool's format.
#pragma once

#include "gr_common.h"
#include "attn_internal.h"

namespace gr {

// ------------------------------------------------------------- setup helpers

// pair index i (0..D/2) of lane: rope pairs (i, i+D/2) [neox] or (2i, 2i+1) [norm]
GR_DEV void pair_dims(int i, int D, int style, int& da, int& db) {
  if (style == 0) {
    da = i;
    db = i + D / 2;
  } else {
    da = 2 * i;
    db = 2 * i + 1;
  }
}

// Per-head vector in pair layout (lane i < D/2 holds dims da, db): optional RMSNorm
// over the head, then RoPE at position pos with angles in fp64.
GR_DEV void norm_rope(float& a, float& b, bool active, const float* gain, float eps, int D, int da, int db,
                      double cs, double sn) {
  if (gain) {
    float ss = active ? a * a + b * b : 0.0f;
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
    if (active) {
      a = a * r * gain[da];
      b = b * r * gain[db];
    }
  }
  if (active) {
    const double ad = a, bd = b;
    a = (float)(ad * cs - bd * sn);
    b = (float)(ad * sn + bd * cs);
  }
}

template <int KVDT>
GR_DEV int kv_head_bytes_t(int D) {
  if constexpr (KVDT == KV_F32_T) return kPage * D * 4;
  if constexpr (KVDT == KV_F16_T) return kPage * D * 2;
  return kPage * D + kPage * (D / 32) * 2;
}

// Store a token's vector (LDS f32 [D]) in pool format: into the LDS staging row
// `stage` (format of patch_page) and, if `dst_head` is set, into the pool head block.
template <int KVDT>
GR_DEV void store_token(const float* vals, uint8_t* stage, uint8_t* dst_head, bool is_v, int D, int slot, int lane) {
  const int epl = D / 64;  // elements per lane
  if constexpr (KVDT == KV_Q8_T) {
    // lane holds elements epl*lane + e; 32-element blocks span 32/epl lanes
    float x[2] = {0.f, 0.f};
    float amax = 0.f;
    for (int e = 0; e < epl; ++e) {
      x[e] = vals[epl * lane + e];
      amax = fmaxf(amax, fabsf(x[e]));
    }
    const int span = 32 / epl;
    for (int o = 1; o < span; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float dsc = amax / 127.0f;
    for (int e = 0; e < epl; ++e) {
      const int d = epl * lane + e;
      float qf = dsc != 0.0f ? roundf(x[e] / dsc) : 0.0f;
      qf = fminf(127.0f, fmaxf(-127.0f, qf));
      const uint8_t c = (uint8_t)(int8_t)qf;
      stage[d] = c;
      if (dst_head) dst_head[is_v ? d * kPage + slot : slot * D + d] = c;
    }
    const int blk = (epl * lane) / 32;
    if (((epl * lane) & 31) == 0) {
      const u16 h = f2h(dsc);
      ((u16*)(stage + D))[blk] = h;
      if (dst_head) ((u16*)(dst_head + kPage * D))[slot * (D / 32) + blk] = h;
    }
  } else {
    for (int e = 0; e < epl; ++e) {
      const int d = epl * lane + e;
      const int idx = is_v ? d * kPage + slot : slot * D + d;
      if constexpr (KVDT == KV_F16_T) {
        const u16 h = f2h(vals[d]);
        ((u16*)stage)[d] = h;
        if (dst_head) ((u16*)dst_head)[idx] = h;
      } else {
        const float f = vals[d];
        ((float*)stage)[d] = f;
        if (dst_head) ((float*)dst_head)[idx] = f;
      }
    }
  }
}

}  // namespace gr
