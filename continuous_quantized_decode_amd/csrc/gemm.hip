// gemm.hip -- fused-dequant skinny GEMM for GGUF Q4_K / Q6_K weights on gfx950.
//
// y[b][n] = sum_k W[n][k] x[b][k] for the B active decode rows sharing one pass over
// the weights (Leone, intro: active decode rows share matrix operations).  Every
// weight byte is read from HBM exactly once per call.
//
// Design (gfx950):
//  * One wave owns NT tiles of 16 weight rows and a range of super-blocks (split-K).
//  * Quants are expanded in registers into exact bf16 integers (128 + q via an OR
//    with the exponent bits) and fed as the B operand of v_mfma_f32_16x16x32_bf16
//    (Q4_K: one 32-weight sub-block per MFMA) or v_mfma_f32_16x16x16_bf16 (Q6_K: one
//    16-weight sub-block per MFMA).  The A operand is the activation tile in bf16
//    hi/lo form (actpack), so products and sums are exact up to fp32 accumulation.
//  * Each MFMA result is scaled per (row, sub-block) in fp32:
//      Q4_K: acc += d*sc*D - (128*d*sc + dmin*m) * S
//      Q6_K: acc += d*sc*D - 160*d*sc * S
//    where S is the sub-block sum of the activation part (precomputed in actpack).
//  * Weight loads for super-block sb+1 are issued before the MFMAs of sb.
#include "gr_internal.h"
#include "quant.h"

namespace gr {

template <int NT, int BTN>
__global__ __launch_bounds__(256) void q4k_gemm_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= p.total_items) return;
  const int split = item / p.total_groups;
  const int gidx = item - split * p.total_groups;
  int s = 0;
  while (s + 1 < p.nseg && gidx >= p.seg[s + 1].group_off) ++s;
  const GemmSeg sg = p.seg[s];
  const int group = gidx - sg.group_off;
  const int col = lane & 15, kg = lane >> 4;

  const uint8_t* rowp[NT];
  int nloc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    nloc[t] = (group * NT + t) * 16 + col;
    rowp[t] = sg.w + (size_t)min(nloc[t], sg.rows - 1) * p.row_bytes;
  }
  const int sb0 = split * p.sb_per_split;
  const int sb1 = min(p.nsb, sb0 + p.sb_per_split);

  f32x4 acc[NT][BTN];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < BTN; ++b) acc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4* xp = (const u32x4*)p.xpack;
  const f32x4* xs = (const f32x4*)p.xsum;

  Q4Regs cur[NT], nxt[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) q4_load(cur[t], rowp[t] + (size_t)sb0 * kQ4KBytes, kg);

  for (int sb = sb0; sb < sb1; ++sb) {
    if (sb + 1 < sb1) {
#pragma unroll
      for (int t = 0; t < NT; ++t) q4_load(nxt[t], rowp[t] + (size_t)(sb + 1) * kQ4KBytes, kg);
    }
    float sd[NT][8], mm[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      q4_scales(cur[t].hdr, sd[t], mm[t]);
#pragma unroll
      for (int j = 0; j < 8; ++j) mm[t][j] = __builtin_fmaf(128.0f, sd[t][j], mm[t][j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int slice = sb * 8 + j;
      u32x4 a[BTN];
      f32x4 ssum[BTN];
#pragma unroll
      for (int b = 0; b < BTN; ++b) {
        a[b] = xp[((size_t)b * p.nslices + slice) * 64 + lane];
        ssum[b] = xs[((size_t)b * p.nslices + slice) * 4 + kg];
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 bq = q4_expand(cur[t].qs[j >> 1], (j & 1) != 0);
#pragma unroll
        for (int b = 0; b < BTN; ++b) {
          const f32x4 dd = mfma_bf16_k32(a[b], bq, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[t][b][i] = __builtin_fmaf(sd[t][j], dd[i], __builtin_fmaf(-mm[t][j], ssum[b][i], acc[t][b][i]));
        }
      }
    }
    if (sb + 1 < sb1) {
#pragma unroll
      for (int t = 0; t < NT; ++t) cur[t] = nxt[t];
    }
  }
  gemm_store<NT, BTN>(p, acc, sg, nloc, split, lane);
}

template <int NT, int BTN>
__global__ __launch_bounds__(256) void q6k_gemm_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= p.total_items) return;
  const int split = item / p.total_groups;
  const int gidx = item - split * p.total_groups;
  int s = 0;
  while (s + 1 < p.nseg && gidx >= p.seg[s + 1].group_off) ++s;
  const GemmSeg sg = p.seg[s];
  const int group = gidx - sg.group_off;
  const int col = lane & 15, kg = lane >> 4;

  const uint8_t* rowp[NT];
  int nloc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    nloc[t] = (group * NT + t) * 16 + col;
    rowp[t] = sg.w + (size_t)min(nloc[t], sg.rows - 1) * p.row_bytes;
  }
  const int sb0 = split * p.sb_per_split;
  const int sb1 = min(p.nsb, sb0 + p.sb_per_split);

  f32x4 acc[NT][BTN];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < BTN; ++b) acc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x2* xp = (const u32x2*)p.xpack;
  const f32x4* xs = (const f32x4*)p.xsum;

  Q6Regs cur[NT], nxt[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) q6_load(cur[t], rowp[t] + (size_t)sb0 * kQ6KBytes, kg);

  for (int sb = sb0; sb < sb1; ++sb) {
    if (sb + 1 < sb1) {
#pragma unroll
      for (int t = 0; t < NT; ++t) q6_load(nxt[t], rowp[t] + (size_t)(sb + 1) * kQ6KBytes, kg);
    }
    float dsc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) dsc[t] = h2f(cur[t].d);
#pragma unroll
    for (int hu = 0; hu < 4; ++hu) {
      const int h = hu >> 1, u = hu & 1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sub = 8 * h + 2 * r + u;  // 16-weight sub-block within the super-block
        const int slice = sb * 16 + sub;
        u32x2 a[BTN];
        f32x4 ssum[BTN];
#pragma unroll
        for (int b = 0; b < BTN; ++b) {
          a[b] = xp[((size_t)b * p.nslices + slice) * 64 + lane];
          ssum[b] = xs[((size_t)b * p.nslices + slice) * 4 + kg];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const u32x2 bq = q6_expand(cur[t].part[hu], r);
          const int scv = (int)(int8_t)((cur[t].sc[sub >> 2] >> (8 * (sub & 3))) & 0xFF);
          const float sd = dsc[t] * (float)scv;
          const float c160 = 160.0f * sd;
#pragma unroll
          for (int b = 0; b < BTN; ++b) {
            const f32x4 dd = mfma_bf16_k16(a[b], bq, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[t][b][i] = __builtin_fmaf(sd, dd[i], __builtin_fmaf(-c160, ssum[b][i], acc[t][b][i]));
          }
        }
      }
    }
    if (sb + 1 < sb1) {
#pragma unroll
      for (int t = 0; t < NT; ++t) cur[t] = nxt[t];
    }
  }
  gemm_store<NT, BTN>(p, acc, sg, nloc, split, lane);
}

// ---------------------------------------------------------------------------------
// launch

#define GR_GEMM_CASES(KER)                                                                         \
  switch (nt * 100 + btn) {                                                                        \
    case 101: KER<1, 1><<<grid, 256, 0, st>>>(p); break;                                           \
    case 102: KER<1, 2><<<grid, 256, 0, st>>>(p); break;                                           \
    case 104: KER<1, 4><<<grid, 256, 0, st>>>(p); break;                                           \
    case 108: KER<1, 8><<<grid, 256, 0, st>>>(p); break;                                           \
    case 201: KER<2, 1><<<grid, 256, 0, st>>>(p); break;                                           \
    case 202: KER<2, 2><<<grid, 256, 0, st>>>(p); break;                                           \
    case 204: KER<2, 4><<<grid, 256, 0, st>>>(p); break;                                           \
    case 401: KER<4, 1><<<grid, 256, 0, st>>>(p); break;                                           \
    case 402: KER<4, 2><<<grid, 256, 0, st>>>(p); break;                                           \
    default: return hipErrorInvalidValue;                                                          \
  }

GemmPlan plan_gemm(int wtype, const int* seg_rows, int nseg, int K, int B, int max_splits) {
  GemmPlan pl{};
  int tiles = 0;
  for (int i = 0; i < nseg; ++i) tiles += (seg_rows[i] + 15) / 16;
  const int btn = B <= 8 ? 1 : B <= 16 ? 2 : B <= 32 ? 4 : 8;
  int nt = 1;
  if (tiles >= 4096)
    nt = 4;
  else if (tiles >= 1024)
    nt = 2;
  // registers: keep NT*BTN accumulators modest
  while (nt > 1 && nt * btn > 8) nt >>= 1;
  if (btn == 8) nt = 1;
  int groups = 0;
  for (int i = 0; i < nseg; ++i) groups += (seg_rows[i] + 16 * nt - 1) / (16 * nt);
  const int nsb = K / kQK;
  int splits = 1;
  if (groups < 1536) splits = (2048 + groups - 1) / groups;
  if (splits > max_splits) splits = max_splits;
  int min_sb = wtype == 12 ? 2 : 1;
  if (splits > nsb / min_sb) splits = nsb / min_sb;
  if (splits < 1) splits = 1;
  int per = (nsb + splits - 1) / splits;
  splits = (nsb + per - 1) / per;
  pl.nt = nt;
  pl.btn = btn;
  pl.groups = groups;
  pl.splits = splits;
  pl.sb_per_split = per;
  return pl;
}

hipError_t launch_gemm(int wtype, const GemmPlan& pl, const uint8_t* const* w, const int* seg_rows, int nseg, int K,
                       int B, const void* xpack, const float* xsum, float* y, int ldy, int mode, hipStream_t st) {
  GemmParams p{};
  p.nseg = nseg;
  int goff = 0, roff = 0;
  for (int i = 0; i < nseg; ++i) {
    p.seg[i].w = w[i];
    p.seg[i].rows = seg_rows[i];
    p.seg[i].row_off = roff;
    p.seg[i].group_off = goff;
    goff += (seg_rows[i] + 16 * pl.nt - 1) / (16 * pl.nt);
    roff += seg_rows[i];
  }
  p.total_groups = goff;
  p.nsb = K / kQK;
  p.row_bytes = (size_t)(K / kQK) * (wtype == 12 ? kQ4KBytes : kQ6KBytes);
  p.xpack = xpack;
  p.xsum = xsum;
  p.nslices = wtype == 12 ? K / 32 : K / 16;
  p.B = B;
  p.y = y;
  p.ldy = ldy;
  p.splits = pl.splits;
  p.sb_per_split = pl.sb_per_split;
  p.total_items = goff * pl.splits;
  p.mode = mode;
  const int nt = pl.nt, btn = pl.btn;
  const dim3 grid((p.total_items + 3) / 4);
  if (wtype == 12) {
    GR_GEMM_CASES(q4k_gemm_kernel)
  } else {
    GR_GEMM_CASES(q6k_gemm_kernel)
  }
  return hipGetLastError();
}

}  // namespace gr
