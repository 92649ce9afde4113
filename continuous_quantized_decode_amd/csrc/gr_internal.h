// gr_internal.h -- internal declarations shared by the translation units of libgr.
#pragma once

#include "gr_common.h"
#include "../../include/gr.h"

namespace gr {

// ------------------------------------------------------------------------ GEMM

struct GemmSeg {
  const uint8_t* w;
  int rows;       // rows of this matrix
  int row_off;    // first output column of this matrix in y
  int group_off;  // first wave group of this matrix
};

struct GemmParams {
  GemmSeg seg[3];
  int nseg;
  int total_groups;
  int nsb;  // super-blocks per row
  size_t row_bytes;
  const void* xpack;
  const float* xsum;
  int nslices;
  int B;
  float* y;
  int ldy;
  int splits, sb_per_split;
  int total_items;
  int mode;  // kStorePartial, kStoreAtomic, kStoreDirect
};

enum { kStorePartial = 0, kStoreAtomic = 1, kStoreDirect = 2 };

struct GemmPlan {
  int nt, btn, groups, splits, sb_per_split;
};

// Write a wave's accumulators.  Lane (col, kg) holds MFMA rows 4kg..4kg+3 of column
// col: kg 0,1 are the hi parts of batch rows 4kg..4kg+3, kg 2,3 the lo parts of the
// same rows, so y = acc(kg) + acc(kg+2).
template <int NT, int BTN>
GR_DEV void gemm_store(const GemmParams& p, f32x4 (&acc)[NT][BTN], const GemmSeg& sg, const int (&nloc)[NT],
                       int split, int lane) {
  const int kg = lane >> 4;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int b = 0; b < BTN; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[t][b][i];
        v += __shfl_xor(v, 32, 64);
        const int row = 8 * b + 4 * kg + i;
        if (kg < 2 && nloc[t] < sg.rows && row < p.B) {
          const size_t col = (size_t)sg.row_off + nloc[t];
          if (p.mode == kStorePartial)
            p.y[((size_t)split * p.B + row) * p.ldy + col] = v;
          else if (p.mode == kStoreAtomic)
            atomicAdd(p.y + (size_t)row * p.ldy + col, v);
          else
            p.y[(size_t)row * p.ldy + col] = v;
        }
      }
    }
  }
}

GemmPlan plan_gemm(int wtype, const int* seg_rows, int nseg, int K, int B, int max_splits);
hipError_t launch_gemm(int wtype, const GemmPlan& pl, const uint8_t* const* w, const int* seg_rows, int nseg, int K,
                       int B, const void* xpack, const float* xsum, float* y, int ldy, int mode, hipStream_t st);

// ---------------------------------------------------------------------- actpack

// Store activation v of (row b, column k) into an actpack as bf16 hi/lo and update
// the per-slice sums.  All 64 lanes of the wave must call it together with
// k = k0 + lane, k0 a multiple of 64 (slices then align with lane groups).
GR_DEV void actpack_put_lane(u16* pack, float* sums, int kind, int nslices, int b, int k, float v, int lane) {
  u16 hi, lo;
  split_bf16(v, hi, lo);
  const int t = b >> 3, r = b & 7;
  int s;
  size_t ih, il;
  if (kind == kK32) {
    s = k >> 5;
    const int w = k & 31, g = w >> 3, i = perm8(w & 7);
    const size_t fb = ((size_t)t * nslices + s) * 64;
    ih = (fb + g * 16 + r) * 8 + i;
    il = (fb + g * 16 + 8 + r) * 8 + i;
  } else {
    s = k >> 4;
    const int w = k & 15, g = w >> 2, i = perm4(w & 3);
    const size_t fb = ((size_t)t * nslices + s) * 64;
    ih = (fb + g * 16 + r) * 4 + i;
    il = (fb + g * 16 + 8 + r) * 4 + i;
  }
  pack[ih] = hi;
  pack[il] = lo;
  float sh = bf2f(hi), sl = bf2f(lo);
  const int span = kind == kK32 ? 32 : 16;
  for (int o = 1; o < span; o <<= 1) {
    sh += __shfl_xor(sh, o, 64);
    sl += __shfl_xor(sl, o, 64);
  }
  if ((lane & (span - 1)) == 0) {
    sums[((size_t)t * nslices + s) * 16 + r] = sh;
    sums[((size_t)t * nslices + s) * 16 + 8 + r] = sl;
  }
}

// Zero the padding rows b in [B, 8*actpack_tiles(B)) of an actpack; `slot`
// enumerates (row, k) over the padding.
GR_DEV void actpack_zero_pad(u16* pack, float* sums, int kind, int nslices, int B, int K, size_t slot) {
  const int tiles = B <= 8 ? 1 : B <= 16 ? 2 : B <= 32 ? 4 : 8, pad = tiles * 8 - B;
  if (pad == 0) return;
  const size_t total = (size_t)pad * K;
  if (slot >= total) return;
  const int b = B + (int)(slot / K), k = (int)(slot % K);
  const int t = b >> 3, r = b & 7;
  if (kind == kK32) {
    const int s = k >> 5, w = k & 31, g = w >> 3, i = perm8(w & 7);
    const size_t fb = ((size_t)t * nslices + s) * 64;
    pack[(fb + g * 16 + r) * 8 + i] = 0;
    pack[(fb + g * 16 + 8 + r) * 8 + i] = 0;
    if (w == 0) sums[((size_t)t * nslices + s) * 16 + r] = sums[((size_t)t * nslices + s) * 16 + 8 + r] = 0.f;
  } else {
    const int s = k >> 4, w = k & 15, g = w >> 2, i = perm4(w & 3);
    const size_t fb = ((size_t)t * nslices + s) * 64;
    pack[(fb + g * 16 + r) * 4 + i] = 0;
    pack[(fb + g * 16 + 8 + r) * 4 + i] = 0;
    if (w == 0) sums[((size_t)t * nslices + s) * 16 + r] = sums[((size_t)t * nslices + s) * 16 + 8 + r] = 0.f;
  }
}

// ----------------------------------------------------------------- pack launchers

struct PackOut {
  u16* pack;
  float* sums;
  int kind;  // kK32 / kK16; pack == nullptr: unused
};

// x [B][K] (row stride ldx) -> up to two actpacks; with `gain`, rows are RMS-normalized
// (x / sqrt(mean(x^2) + eps) * gain) first.  Also zeroes zero_n floats at zero_ptr.
hipError_t launch_pack_rows(const float* x, int ldx, int B, int K, const float* gain, float eps, PackOut o1,
                            PackOut o2, float* zero_ptr, size_t zero_n, hipStream_t st);
// gu [B][2F] (gate | up) -> actpack of silu(gate) * up.
hipError_t launch_swiglu_pack(const float* gu, int B, int F, PackOut o, hipStream_t st);

// Batch tiles an actpack holds for B rows: the GEMM kernels process 1, 2, 4 or 8
// tiles of 8 rows at once, so the pack is padded (with zero rows) to that count.
__host__ __device__ inline int actpack_tiles(int B) { return B <= 8 ? 1 : B <= 16 ? 2 : B <= 32 ? 4 : 8; }

// Bytes of the fragments / sums of an actpack for B rows of K values.
inline size_t actpack_frag_bytes(int B, int K, int kind) {
  (void)kind;
  return (size_t)actpack_tiles(B) * K * 16 * 2;  // 16 MFMA rows (8 hi + 8 lo) x K bf16
}
inline size_t actpack_sum_bytes(int B, int K, int kind) {
  const int nsl = kind == kK32 ? K / 32 : K / 16;
  return (size_t)actpack_tiles(B) * nsl * 16 * sizeof(float);
}

}  // namespace gr
