// gr_common.h -- device-side helpers shared by the gfx950 kernels of libgr.
//
// Vector types, fp16 / bf16 bit helpers, the MFMA wrappers, and the layout of the
// packed activation operand ("actpack") that every fused-dequant GEMM consumes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define GR_DEV __device__ __forceinline__

typedef uint32_t u32;
typedef unsigned short u16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));

namespace gr {

constexpr int kPage = 16;
constexpr int kQK = 256;  // weights per K-quant super-block
constexpr int kQ4KBytes = 144;
constexpr int kQ6KBytes = 210;
constexpr int kWave = 64;

// ------------------------------------------------------------------ fp16 / bf16

// Bit reinterpretation through a by-value argument: clang's __builtin_bit_cast applied
// directly to an ext_vector element (v.y) reads element 0, so elements are always
// passed through these helpers.
GR_DEV float u2f(u32 x) { return __builtin_bit_cast(float, x); }
GR_DEV u32 f2u(float x) { return __builtin_bit_cast(u32, x); }

GR_DEV float h2f(u16 h) { return (float)__builtin_bit_cast(_Float16, h); }
GR_DEV u16 f2h(float f) { return __builtin_bit_cast(u16, (_Float16)f); }  // round to nearest even

GR_DEV u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }  // round to nearest even
GR_DEV float bf2f(u16 b) { return __builtin_bit_cast(float, (u32)b << 16); }

// x = hi + lo with hi, lo bf16: hi = bf16(x), lo = bf16(x - hi).  |x - hi - lo| <= 2^-16 |x|.
GR_DEV void split_bf16(float x, u16& hi, u16& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

// -------------------------------------------------------------------- MFMA

// D[16x16] = A[16x32] B[32x16], bf16 in, fp32 out.  Lane l holds A row l%16 and
// B column l%16, eight K values each in K group l/16; D rows 4(l/16)..+3 of column l%16.
GR_DEV f32x4 mfma_bf16_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
// Same with K=16 (four K values per lane).
GR_DEV f32x4 mfma_bf16_k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                   0, 0);
}
GR_DEV f32x4 mfma_f16_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}
GR_DEV f32x4 mfma_f16_k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                               0);
}

// -------------------------------------------------------------- actpack layout
//
// The activation operand of a GEMM, x [B][K] f32, is stored once per step as bf16
// pairs x = hi + lo so the MFMA sees it at ~fp32 accuracy.  Batch rows are grouped
// in tiles of 8; a tile is the A operand of 16 MFMA rows: row m < 8 is the hi part of
// batch row 8t+m, row m >= 8 the lo part of batch row 8t+m-8.
//
// Kind K32 (Q4_K consumers): slice s covers K [32s, 32s+32) (one Q4_K sub-block).
//   Lane l = (m = l%16, g = l/16) of slice s holds 8 bf16 (16 B) at K positions
//   32s + 8g + kPerm8[i], i = 0..7.
// Kind K16 (Q6_K consumers): slice s covers K [16s, 16s+16) (one Q6_K sub-block).
//   Lane l holds 4 bf16 (8 B) at K positions 16s + 4g + kPerm4[i].
// The permutations match the order in which the weight decoders emit quants (byte
// pairs 0,2 then 1,3 of each dword).
// Fragment of (tile t, slice s, lane l) sits at element ((t*nslices + s)*64 + l).
// Sums: sums[(t*nslices + s)*16 + m] = sum over the slice of row m's values (hi or
// lo part), used for the weight-offset terms.

enum ActKind { kK32 = 0, kK16 = 1 };

GR_DEV int perm8(int i) { return (i & 4) | ((i & 1) << 1) | ((i >> 1) & 1); }  // 0,2,1,3,4,6,5,7
GR_DEV int perm4(int i) { return ((i & 1) << 1) | ((i >> 1) & 1); }            // 0,2,1,3

// ---------------------------------------------------------------- reductions

GR_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
GR_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Aligned 4-byte load of a possibly 2-byte-aligned address.
GR_DEV u32 load_u32_a2(const uint8_t* p) {
  uintptr_t a = (uintptr_t)p;
  const u32* base = (const u32*)(a & ~(uintptr_t)3);
  u32 lo = __builtin_nontemporal_load(base);
  if ((a & 3) == 0) return lo;
  u32 hi = __builtin_nontemporal_load(base + 1);
  return __builtin_amdgcn_alignbyte(hi, lo, (u32)(a & 3));
}

}  // namespace gr
