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
constexpr int kQ5KBytes = 176;
constexpr int kQ6KBytes = 210;
constexpr int kQ8SbBytes = 272;  // eight 34-byte q8_0 blocks: 256 weights of a Q8_0 row

// Bytes of 256 consecutive weights of a matrix row (GGUF type ids: Q8_0 8, Q4_K 12, Q5_K
// 13, Q6_K 14).
constexpr int sb_bytes(int wtype) {
  return wtype == 12 ? kQ4KBytes : wtype == 13 ? kQ5KBytes : wtype == 8 ? kQ8SbBytes : kQ6KBytes;
}
constexpr int kWave = 64;

// Streamed loads (weights, KV pages).  Plain cached loads: a row's 128-byte lines are
// read by several instructions of the same wave, which must hit in L2 (the
// non-temporal policy refetches such lines from HBM).
template <class T>
GR_DEV T gr_ld(const T* p) {
  return *p;
}

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
// pairs x = hi + lo so that the MFMA sees it at ~fp32 accuracy.  Batch rows are
// grouped in tiles of 8; a tile is the A operand of 16 MFMA rows: row m holds part
// (m & 1) (0: hi, 1: lo) of batch row 8t + (m >> 1).  With the MFMA output layout
// (lane (n, g) holds rows 4g..4g+3) each lane then owns hi and lo of batch rows
// 8t + 2g and 8t + 2g + 1 and combines them without any lane exchange.
//
// Kind K32 (Q4_K consumers): slice s covers K [32s, 32s+32) (one Q4_K sub-block).
//   Lane l = (m = l%16, g = l/16) of slice s holds 8 bf16 (16 B) at K positions
//   32s + 8g + perm8(i), i = 0..7.
// Kind K16 (Q6_K consumers): slice s covers K [16s, 16s+16) (one Q6_K sub-block).
//   Lane l holds 4 bf16 (8 B) at K positions 16s + 4g + perm4(i); the fragments of
//   slices 2p and 2p+1 sit side by side (16 B per lane, slice 2p first).
// The permutations match the order in which the weight decoders emit quants (byte
// pairs 0,2 then 1,3 of each dword).
// K32: the 16 B of (tile t, slice s, lane l) are unit ((t*nslices + s)*64 + l);
// K16: the 16 B of (tile t, slices 2p and 2p+1, lane l) are unit ((t*nslices/2 + p)*64 + l).
// Producers write x * gain (the RMSNorm gain, or 1); the 1/rms factor of each row is
// applied by the consuming GEMM to its outputs (the product is linear in x).

enum ActKind { kK32 = 0, kK16 = 1 };

GR_DEV int perm8(int i) { return (i & 4) | ((i & 1) << 1) | ((i >> 1) & 1); }  // 0,2,1,3,4,6,5,7
GR_DEV int perm4(int i) { return ((i & 1) << 1) | ((i >> 1) & 1); }            // 0,2,1,3

// ---------------------------------------------------------------- pipelining
//
// Software pipeline over items [i0, i1) with two register buffers used in turn: b0
// holds item i0, issued by the caller before its own setup work; the loads of item
// i+1 are issued into the idle buffer (and pinned there by a scheduling barrier)
// before item i is processed from the other.  Unrolled by two so that no buffer is
// ever copied (a loop-carried copy makes the compiler wait for the fresh loads in the
// middle of the compute).  step(buffer, item, newer_in_flight) is told whether the next
// item's loads were issued after this buffer's.
template <class Buf, class Load, class Step>
GR_DEV void pipeline2_loaded(int i0, int i1, Buf& b0, Buf& b1, Load&& load, Step&& step) {
  int i = i0;
  for (; i + 2 < i1; i += 2) {
    load(b1, i + 1);
    __builtin_amdgcn_sched_barrier(0);
    step(b0, i, true);
    __builtin_amdgcn_sched_barrier(0);
    load(b0, i + 2);
    __builtin_amdgcn_sched_barrier(0);
    step(b1, i + 1, true);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (i + 1 < i1) {
    load(b1, i + 1);
    __builtin_amdgcn_sched_barrier(0);
    step(b0, i, true);
    __builtin_amdgcn_sched_barrier(0);
    step(b1, i + 1, false);
  } else {
    step(b0, i, false);
  }
}

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

}  // namespace gr
