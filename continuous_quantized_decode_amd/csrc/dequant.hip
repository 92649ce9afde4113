// dequant.hip -- bit-exactness exports: weight-block dequantization and the paged KV
// gather.  Both run the same register-level decoders as the hot path (quant.h and
// kvpage.h), so a bit-exact match with the oracle pins the hot path's unpacking and
// page walk.
#include "gr_internal.h"
#include "attn_internal.h"
#include "kvpage.h"
#include "quant.h"

namespace gr {

// One wave per 16 Q4_K blocks: lane (col, kg) handles block 16w + col, quants of
// K group kg, exactly as a GEMM wave does for one super-block of 16 rows.
__global__ __launch_bounds__(256) void q4k_dequant_kernel(const uint8_t* __restrict__ blocks, int64_t n_blocks,
                                                          float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int64_t blk = w * 16 + col;
  if (w * 16 >= n_blocks) return;
  const int64_t src = blk < n_blocks ? blk : n_blocks - 1;
  Q4Regs r;
  q4_load(r, blocks + src * kQ4KBytes, kg);
  float sd[8], dm[8];
  q4_scales(r.hdr, sd, dm);
  if (blk >= n_blocks) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 bq = q4_expand(r.qs[j >> 1], (j & 1) != 0);
    const u32 wv[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = bf2f((u16)(wv[i >> 1] >> (16 * (i & 1)))) - 128.0f;
      out[blk * kQK + 32 * j + 8 * kg + perm8(i)] = __builtin_fmaf(sd[j], q, -dm[j]);
    }
  }
}

__global__ __launch_bounds__(256) void q6k_dequant_kernel(const uint8_t* __restrict__ blocks, int64_t n_blocks,
                                                          float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int64_t blk = w * 16 + col;
  if (w * 16 >= n_blocks) return;
  const int64_t src = blk < n_blocks ? blk : n_blocks - 1;
  Q6Regs r;
  q6_load(r, blocks + src * kQ6KBytes, kg);
  if (blk >= n_blocks) return;
  const float d = h2f(r.d);
#pragma unroll
  for (int hu = 0; hu < 4; ++hu) {
    const int h = hu >> 1, u = hu & 1;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int sub = 8 * h + 2 * rr + u;
      const u32x2 bq = q6_expand(r.part[hu], rr);
      const float sd = d * (float)(int)(int8_t)((r.sc[sub >> 2] >> (8 * (sub & 3))) & 0xFF);
      const u32 wv[2] = {bq.x, bq.y};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float q = bf2f((u16)(wv[i >> 1] >> (16 * (i & 1)))) - 160.0f;  // q - 32
        out[blk * kQK + 16 * sub + 4 * kg + perm4(i)] = sd * q;
      }
    }
  }
}

// GGUF q8_0 blocks (34 B: fp16 d, 32 int8): thread per block, through the same
// int8 -> f16 expansion the q8_0 KV path uses.
__global__ __launch_bounds__(256) void q8_0_dequant_kernel(const uint8_t* __restrict__ blocks, int64_t n_blocks,
                                                           float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_blocks) return;
  const uint8_t* b = blocks + i * 34;
  const u16* h = (const u16*)b;  // blocks are 2-byte aligned: read halves only
  const float d = h2f(h[0]);
#pragma unroll
  for (int wd = 0; wd < 8; ++wd) {
    const u32 codes = (u32)h[1 + 2 * wd] | ((u32)h[2 + 2 * wd] << 16);
    const u32x2 hv = q8_to_f16x4(codes);
    const u32 wv[2] = {hv.x, hv.y};
#pragma unroll
    for (int e = 0; e < 4; ++e) out[i * 32 + 4 * wd + perm4(e)] = d * h2f((u16)(wv[e >> 1] >> (16 * (e & 1))));
  }
}

// Gather: one wave per (row b, KV head g, page j); the page is read with the
// attention kernel's loader and written out as f32 values [B][max_ctx][Hkv][D].
template <int KVDT, int D>
__global__ __launch_bounds__(64) void gather_kernel(const uint8_t* __restrict__ pool, int is_v,
                                                    const int32_t* __restrict__ block_table,
                                                    const int32_t* __restrict__ ctx_lens, int max_blocks,
                                                    int n_kv_heads, int max_ctx, float* __restrict__ out) {
  const int lane = threadIdx.x;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int ctx = ctx_lens[b];
  if (j * kPage >= ctx) return;
  const int HB = KVDT == KV_F32_T ? kPage * D * 4 : KVDT == KV_F16_T ? kPage * D * 2 : kPage * D + kPage * (D / 32) * 2;
  const uint8_t* head = pool + (size_t)block_table[(size_t)b * max_blocks + j] * HB * n_kv_heads + (size_t)g * HB;
  PageRegs<KVDT, D> r;
  load_page<KVDT, D>(r, head, head, lane);
  const int n = lane & 15, kg = lane >> 4;
  auto put = [&](int tok, int d, float v) {
    const int t = j * kPage + tok;
    if (t < ctx) out[(((size_t)b * max_ctx + t) * n_kv_heads + g) * D + d] = v;
  };
  if (!is_v) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      float v[8];
      if constexpr (KVDT == KV_F16_T) {
        const u32 w[4] = {r.k[s].x, r.k[s].y, r.k[s].z, r.k[s].w};
        for (int i = 0; i < 8; ++i) v[i] = h2f((u16)(w[i >> 1] >> (16 * (i & 1))));
      } else if constexpr (KVDT == KV_F32_T) {
        const u32 w[8] = {r.k[s][0].x, r.k[s][0].y, r.k[s][0].z, r.k[s][0].w,
                          r.k[s][1].x, r.k[s][1].y, r.k[s][1].z, r.k[s][1].w};
        for (int i = 0; i < 8; ++i) v[i] = u2f(w[i]);
      } else {
        const u32x2 c0 = q8_to_f16x4(r.k[s].x), c1 = q8_to_f16x4(r.k[s].y);
        const u32 w[4] = {c0.x, c0.y, c1.x, c1.y};
        const u32 sw = r.ksc[s >> 1];
        const float ks = h2f((u16)((s & 1) ? (sw >> 16) : (sw & 0xFFFF)));
        float tmp[8];
        for (int i = 0; i < 8; ++i) tmp[i] = ks * h2f((u16)(w[i >> 1] >> (16 * (i & 1))));
        for (int i = 0; i < 8; ++i) v[perm8(i)] = tmp[i];
      }
      for (int i = 0; i < 8; ++i) put(n, 32 * s + 8 * kg + i, v[i]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      float v[4];
      if constexpr (KVDT == KV_F16_T) {
        const u32 w[2] = {r.v[t].x, r.v[t].y};
        for (int i = 0; i < 4; ++i) v[i] = h2f((u16)(w[i >> 1] >> (16 * (i & 1))));
      } else if constexpr (KVDT == KV_F32_T) {
        v[0] = u2f(r.v[t].x);
        v[1] = u2f(r.v[t].y);
        v[2] = u2f(r.v[t].z);
        v[3] = u2f(r.v[t].w);
      } else {
        const u32x2 c = q8_to_f16x4(r.v[t]);
        const u32 w[2] = {c.x, c.y};
        const int blkd = (16 * t) / 32;
        for (int i = 0; i < 4; ++i) {
          const int tok = 4 * kg + perm4(i);
          const u32 sw = __shfl(r.vsc[blkd >> 1], tok, 64);  // lane `tok` holds token tok's scales
          const float vs = h2f((u16)((blkd & 1) ? (sw >> 16) : (sw & 0xFFFF)));
          v[perm4(i)] = vs * h2f((u16)(w[i >> 1] >> (16 * (i & 1))));
        }
      }
      for (int i = 0; i < 4; ++i) put(4 * kg + i, 16 * t + n, v[i]);
    }
  }
}

hipError_t launch_dequant(int kind, const void* blocks, int64_t n, float* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (kind == 12) {
    const int64_t waves = (n + 15) / 16;
    q4k_dequant_kernel<<<dim3((unsigned)((waves + 3) / 4)), 256, 0, st>>>((const uint8_t*)blocks, n, out);
  } else if (kind == 14) {
    const int64_t waves = (n + 15) / 16;
    q6k_dequant_kernel<<<dim3((unsigned)((waves + 3) / 4)), 256, 0, st>>>((const uint8_t*)blocks, n, out);
  } else {
    q8_0_dequant_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>((const uint8_t*)blocks, n, out);
  }
  return hipGetLastError();
}

hipError_t launch_gather(int kv_dtype, int D, const void* pool, int is_v, const int32_t* bt, const int32_t* ctx,
                         int B, int max_blocks, int n_kv_heads, int max_ctx, float* out, hipStream_t st) {
  const int max_pages = (max_ctx + kPage - 1) / kPage;
  const dim3 grid(max_pages, n_kv_heads, B);
  const uint8_t* pl = (const uint8_t*)pool;
#define GR_G(KV, DD) gather_kernel<KV, DD><<<grid, 64, 0, st>>>(pl, is_v, bt, ctx, max_blocks, n_kv_heads, max_ctx, out)
  if (D == 128) {
    if (kv_dtype == 0) GR_G(KV_F32_T, 128);
    else if (kv_dtype == 1) GR_G(KV_F16_T, 128);
    else GR_G(KV_Q8_T, 128);
  } else {
    if (kv_dtype == 0) GR_G(KV_F32_T, 64);
    else if (kv_dtype == 1) GR_G(KV_F16_T, 64);
    else GR_G(KV_Q8_T, 64);
  }
#undef GR_G
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Read-only stream (measurement aid): every workgroup's waves walk the buffer in 8 KB
// steps (eight 1 KB loads of 16 bytes per lane in flight per wave), grid-stride, and
// fold what they read into one checksum word per workgroup (plain stores: same-address
// atomics from every workgroup would serialize and show up in the time): the ceiling a
// plain streaming read reaches on this GPU, next to which the step's kernels are
// measured.
constexpr int kStreamGrid = GR_STREAM_READ_WORDS, kStreamDepth = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t step = (size_t)gridDim.x * 4 * kStreamDepth * 64;
  uint32_t acc = 0;
  for (size_t base = ((size_t)blockIdx.x * 4 + wave) * kStreamDepth * 64; base < n16; base += step) {
    u32x4 v[kStreamDepth];
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d) {
      const size_t i = base + (size_t)d * 64 + lane;
      v[d] = p[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d)
      if (base + (size_t)d * 64 + lane < n16) acc ^= v[d].x ^ v[d].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  __shared__ uint32_t s_acc[4];
  if (lane == 0) s_acc[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
}

hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* out, hipStream_t st) {
  if (bytes < 16) return hipSuccess;
  stream_read_kernel<<<dim3(kStreamGrid), 256, 0, st>>>((const u32x4*)p, bytes / 16, out);
  return hipGetLastError();
}

}  // namespace gr
