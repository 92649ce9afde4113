// pack.hip -- producers of the GEMM activation operand (actpack): RMSNorm + pack of
// the residual stream, and SwiGLU + pack of the gate/up products.
//
// RMSNorm and SwiGLU are the Qwen3 components tinyllm lists (Status): RMSNorm
// x / sqrt(mean(x^2) + eps) * g; SwiGLU silu(gate) * up with silu(z) = z / (1 + e^-z).
#include "gr_internal.h"

namespace gr {

constexpr int kPackThreads = 256;

// grid (B, ceil(K / 256)); block 256.  Every block recomputes its row's rms (the row
// is L2-resident and small) so that no second pass is needed.
__global__ __launch_bounds__(kPackThreads) void pack_rows_kernel(const float* __restrict__ x, int ldx, int B, int K,
                                                                 const float* __restrict__ gain, float eps,
                                                                 PackOut o1, PackOut o2, float* zero_ptr,
                                                                 size_t zero_n) {
  const int b = blockIdx.x, chunk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const float* xr = x + (size_t)b * ldx;
  __shared__ float red[kPackThreads / 64];
  float scale = 1.0f;
  if (gain) {
    float ss = 0.f;
    for (int k = tid; k < K; k += kPackThreads) ss = __builtin_fmaf(xr[k], xr[k], ss);
    ss = wave_sum(ss);
    if (lane == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kPackThreads / 64; ++w) tot += red[w];
    scale = 1.0f / sqrtf(tot / (float)K + eps);
  }
  const int k = chunk * kPackThreads + tid;
  if (chunk * kPackThreads < K) {  // K % 64 == 0: whole waves are in or out
    if (k - lane < K) {
      const float v = gain ? xr[k] * scale * gain[k] : xr[k];
      if (o1.pack) actpack_put_lane(o1.pack, o1.sums, o1.kind, o1.kind == kK32 ? K / 32 : K / 16, b, k, v, lane);
      if (o2.pack) actpack_put_lane(o2.pack, o2.sums, o2.kind, o2.kind == kK32 ? K / 32 : K / 16, b, k, v, lane);
    }
  }
  // padding rows of the last batch tile, and the zero fill, spread over all blocks
  const size_t nblk = (size_t)gridDim.x * gridDim.y;
  const size_t bid = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  const size_t pad_total = (size_t)(actpack_tiles(B) * 8 - B) * K;
  for (size_t i = bid * kPackThreads + tid; i < pad_total; i += nblk * kPackThreads) {
    if (o1.pack) actpack_zero_pad(o1.pack, o1.sums, o1.kind, o1.kind == kK32 ? K / 32 : K / 16, B, K, i);
    if (o2.pack) actpack_zero_pad(o2.pack, o2.sums, o2.kind, o2.kind == kK32 ? K / 32 : K / 16, B, K, i);
  }
  if (zero_ptr)
    for (size_t i = bid * kPackThreads + tid; i < zero_n; i += nblk * kPackThreads) zero_ptr[i] = 0.f;
}

__global__ __launch_bounds__(kPackThreads) void swiglu_pack_kernel(const float* __restrict__ gu, int B, int F,
                                                                   PackOut o) {
  const int b = blockIdx.x, chunk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int k = chunk * kPackThreads + tid;
  const int nsl = o.kind == kK32 ? F / 32 : F / 16;
  if (k - lane < F) {
    const float gv = gu[(size_t)b * 2 * F + k], uv = gu[(size_t)b * 2 * F + F + k];
    const float a = gv / (1.0f + expf(-gv)) * uv;
    actpack_put_lane(o.pack, o.sums, o.kind, nsl, b, k, a, lane);
  }
  const size_t nblk = (size_t)gridDim.x * gridDim.y;
  const size_t bid = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  const size_t pad_total = (size_t)(actpack_tiles(B) * 8 - B) * F;
  for (size_t i = bid * kPackThreads + tid; i < pad_total; i += nblk * kPackThreads)
    actpack_zero_pad(o.pack, o.sums, o.kind, nsl, B, F, i);
}

hipError_t launch_pack_rows(const float* x, int ldx, int B, int K, const float* gain, float eps, PackOut o1,
                            PackOut o2, float* zero_ptr, size_t zero_n, hipStream_t st) {
  const dim3 grid(B, (K + kPackThreads - 1) / kPackThreads);
  pack_rows_kernel<<<grid, kPackThreads, 0, st>>>(x, ldx, B, K, gain, eps, o1, o2, zero_ptr, zero_n);
  return hipGetLastError();
}

hipError_t launch_swiglu_pack(const float* gu, int B, int F, PackOut o, hipStream_t st) {
  const dim3 grid(B, (F + kPackThreads - 1) / kPackThreads);
  swiglu_pack_kernel<<<grid, kPackThreads, 0, st>>>(gu, B, F, o);
  return hipGetLastError();
}

}  // namespace gr
