// pack.hip -- producer of the GEMM activation operand (actpack) for a row-major
// activation matrix: the first layer's RMSNorm input of a step, the output head of a
// standalone call, and the standalone GEMM.
//
// RMSNorm (tinyllm, Status: the Qwen3 components) is x / sqrt(mean(x^2) + eps) * g;
// the pack holds x * g and the per-row sum of squares (slot 0 of the ss_slots partial
// sums, the others zero), and the consuming GEMM applies 1 / sqrt(sum/K + eps) to its
// outputs.
#include "gr_internal.h"

namespace gr {

constexpr int kPackThreads = 1024;

// grid: 8 * actpack_tiles(B) blocks, one per (padded) batch row, and with a work list to
// build or counters to clear one more block that does that; each thread takes four
// consecutive columns per pass (K % 256 == 0, x rows 16-byte aligned).
__global__ __launch_bounds__(kPackThreads) void pack_rows_kernel(const float* __restrict__ x, int ldx, int B, int K,
                                                                 const float* __restrict__ gain, PackOut o1,
                                                                 PackOut o2, double* ss_out, RopeTable rope,
                                                                 RowSel sel, AttnSched sched) {
  const int b = blockIdx.x, tid = threadIdx.x;
  if ((sched.list || sched.cnt) && b == (int)gridDim.x - 1) {  // the extra last block
    if (sched.list) {  // the attention's work list (and the arrival counters cleared)
      __shared__ uint32_t sched_scan[kSchedScratchWords];
      static_assert(kPackThreads <= 1024, "the work list's scratch");
      build_attn_sched(sched, sched_scan);
    } else {
      for (int i = tid; i < sched.n_cnt; i += kPackThreads) sched.cnt[i] = 0u;
    }
    return;
  }
  const int src = (sel.idx && b < B) ? min(max(sel.idx[b], 0), sel.src_rows - 1) : b;
  if (rope.out && b < B && tid < rope.half_d) {
    const double inv = pow(rope.theta, -2.0 * (double)tid / (double)(2 * rope.half_d));
    double sn, cs;
    const int T = rope.tokens_per_seq > 0 ? rope.tokens_per_seq : 1;
    // row b: the token at row_pos[b], or token b % T of sequence b / T
    const int pos = rope.row_pos ? rope.row_pos[b] : rope.ctx[b / T] + b % T;
    sincos((double)pos * inv, &sn, &cs);
    rope.out[((size_t)b * rope.half_d + tid) * 2] = cs;
    rope.out[((size_t)b * rope.half_d + tid) * 2 + 1] = sn;
  }
  const int ns1 = o1.kind == kK32 ? K / 32 : K / 16, ns2 = o2.kind == kK32 ? K / 32 : K / 16;
  __shared__ float red[kPackThreads / 64];
  float ss = 0.f;
  for (int k0 = 4 * tid; k0 < K; k0 += 4 * kPackThreads) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (b < B) {
      const f32x4 xv = *(const f32x4*)(x + (size_t)src * ldx + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ss = __builtin_fmaf(xv[i], xv[i], ss);
        v[i] = gain ? xv[i] * gain[k0 + i] : xv[i];  // gains are only 4-byte aligned
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (o1.pack) actpack_put(o1.pack, o1.kind, ns1, b, k0 + i, v[i]);
      if (o2.pack) actpack_put(o2.pack, o2.kind, ns2, b, k0 + i, v[i]);
    }
  }
  if (ss_out && b < B) {
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
      for (int w = 0; w < kPackThreads / 64; ++w) tot += red[w];
      ss_out[b] = (double)tot;
      for (int s = 1; s < ss_slots(B); ++s) ss_out[(size_t)s * B + b] = 0.0;
    }
  }
}

hipError_t launch_pack_rows(const float* x, int ldx, int B, int K, const float* gain, PackOut o1, PackOut o2,
                            double* ss_out, hipStream_t st, RopeTable rope, RowSel sel, AttnSched sched) {
  if (rope.out && (rope.half_d <= 0 || rope.half_d > kPackThreads || (!rope.ctx && !rope.row_pos)))
    return hipErrorInvalidValue;
  if (sel.idx && sel.src_rows <= 0) return hipErrorInvalidValue;
  const int blocks = 8 * actpack_tiles(B) + (sched.list || sched.cnt ? 1 : 0);
  launch_kernel(pack_rows_kernel, dim3(blocks), dim3(kPackThreads), 0, st, x, ldx, B, K, gain, o1, o2, ss_out, rope,
                sel, sched);
  return hipGetLastError();
}

}  // namespace gr
