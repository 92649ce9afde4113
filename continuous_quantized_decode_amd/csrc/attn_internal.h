// attn_internal.h -- parameters of the split-context paged attention kernels.
#pragma once

#include "gr_common.h"

namespace gr {

constexpr int KV_F32_T = 0;
constexpr int KV_F16_T = 1;
constexpr int KV_Q8_T = 2;

struct AttnParams {
  // B attention rows; row b is token b % tokens_per_seq of sequence b / tokens_per_seq, at
  // position ctx_lens[seq] + b % tokens_per_seq (its sequence's block table row is seq)
  int B, n_q_heads, n_kv_heads, head_dim;
  int tokens_per_seq;  // 1 for a decode step
  int self_in_pool;    // standalone: 1 if the row's own token is already stored (n_tok = pos + 1)
  int rows_per_unit;   // standalone: consecutive rows per wave when they share a sequence
                       // (rows_per_unit * n_q_heads / n_kv_heads <= 8); 0 or 1: one row
  // when set, row b is the token at position row_pos[b] of sequence row_seq[b] instead
  const int32_t* row_seq;
  const int32_t* row_pos;
  int max_blocks, pages_per_split, max_splits;
  float scale;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const void* k_pages;  // non-const in the fused variant (the new token is stored)
  const void* v_pages;
  // standalone: q f32 [B][Hq][D]
  const float* q;
  // fused: q/k/v f32 [B][qkv_ld] (q at 0, k at q_dim, v at q_dim + kv_dim)
  const float* qkv;
  int qkv_ld, q_dim, kv_dim;
  const float* q_norm;  // NULL: no QK-norm
  const float* k_norm;
  float eps;
  int rope_style;
  const double* rope;  // fused: cos, sin of each row's new position per pair [B][D/2][2]
  // partials [B][Hq][max_splits](*D)
  float* o_part;
  float* m_part;
  float* l_part;
  // decode kernel (one token per row; the log-sum-exp merge is done by the workgroup
  // that finishes a (row, KV head) last): workgroup partials [B * Hkv][wg_max][R (D + 2)]
  // (o[R][D], then m[R], l[R]), arrival counters [B * Hkv] (zero between launches), and
  // the output: f32 out [B][Hq][D] and / or the Wo input actpack (pack, kind, nslices)
  float* wg_part;
  uint32_t* wg_cnt;
  int wg_max, wg_pages;
  const uint32_t* sched;  // the work list (AttnSched): workgroup i * Hkv + g takes entry i
  float* out;
  uint16_t* pack;
  int pack_kind, pack_nslices;
};

// Sequence and position of attention row b.
GR_DEV void attn_row_place(const AttnParams& p, int b, int& seq, int& pos) {
  if (p.row_pos) {
    seq = p.row_seq[b];
    pos = p.row_pos[b];
  } else {
    const int T = p.tokens_per_seq > 0 ? p.tokens_per_seq : 1;
    seq = b / T;
    pos = p.ctx_lens[seq] + (b - seq * T);
  }
}

struct AttnPlan {
  int pages_per_split, max_splits;
  int dec_wg_max = 0, dec_wg_pages = 0;  // decode kernel (one token per row): workgroups per
                                         // (row, KV head), pages per workgroup,
  int dec_slots = 0;                     // resident workgroups (attn_dec_slots)
};

AttnPlan plan_attn(int B, int n_kv_heads, int max_ctx_tokens);
size_t attn_partial_floats(int B, int n_q_heads, int head_dim, const AttnPlan& pl);
hipError_t launch_attn_split(int kv_dtype, bool fused, const AttnParams& p, hipStream_t st);
hipError_t launch_attn_merge(const AttnParams& p, float* out, uint16_t* pack, int kind, int nslices, int fused,
                             hipStream_t st);
// Decode attention with the merge folded in (one token per row): workgroups of
// kAttnDecWaves waves take kAttnDecWaves * attn_dec_pages consecutive pages of one (row,
// KV head); each wave loads its pages all at once.
constexpr int kAttnDecWaves = 4;
constexpr int kAttnDecMaxWg = 512;  // workgroups per (row, KV head) one merge takes
constexpr int kAttnDecMaxGroups = 12;  // groups of pages per workgroup (8: long-context step 2 % slower)
// pages per wave (a group's pages sit in registers at once; measured: f16 two pages
// 21.2 us per Llama-3-8B layer against 22.8 us for four, whose refills wait a whole
// group; q8_0 three pages, within the 168 VGPRs of three waves per SIMD, took the
// Qwen3-8B step from 7.46 ms (six pages, two waves per SIMD) to 6.93 ms)
__host__ __device__ constexpr int attn_dec_pages(int kv_dtype) {
  return kv_dtype == KV_F32_T ? 2 : kv_dtype == KV_F16_T ? 2 : 3;
}
struct AttnDecPlan {
  int wg_pages;  // pages per workgroup
  int wg_max;    // the most workgroups of one (row, KV head); 0: max_tokens too long
};
AttnDecPlan plan_attn_dec(int kv_dtype, int max_tokens);
// resident decode-attention workgroups of the device for a KV format: three per CU for
// q8_0 (three waves per SIMD), two otherwise (three per CU for f16 measured no faster)
int attn_dec_slots(int kv_dtype);
size_t attn_dec_part_floats(int B, int n_q_heads, int head_dim, int wg_max);
// fused: the decode layer's variant (QK-norm, RoPE and the KV append of the new token
// from p.qkv, n_tok = ctx + 1); otherwise q from p.q and ctx tokens already in the pool.
hipError_t launch_attn_decode(int kv_dtype, bool fused, const AttnParams& p, hipStream_t st);
// The work list and cleared counters of a standalone call (one workgroup).
hipError_t launch_attn_sched(const struct AttnSched& s, hipStream_t st);

// QK-norm and RoPE of every row's q and k, the row's K/V stored at its position (several
// tokens of a sequence in one step), q written to q_out [B][Hq][D] for the standalone kernel.
hipError_t launch_attn_append(int kv_dtype, const AttnParams& p, float* q_out, hipStream_t st);

}  // namespace gr
