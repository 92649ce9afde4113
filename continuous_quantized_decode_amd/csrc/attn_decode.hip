// attn_decode.hip -- paged GQA decode attention with the split merge folded in (gfx950).
//
// One decode token per row: every active row attends over its own cache (Leone, intro),
// reading pages of a physical pool through its logical block table (tinyllm, Status)
// in place, never gathered into contiguous K/V.
//
// Work: a workgroup of kAttnDecWaves waves takes one (row b, KV head g) and a range of
// kAttnDecWaves * attn_dec_pages pages of the row.  The waves share the set-up (q of the
// group's R query heads, and in the decode layer QK-RMSNorm, RoPE and the store of the
// new token's K/V), then each wave walks its own pages with all of their loads in flight
// at once:
//   scores  S[m][t] = q_m . K[t]   v_mfma_f32_16x16x32_f16, A = the R heads as f16 hi/lo
//                                  rows (m = 2h + part), B = the page's K
//   softmax online, log2 domain (q pre-scaled by scale * log2 e)
//   output  O[m][d] += P[m][t] V[t][d]  v_mfma_f32_16x16x16_f16, A = P (hi/lo rows,
//                                  transposed through the wave's LDS), B = the page's V
// The waves' (m, l, O) combine in LDS.  A row whose context needs several workgroups
// has each of them write its combined state; the workgroup that arrives last (an
// agent-scope counter per (row, KV head)) merges all of them by log-sum-exp, in
// workgroup order (so the result does not depend on which one is last), writes the
// output and resets the counter.  Merge arithmetic: M = max_j m_j,
// L = sum_j l_j 2^(m_j - M), o = sum_j O_j 2^(m_j - M) / L.
//
// Cross-workgroup visibility: the partial states are written with agent-scope stores
// (write-through past the per-XCD L2) and read with agent-scope loads (which do not hit
// a stale L2 line); a writer waits for its stores to complete before its arrival is
// counted, and the reader loads only after its own arrival returned the final count.
#include "gr_internal.h"
#include "attn_internal.h"
#include "kvpage.h"
#include "attn_dev.h"

namespace gr {

static_assert(kAttnDecMaxGroups <= kSchedMaxGroups, "the work list's bound on groups per range");

namespace {

GR_DEV void st_agent(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
GR_DEV float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS written by some lanes of a wave and read by others: the wave's LDS operations
// execute in order, so completing the writes (lgkmcnt) and keeping the compiler from
// moving memory accesses across is enough; no workgroup barrier.
GR_DEV void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

constexpr int kMaxR = 8;  // query heads per KV head

// Online-softmax state of the R heads: lane (n, kg) holds heads 2kg and 2kg + 1 (e = 0,
// 1): m and l in the log2 domain, and O[t] = MFMA rows 4kg..4kg + 3 (head 2kg hi, lo,
// head 2kg + 1 hi, lo) of dims 16t + n.
template <int D>
struct SmState {
  float m[2], l[2];
  f32x4 O[D / 16];
};

// One page of one row: `valid` tokens (>= 1) of its 16 hold context; the rest may hold
// anything, NaN included, and take no weight.
template <int KVDT, int D>
GR_DEV void dec_page(PageRegs<KVDT, D>& cur, int valid, const u32x4 (&qf)[D / 32], u16 (*sp)[16][16], int lane,
                     bool live, SmState<D>& st) {
  constexpr int NS = D / 32, NT = D / 16;
  const int n = lane & 15, kg = lane >> 4;
  if constexpr (KVDT != KV_Q8_T) {
    // zero the V of slots past the context so that 0 * V stays 0 in the PV product
    if (valid < kPage) mask_v_tail<KVDT, D>(cur, valid, lane);
  }
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if constexpr (KVDT == KV_F16_T) {
      sc = mfma_f16_k32(qf[s], cur.k[s], sc);
    } else if constexpr (KVDT == KV_F32_T) {
      u32x2 h0, l0, h1, l1;
      f32_to_f16hl(cur.k[s][0], h0, l0);
      f32_to_f16hl(cur.k[s][1], h1, l1);
      sc = mfma_f16_k32(qf[s], u32x4{h0.x, h0.y, h1.x, h1.y}, sc);
      sc = mfma_f16_k32(qf[s], u32x4{l0.x, l0.y, l1.x, l1.y}, sc);
    } else {
      const u32x2 c0 = q8_to_f16x4(cur.k[s].x), c1 = q8_to_f16x4(cur.k[s].y);
      const f32x4 part = mfma_f16_k32(qf[s], u32x4{c0.x, c0.y, c1.x, c1.y}, f32x4{0.f, 0.f, 0.f, 0.f});
      const u32 w = cur.ksc[s >> 1];
      const float ks = h2f((u16)((s & 1) ? (w >> 16) : (w & 0xFFFF)));
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = __builtin_fmaf(ks, part[i], sc[i]);
    }
  }
  // lane (token n, kg): rows 4kg..4kg+3 = heads 2kg (hi, lo), 2kg+1 (hi, lo)
  float pv[2], alpha[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float sv = n < valid ? sc[2 * e] + sc[2 * e + 1] : -INFINITY;
    float mx = sv;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float mnew = fmaxf(st.m[e], mx);  // finite: the page has a valid token
    alpha[e] = exp2f(st.m[e] - mnew);
    pv[e] = exp2f(sv - mnew);
    float ps = pv[e];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o, 64);
    st.l[e] = st.l[e] * alpha[e] + ps;
    st.m[e] = mnew;
  }
  // P (f16 hi/lo rows) to the wave's LDS, transposed to the PV A layout
  if constexpr (KVDT == KV_Q8_T) {
    const int col = 4 * (n >> 2) + perm4(n & 3);
#pragma unroll
    for (int blk = 0; blk < D / 32; ++blk) {
      const u32 w = cur.vsc[blk >> 1];
      const float vs = h2f((u16)((blk & 1) ? (w >> 16) : (w & 0xFFFF)));
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float x = n < valid ? pv[e] * vs : 0.0f;
        const u16 h = f2h(x);
        if (live) {
          sp[blk][4 * kg + 2 * e][col] = h;
          sp[blk][4 * kg + 2 * e + 1][col] = f2h(x - h2f(h));
        }
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const u16 h = f2h(pv[e]);
      if (live) {
        sp[0][4 * kg + 2 * e][n] = h;
        sp[0][4 * kg + 2 * e + 1][n] = f2h(pv[e] - h2f(h));
      }
    }
  }
  wave_lds_fence();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    st.O[t][0] *= alpha[0];
    st.O[t][1] *= alpha[0];
    st.O[t][2] *= alpha[1];
    st.O[t][3] *= alpha[1];
  }
  if constexpr (KVDT == KV_Q8_T) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x2 pa = *(const u32x2*)&sp[t >> 1][n][4 * kg];
      st.O[t] = mfma_f16_k16(pa, q8_to_f16x4(cur.v[t]), st.O[t]);
    }
  } else {
    const u32x2 pa = *(const u32x2*)&sp[0][n][4 * kg];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (KVDT == KV_F16_T) {
        st.O[t] = mfma_f16_k16(pa, cur.v[t], st.O[t]);
      } else {
        u32x2 hi, lo;
        f32_to_f16hl(cur.v[t], hi, lo);
        st.O[t] = mfma_f16_k16(pa, hi, st.O[t]);
        st.O[t] = mfma_f16_k16(pa, lo, st.O[t]);
      }
    }
  }
  wave_lds_fence();  // the next page's P writes stay behind these reads
}

}  // namespace

// Grid: B * wg_max * Hkv workgroups; workgroup i * Hkv + g takes entry i of the step's
// work list (row b, page range j) and KV head g, so the workgroups with work come first,
// in one round when they fit, and the rest exit at once; kAttnDecWaves * 64 threads.
// A range is one or more groups of PG pages (the list's pages per workgroup); the waves
// take PW pages of each group with all of their loads in flight at once (two waves per
// SIMD), the next group's block-table entries loaded meanwhile.
template <int KVDT, int D, bool FUSED>
__global__ __launch_bounds__(kAttnDecWaves * 64, KVDT == KV_F32_T ? 2 : 3) void attn_decode_kernel(AttnParams p) {
  constexpr int W = kAttnDecWaves, PW = attn_dec_pages(KVDT), PG = W * PW;
  static_assert(PG <= 64, "one block-table entry per lane");
  constexpr int NS = D / 32;
  constexpr int kVecs = kMaxR + 2;  // query heads, then (decode layer) k and v
  constexpr int kVecPerWave = (kVecs + W - 1) / W;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int item = blockIdx.x / p.n_kv_heads, g = blockIdx.x - item * p.n_kv_heads;
  if (item >= (int)p.sched[0]) return;  // workgroup-uniform
  const u32x2 ent = *(const u32x2*)(p.sched + 2 + 2 * item);
  const int b = (int)(ent.x >> 16), j = (int)(ent.x & 0xFFFFu), ctx = (int)ent.y;
  const int bg = b * p.n_kv_heads + g;
  const int R = p.n_q_heads / p.n_kv_heads;
  const int n = lane & 15, kg = lane >> 4;

  __shared__ __attribute__((aligned(16))) float s_vec[kVecs][D];
  __shared__ __attribute__((aligned(16))) u16 s_p[W][KVDT == KV_Q8_T ? D / 32 : 1][16][16];
  __shared__ __attribute__((aligned(16))) uint8_t s_knew[D * 4 + 64];
  __shared__ __attribute__((aligned(16))) uint8_t s_vnew[D * 4 + 64];
  __shared__ float s_ml[W][2][kMaxR];
  __shared__ __attribute__((aligned(16))) float s_o[W][kMaxR][D];
  __shared__ uint32_t s_last;

  // ---- loads issued before anything waits: the block-table entries of the first group
  // (lane i: page pgw + i) and of the new token's page, and this wave's head vectors
  // (vector hh = wave + W i; lane < D/2 holds pair (da, db)) with the RoPE cosine and
  // sine of the lane's pair and the QK-norm gains
  const int wpp = (int)p.sched[1];  // pages per workgroup, a multiple of PG
  const int32_t* btrow = p.block_table + (size_t)b * p.max_blocks;
  const int pgw = j * wpp;  // the workgroup's first page
  int bt_lane = btrow[min(pgw + (lane < PG ? lane : 0), p.max_blocks - 1)];
  const int new_page = ctx / kPage, new_slot = ctx % kPage;
  const int new_pg_id = FUSED ? btrow[new_page] : 0;
  const bool act = lane < D / 2;
  int da = 0, db = 0;
  pair_dims(act ? lane : 0, D, p.rope_style, da, db);
  const int nh = R + (FUSED ? 2 : 0);
  float va[kVecPerWave], vb[kVecPerWave];
#pragma unroll
  for (int i = 0; i < kVecPerWave; ++i) {
    const int hh = wave + W * i;
    va[i] = 0.f;
    vb[i] = 0.f;
    if (hh < nh && act) {
      const float* src;
      if constexpr (FUSED) {
        // hh < R: query head g R + hh; hh == R: k of head g; hh == R + 1: v of head g
        const int off = hh < R ? (g * R + hh) * D : hh == R ? p.q_dim + g * D : p.q_dim + p.kv_dim + g * D;
        src = p.qkv + (size_t)b * p.qkv_ld + off;
      } else {
        src = p.q + ((size_t)b * p.n_q_heads + g * R + hh) * D;
      }
      va[i] = src[da];
      vb[i] = src[db];
    }
  }
  double cs = 1.0, sn = 0.0;
  float gqa = 1.f, gqb = 1.f, gka = 1.f, gkb = 1.f;
  if (FUSED && act) {
    cs = p.rope[((size_t)b * (D / 2) + lane) * 2];
    sn = p.rope[((size_t)b * (D / 2) + lane) * 2 + 1];
    if (p.q_norm) {
      gqa = p.q_norm[da];
      gqb = p.q_norm[db];
      gka = p.k_norm[da];
      gkb = p.k_norm[db];
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  const int n_tok = FUSED ? ctx + 1 : ctx;
  const int n_pages = (n_tok + kPage - 1) / kPage;
  const int nwg = (n_pages + wpp - 1) / wpp;
  const int ngrp = (min(wpp, n_pages - pgw) + PG - 1) / PG;  // >= 1

  const int HB = kv_head_bytes_t<KVDT>(D);
  const size_t page_bytes = (size_t)HB * p.n_kv_heads;
  const uint8_t* kbase = (const uint8_t*)p.k_pages + (size_t)g * HB;
  const uint8_t* vbase = (const uint8_t*)p.v_pages + (size_t)g * HB;
  // Every wave issues all PW page loads of a group unconditionally, so the compiler's
  // count of loads in flight stays exact (a conditional load makes it wait for older
  // loads at the join): a slot past the row's pages re-reads the row's last page (an L2
  // hit: the waves of a workgroup share a CU) and is never used.
  PageRegs<KVDT, D> r[PW];
  auto load_group = [&](int gp) {  // gp: the group's first page; bt_lane holds its entries
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const u32 pg = (u32)__builtin_amdgcn_readlane(bt_lane, min(wave * PW + i, n_pages - 1 - gp));
      load_page<KVDT, D>(r[i], kbase + (size_t)pg * page_bytes, vbase + (size_t)pg * page_bytes, lane);
    }
  };
  // block-table entries of the group at gp (clamped into the row's table)
  auto load_bt = [&](int gp) { return btrow[min(gp + (lane < PG ? lane : 0), p.max_blocks - 1)]; };
  load_group(pgw);  // in flight during the set-up
  int bt_next = load_bt(pgw + (ngrp > 1 ? PG : 0));  // the next group's entries
  __builtin_amdgcn_sched_barrier(0);

  // ---- set-up: QK-norm and RoPE (rotation in fp64) of the head vectors, to LDS
#pragma unroll
  for (int i = 0; i < kVecPerWave; ++i) {
    const int hh = wave + W * i;
    if (hh < nh) {
      float a = va[i], bb = vb[i];
      if (FUSED && hh <= R) {
        if (p.q_norm) {  // per-head RMSNorm over the D dims (the lanes' pairs)
          float ss = act ? a * a + bb * bb : 0.0f;
          ss = wave_sum(ss);
          const float rn = 1.0f / sqrtf(ss / (float)D + p.eps);
          a = a * rn * (hh < R ? gqa : gka);
          bb = bb * rn * (hh < R ? gqb : gkb);
        }
        // RoPE: rotation by the pair's angle at the row's position, in fp64
        const double ad = a, bd = bb;
        a = (float)(ad * cs - bd * sn);
        bb = (float)(ad * sn + bd * cs);
      }
      if (act) {
        s_vec[hh][da] = a;
        s_vec[hh][db] = bb;
      }
    }
  }
  for (int idx = lane; idx < (int)sizeof(s_p[0]) / 2; idx += 64) (&s_p[wave][0][0][0])[idx] = 0;
  __syncthreads();

  // Q fragments in registers: lane (m = 2h + part, k) of slice s holds dims
  // 32s + 8k + pos(i), i < 8, of head h as f16 hi (part 0) or lo (part 1) of
  // q * scale * log2 e; rows m >= 2R are zero.  pos is the identity, or perm8 for the
  // q8_0 K layout.
  u32x4 qf[NS];
  {
    const float qscale = p.scale * 1.4426950408889634f;
    const int m = lane & 15, k = lane >> 4;
    const bool live_m = m < 2 * R;
    const int hq = live_m ? m >> 1 : 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const f32x4 x0 = *(const f32x4*)&s_vec[hq][32 * s + 8 * k];
      const f32x4 x1 = *(const f32x4*)&s_vec[hq][32 * s + 8 * k + 4];
      const float xv[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      u16 hv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = xv[KVDT == KV_Q8_T ? perm8(i) : i] * qscale;
        const u16 h = f2h(x);
        hv[i] = !live_m ? (u16)0 : (m & 1) ? f2h(x - h2f(h)) : h;
      }
      qf[s] = u32x4{(u32)hv[0] | ((u32)hv[1] << 16), (u32)hv[2] | ((u32)hv[3] << 16),
                    (u32)hv[4] | ((u32)hv[5] << 16), (u32)hv[6] | ((u32)hv[7] << 16)};
    }
  }
  // decode layer: the wave whose pages hold the new token's stores its K and V at slot
  // ctx % 16 and substitutes the stored values when it reads that page (no wave reads
  // the slot from memory)
  const bool owner = FUSED && new_page >= pgw && new_page < pgw + wpp && ((new_page - pgw) % PG) / PW == wave;
  if (owner) {
    const size_t pg = (u32)new_pg_id;
    uint8_t* kdst = (uint8_t*)p.k_pages + pg * page_bytes + (size_t)g * HB;
    uint8_t* vdst = (uint8_t*)p.v_pages + pg * page_bytes + (size_t)g * HB;
    store_token<KVDT>(s_vec[R], s_knew, kdst, false, D, new_slot, lane);
    store_token<KVDT>(s_vec[R + 1], s_vnew, vdst, true, D, new_slot, lane);
    wave_lds_fence();
  }

  // ---- the wave's pages, group by group
  SmState<D> st;
  st.m[0] = st.m[1] = -INFINITY;
  st.l[0] = st.l[1] = 0.f;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) st.O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool live = 2 * kg < R;  // this lane group holds real heads
  // Every group but the workgroup's last: software-pipelined.  Each page's registers are
  // refilled with the next group's page as soon as the page is consumed, so the next
  // group's loads overlap this group's math.  The entries of the group after next are
  // requested first, so reading them later waits for no page load.  All pages of these
  // groups hold context.
  for (int k = 0; k + 1 < ngrp; ++k) {
    const int w0 = pgw + k * PG + wave * PW;  // this wave's first page of the group
    const int nbt = bt_next;                  // entries of group k + 1
    const int gp = pgw + (k + 1) * PG;
    bt_next = load_bt(gp + (k + 2 < ngrp ? PG : 0));
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int pg = w0 + i;
      if (FUSED && owner && pg == new_page) patch_page<KVDT, D>(r[i], s_knew, s_vnew, new_slot, lane);
      dec_page<KVDT, D>(r[i], min(kPage, n_tok - pg * kPage), qf, s_p[wave], lane, live, st);
      // the refill stays behind the page's math (hoisted, it would need a second set
      // of page registers)
      __builtin_amdgcn_sched_barrier(0);
      const u32 npg = (u32)__builtin_amdgcn_readlane(nbt, min(wave * PW + i, n_pages - 1 - gp));
      load_page<KVDT, D>(r[i], kbase + (size_t)npg * page_bytes, vbase + (size_t)npg * page_bytes, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  {  // the last group (pages past the row's end are skipped)
    const int w0 = pgw + (ngrp - 1) * PG + wave * PW;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int pg = w0 + i;
      if (pg < n_pages) {
        if (FUSED && owner && pg == new_page) patch_page<KVDT, D>(r[i], s_knew, s_vnew, new_slot, lane);
        dec_page<KVDT, D>(r[i], min(kPage, n_tok - pg * kPage), qf, s_p[wave], lane, live, st);
      }
    }
  }

  // ---- the waves' states combine in LDS
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int hq = 2 * kg + e;
    if (hq < R) {
      if (n == 0) {
        s_ml[wave][0][hq] = st.m[e];
        s_ml[wave][1][hq] = st.l[e];
      }
#pragma unroll
      for (int t = 0; t < D / 16; ++t) s_o[wave][hq][16 * t + n] = st.O[t][2 * e] + st.O[t][2 * e + 1];
    }
  }
  __syncthreads();

  auto put = [&](int hq, int d, float v) {
    const int h = g * R + hq;
    if (p.out) p.out[((size_t)b * p.n_q_heads + h) * D + d] = v;
    if (p.pack) actpack_put(p.pack, p.pack_kind, p.pack_nslices, b, h * D + d, v);
  };
  const size_t part_stride = (size_t)R * (D + 2);
  float* part = p.wg_part + (size_t)bg * p.wg_max * part_stride;  // this (row, KV head)'s partials
  for (int idx = tid; idx < R * D; idx += W * 64) {
    const int hq = idx / D, d = idx - hq * D;
    float M = s_ml[0][0][hq];  // finite: wave 0 has a page
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, s_ml[w][0][hq]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float sc = exp2f(s_ml[w][0][hq] - M);  // 0 for a wave without pages
      L = __builtin_fmaf(s_ml[w][1][hq], sc, L);
      O = __builtin_fmaf(s_o[w][hq][d], sc, O);
    }
    if (nwg == 1) {
      put(hq, d, O * (1.0f / L));
    } else {
      float* pj = part + (size_t)j * part_stride;
      st_agent(pj + idx, O);
      if (d == 0) {
        st_agent(pj + R * D + hq, M);
        st_agent(pj + R * D + R + hq, L);
      }
    }
  }
  if (nwg == 1) return;

  // ---- arrival: the stores above complete before the count; the last arriver merges
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) s_last = __hip_atomic_fetch_add(p.wg_cnt + bg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_last != (uint32_t)(nwg - 1)) return;

  // Online log-sum-exp over the partials in workgroup order, the loads of kMerge of them
  // issued at once (one memory round trip for up to kMerge partials).
  constexpr int kMerge = 16;
  for (int idx = tid; idx < R * D; idx += W * 64) {
    const int hq = idx / D, d = idx - hq * D;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int j0 = 0; j0 < nwg; j0 += kMerge) {
      float mj[kMerge], lj[kMerge], oj[kMerge];
#pragma unroll
      for (int q = 0; q < kMerge; ++q) {
        const float* pj = part + (size_t)min(j0 + q, nwg - 1) * part_stride;
        mj[q] = ld_agent(pj + R * D + hq);
        lj[q] = ld_agent(pj + R * D + R + hq);
        oj[q] = ld_agent(pj + idx);
      }
#pragma unroll
      for (int q = 0; q < kMerge; ++q) {
        if (j0 + q < nwg) {
          const float Mn = fmaxf(M, mj[q]);
          const float so = exp2f(M - Mn), sj = exp2f(mj[q] - Mn);  // so = 0 while M = -inf
          L = __builtin_fmaf(L, so, lj[q] * sj);
          O = __builtin_fmaf(O, so, oj[q] * sj);
          M = Mn;
        }
      }
    }
    put(hq, d, O * (1.0f / L));
  }
  if (tid == 0) __hip_atomic_store(p.wg_cnt + bg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int attn_dec_slots(int kv_dtype) {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                hipSuccess && n > 0)
      return n;
    (void)hipGetLastError();
    return 256;
  }();
  return cus * (kv_dtype == KV_Q8_T ? 3 : 2);
}

AttnDecPlan plan_attn_dec(int kv_dtype, int max_tokens) {
  AttnDecPlan pl{};
  pl.wg_pages = kAttnDecWaves * attn_dec_pages(kv_dtype);
  const long long pages = ((long long)(max_tokens > 0 ? max_tokens : 1) + kPage - 1) / kPage;
  const long long w = (pages + pl.wg_pages - 1) / pl.wg_pages;
  pl.wg_max = w > kAttnDecMaxWg ? 0 : (int)w;
  return pl;
}

size_t attn_dec_part_floats(int B, int n_q_heads, int head_dim, int wg_max) {
  return (size_t)B * n_q_heads * wg_max * (head_dim + 2);
}

__global__ __launch_bounds__(1024) void attn_sched_kernel(AttnSched sc) {
  __shared__ uint32_t scan[kSchedScratchWords];
  build_attn_sched(sc, scan);
}

hipError_t launch_attn_sched(const AttnSched& sc, hipStream_t st) {
  launch_kernel(attn_sched_kernel, dim3(1), dim3(1024), 0, st, sc);
  return hipGetLastError();
}

hipError_t launch_attn_decode(int kv_dtype, bool fused, const AttnParams& p, hipStream_t st) {
  if (p.wg_max < 1 || p.wg_max > kAttnDecMaxWg || p.n_q_heads / p.n_kv_heads > kMaxR || !p.wg_cnt ||
      (p.wg_max > 1 && !p.wg_part) || (!p.out && !p.pack) || p.wg_pages != kAttnDecWaves * attn_dec_pages(kv_dtype) ||
      !p.sched || p.B > 65535)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((size_t)p.B * p.n_kv_heads * p.wg_max)), block(kAttnDecWaves * 64);
#define GR_AD(KV, DD, FU) launch_kernel(attn_decode_kernel<KV, DD, FU>, grid, block, 0, st, p)
#define GR_ADD(KV, FU)   \
  if (p.head_dim == 128) \
    GR_AD(KV, 128, FU);  \
  else                   \
    GR_AD(KV, 64, FU);
#define GR_ADK(FU)             \
  if (kv_dtype == 0) {         \
    GR_ADD(KV_F32_T, FU)       \
  } else if (kv_dtype == 1) {  \
    GR_ADD(KV_F16_T, FU)       \
  } else {                     \
    GR_ADD(KV_Q8_T, FU)        \
  }
  if (fused) {
    GR_ADK(true)
  } else {
    GR_ADK(false)
  }
#undef GR_ADK
#undef GR_ADD
#undef GR_AD
  return hipGetLastError();
}

}  // namespace gr
