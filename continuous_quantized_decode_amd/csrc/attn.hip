// attn.hip -- split-context paged GQA decode attention on gfx950.
//
// Each row keeps its own attention over its own pages (Leone, intro; tinyllm, Status:
// a physical page pool addressed through a logical block table per sequence).
// Instead of gathering pages into contiguous K/V (the reference path tinyllm
// describes under Known limitations), every wave walks the block table directly.
//
// Work unit: one wave per (row b, KV head g, split s); split s covers a page-aligned
// range of the row's context.  Per page (16 tokens):
//   scores  S[m][t] = sum_d Q[m][d] K[t][d]  -- v_mfma_f32_16x16x32_f16, A = the R query
//           heads of group g as f16 hi/lo rows (m = 2h + part), B = the page's K
//   softmax online in the log2 domain (q is pre-scaled by scale*log2 e); running max
//           and sum over the 16 tokens by lane shuffles inside each 16-lane group
//   output  O[m][d] += P[m][t] V[t][d]        -- v_mfma_f32_16x16x16_f16, A = P as f16
//           hi/lo rows (transposed through LDS), B = the page's V (dim-major pages)
// q8_0 pages are expanded to exact f16 integers in registers; their per-token,
// per-32-element scales multiply the K scores (K) or fold into P (V).  f32 pages are
// split into f16 hi/lo operands.  Partials (unnormalized O, running max m, sum l)
// are merged across splits by log-sum-exp in attn_merge_kernel.
//
// The fused variant (used by the decode layer) also reads q, k, v from the QKV
// GEMM's output, applies QK-RMSNorm and RoPE (fp64 angles, one table per step), stores the new token's K/V
// at slot ctx%16 of page block_table[b][ctx/16] in the pool's format, and
// substitutes those stored values for the slot's contents when it reads that page.
#include "gr_internal.h"
#include "attn_internal.h"
#include "kvpage.h"
#include "attn_dev.h"

namespace gr {

// ------------------------------------------------------------------- the kernel

// Three waves per SIMD (registers <= 168) with a chunk of pages in flight: two f16 pages
// or four q8_0 pages; f32 pages (two in flight) need more registers.
template <int KVDT, int D, bool FUSED>
__global__ __launch_bounds__(64, KVDT == KV_F32_T ? 2 : 3) void attn_split_kernel(AttnParams p) {
  constexpr int NS = D / 32;  // QK slices
  constexpr int NT = D / 16;  // PV tiles
  const int lane = threadIdx.x;
  const int unit = blockIdx.x;
  const int split = unit % p.max_splits;
  const int bg = unit / p.max_splits;
  const int g = bg % p.n_kv_heads;
  const int R = p.n_q_heads / p.n_kv_heads;
  const int pg0 = split * p.pages_per_split;
  const int n = lane & 15, kg = lane >> 4;

  // Row groups: rows are taken P at a time (P = 1 in the fused layer).  When a group's
  // rows belong to one sequence, the unit of its first row takes them through the pages
  // together, their R P query heads side by side in the MFMA rows (R P <= 8), so each
  // page is read once for all of them, each row masked to its own token count, and the
  // other rows' units have nothing to do; otherwise every row's unit takes its own row.
  const int P = FUSED ? 1 : (p.rows_per_unit > 0 ? p.rows_per_unit : 1);
  const int brow = bg / p.n_kv_heads;
  const int b0 = brow - brow % P;
  const int nr = min(P, p.B - b0);
  bool together = true;
  if constexpr (!FUSED) {
    int seq0, pos0;
    attn_row_place(p, b0, seq0, pos0);
    for (int r = 1; r < nr; ++r) {
      int sr, pr;
      attn_row_place(p, b0 + r, sr, pr);
      together = together && sr == seq0;
    }
  }

  __shared__ __attribute__((aligned(16))) float s_vec[10][128];  // head vectors, linear layout
  __shared__ __attribute__((aligned(16))) u16 s_p[KVDT == KV_Q8_T ? D / 32 : 1][16][16];  // P transpose
  __shared__ __attribute__((aligned(16))) uint8_t s_knew[D * 4 + 64];
  __shared__ __attribute__((aligned(16))) uint8_t s_vnew[D * 4 + 64];

  // rows b .. b + nrows - 1 of one sequence
  auto run = [&](const int b, const int nrows) {
  int seq, ctx;  // the first row's sequence and position
  attn_row_place(p, b, seq, ctx);
  const int nq = R * nrows;  // query head vectors (MFMA row pairs) in use
  // token counts of the rows of this lane's two MFMA row pairs (head vectors 2 kg, 2 kg + 1)
  int ntok_e[2] = {0, 0};
  int n_tok = 0;  // the most tokens any row attends to
  if constexpr (FUSED) {
    n_tok = ctx + 1;
    ntok_e[0] = ntok_e[1] = n_tok;
  } else {
    for (int r = 0; r < nrows; ++r) {
      int sr, pr;
      attn_row_place(p, b + r, sr, pr);
      const int t = pr + p.self_in_pool;
      n_tok = max(n_tok, t);
      if ((2 * kg) / R == r) ntok_e[0] = t;
      if ((2 * kg + 1) / R == r) ntok_e[1] = t;
    }
  }
  const int32_t* bt = p.block_table + (size_t)seq * p.max_blocks;

  // ---- loads issued before anything waits: the row's context length, the page ids
  // of the split's first 64 pages (lane i: page pg0 + i; ids past the row's pages are
  // never used), the head vectors (q of the R heads; k and v of head g as well in the
  // fused layer), pairs (da, db) per lane, and the RoPE cosine and sine of the lane's
  // pair at the row's new position (computed in fp64 once per step)
  constexpr int kMaxHeads = 10;  // R P <= 8 query heads, then k and v
  int bt_chunk = pg0;
  int bt_lane = pg0 + lane < p.max_blocks ? bt[pg0 + lane] : 0;
  const bool act = lane < D / 2;
  int da = 0, db = 0;
  pair_dims(act ? lane : 0, D, p.rope_style, da, db);
  const int nh = nq + (FUSED ? 2 : 0);
  double cs = 1.0, sn = 0.0;
  if (FUSED && act) {
    cs = p.rope[((size_t)b * (D / 2) + lane) * 2];
    sn = p.rope[((size_t)b * (D / 2) + lane) * 2 + 1];
  }
  float va[kMaxHeads], vb[kMaxHeads];
#pragma unroll
  for (int hh = 0; hh < kMaxHeads; ++hh) {
    va[hh] = 0.f;
    vb[hh] = 0.f;
    if (hh < nh && act) {
      const float* src;
      if (FUSED) {
        // hh < R: query head g*R + hh; hh == R: k of head g; hh == R+1: v of head g
        const int off = hh < R ? (g * R + hh) * D : hh == R ? p.q_dim + g * D : p.q_dim + p.kv_dim + g * D;
        src = p.qkv + (size_t)b * p.qkv_ld + off;
      } else {
        src = p.q + ((size_t)(b + hh / R) * p.n_q_heads + g * R + hh % R) * D;
      }
      va[hh] = src[da];
      vb[hh] = src[db];
    }
  }

  const int n_pages = (n_tok + kPage - 1) / kPage;
  if (pg0 >= n_pages) return;
  const int pg1 = min(n_pages, pg0 + p.pages_per_split);

  const int HB = kv_head_bytes_t<KVDT>(D);
  const size_t page_bytes = (size_t)HB * p.n_kv_heads;
  const int new_page = ctx / kPage, new_slot = ctx % kPage;
  const bool owner = FUSED && new_page >= pg0 && new_page < pg1;
  const uint8_t* kbase = (const uint8_t*)p.k_pages + (size_t)g * HB;
  const uint8_t* vbase = (const uint8_t*)p.v_pages + (size_t)g * HB;

  // page j's id: from the lanes' chunk (wave-uniform read), reloaded every 64 pages
  auto page_id = [&](int j) -> size_t {
    if (j - bt_chunk >= 64) {
      bt_chunk = pg0 + ((j - pg0) & ~63);
      bt_lane = bt_chunk + lane < p.max_blocks ? bt[bt_chunk + lane] : 0;
    }
    return (size_t)(u32)__builtin_amdgcn_readlane(bt_lane, j - bt_chunk);
  };
  auto load = [&](PageRegs<KVDT, D>& r, int j) {
    const size_t pg = page_id(j);
    load_page<KVDT, D>(r, kbase + pg * page_bytes, vbase + pg * page_bytes, lane);
  };
  // Pages go in chunks of NP, all of a chunk's loads in flight at once (as many as the
  // registers of three waves per SIMD allow); the first chunk is in flight during the
  // setup below.
  constexpr int NP = KVDT == KV_Q8_T ? (FUSED ? 4 : 2) : 2;  // the standalone kernel's extra row state
  PageRegs<KVDT, D> r[NP];
  auto issue_chunk = [&](int c0) {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (c0 + i < pg1) load(r[i], c0 + i);
  };
  issue_chunk(pg0);

  // ---- QK-norm and RoPE (rotation in fp64) of the head vectors, to LDS -------------
  {
#pragma unroll
    for (int hh = 0; hh < kMaxHeads; ++hh) {
      if (hh < nh) {
        float a = va[hh], bb = vb[hh];
        if (FUSED && hh <= R) norm_rope(a, bb, act, hh < R ? p.q_norm : p.k_norm, p.eps, D, da, db, cs, sn);
        if (act) {
          s_vec[hh][da] = a;
          s_vec[hh][db] = bb;
        }
      }
    }
  }
  __syncthreads();

  // Q fragments in registers: lane (m = 2h + part, k) of slice s holds dims
  // 32s + 8k + pos(i), i < 8, of head h as f16 hi (part 0) or lo (part 1) of
  // q * scale * log2 e; rows m >= 2R are zero.  pos is the identity, or perm8 for the
  // q8_0 K layout.
  u32x4 qf[NS];
  {
    const float qscale = p.scale * 1.4426950408889634f;
    const int m = lane & 15, k = lane >> 4;
    const bool live_m = m < 2 * nq;
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
    for (int idx = lane; idx < (int)sizeof(s_p) / 2; idx += 64) (&s_p[0][0][0])[idx] = 0;
  }
  if (owner) {
    const size_t pg = (size_t)bt[new_page];
    uint8_t* kdst = (uint8_t*)p.k_pages + pg * page_bytes + (size_t)g * HB;
    uint8_t* vdst = (uint8_t*)p.v_pages + pg * page_bytes + (size_t)g * HB;
    store_token<KVDT>(s_vec[R], s_knew, kdst, false, D, new_slot, lane);
    store_token<KVDT>(s_vec[R + 1], s_vnew, vdst, true, D, new_slot, lane);
  }
  __syncthreads();

  // ---- page loop -------------------------------------------------------------------
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  f32x4 O[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One page: scores, online softmax, P transpose, PV.
  auto page = [&](PageRegs<KVDT, D>& cur, int j) {
    if (FUSED && owner && j == new_page) patch_page<KVDT, D>(cur, s_knew, s_vnew, new_slot, lane);
    const int valid = min(kPage, n_tok - j * kPage);  // of the row with the most tokens
    const int valid_e[2] = {FUSED ? valid : min(kPage, ntok_e[0] - j * kPage),
                            FUSED ? valid : min(kPage, ntok_e[1] - j * kPage)};
    if constexpr (KVDT != KV_Q8_T) {
      // slots past the context may hold anything (NaN included): zero their V so
      // that 0 * V stays 0 in the PV product
      if (valid < kPage) mask_v_tail<KVDT, D>(cur, valid, lane);
    }

    // scores
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
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
    float sv[2], pv[2], alpha[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      sv[e] = n < valid_e[e] ? sc[2 * e] + sc[2 * e + 1] : -INFINITY;
      float mx = sv[e];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float mnew = fmaxf(m_run[e], mx);
      // a row with no token yet (its tokens start on a later page) keeps m = -inf and
      // l = 0: scale against 0 instead of -inf so nothing becomes NaN
      const float mref = (!FUSED && mnew == -INFINITY) ? 0.f : mnew;
      alpha[e] = exp2f(m_run[e] - mref);
      pv[e] = exp2f(sv[e] - mref);
      float ps = pv[e];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o, 64);
      l_run[e] = l_run[e] * alpha[e] + ps;
      m_run[e] = mnew;
    }
    // P (f16 hi/lo rows) to LDS, transposed to the PV A layout
    const bool live = 2 * kg < nq;  // this lane group holds real heads
    if constexpr (KVDT == KV_Q8_T) {
      const int col = 4 * (n >> 2) + perm4(n & 3);
#pragma unroll
      for (int blk = 0; blk < D / 32; ++blk) {
        const u32 w = cur.vsc[blk >> 1];
        const float vs = h2f((u16)((blk & 1) ? (w >> 16) : (w & 0xFFFF)));
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x = n < valid_e[e] ? pv[e] * vs : 0.0f;
          const u16 h = f2h(x);
          if (live) {
            s_p[blk][4 * kg + 2 * e][col] = h;
            s_p[blk][4 * kg + 2 * e + 1][col] = f2h(x - h2f(h));
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const u16 h = f2h(pv[e]);
        if (live) {
          s_p[0][4 * kg + 2 * e][n] = h;
          s_p[0][4 * kg + 2 * e + 1][n] = f2h(pv[e] - h2f(h));
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      O[t][0] *= alpha[0];
      O[t][1] *= alpha[0];
      O[t][2] *= alpha[1];
      O[t][3] *= alpha[1];
    }
    if constexpr (KVDT == KV_Q8_T) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x2 pa = *(const u32x2*)&s_p[t >> 1][n][4 * kg];
        O[t] = mfma_f16_k16(pa, q8_to_f16x4(cur.v[t]), O[t]);
      }
    } else {
      const u32x2 pa = *(const u32x2*)&s_p[0][n][4 * kg];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (KVDT == KV_F16_T) {
          O[t] = mfma_f16_k16(pa, cur.v[t], O[t]);
        } else {
          u32x2 hi, lo;
          f32_to_f16hl(cur.v[t], hi, lo);
          O[t] = mfma_f16_k16(pa, hi, O[t]);
          O[t] = mfma_f16_k16(pa, lo, O[t]);
        }
      }
    }
    __syncthreads();
  };

  // The split's pages, chunk by chunk (the first chunk already in flight).
  for (int c0 = pg0; c0 < pg1; c0 += NP) {
    if (c0 != pg0) issue_chunk(c0);
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (c0 + i < pg1) page(r[i], c0 + i);
  }

  // ---- partial results: for each row with tokens in this split ----------------------
  if (2 * kg < nq) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int hq = 2 * kg + e;
      if (hq >= nq) break;
      if (!FUSED && pg0 * kPage >= ntok_e[e]) continue;  // the row ends before this split
      const int h = g * R + hq % R;
      const size_t base = ((size_t)(b + hq / R) * p.n_q_heads + h) * p.max_splits + split;
#pragma unroll
      for (int t = 0; t < NT; ++t) p.o_part[base * D + 16 * t + n] = O[t][2 * e] + O[t][2 * e + 1];
      if (n == 0) {
        p.m_part[base] = m_run[e];
        p.l_part[base] = l_run[e];
      }
    }
  }
  };  // run

  if (FUSED || !together) {
    run(brow, 1);
  } else if (brow == b0) {
    run(b0, nr);
  }
}

// ----------------------------------------------------------------------- merge
// Per (row b, query head h): M = max_s m_s, L = sum_s l_s 2^(m_s - M),
// o = sum_s o_s 2^(m_s - M) / L (the partials are in the log2 domain).  Writes f32
// out [B][Hq][D] and/or the actpack of the output projection (K = Hq*D, `kind`).
// Wave w takes splits w, w + 4, w + 8, ...: it issues the loads of up to kMergeChunk
// of its splits (m, l and the o vectors) at once, so the common case costs one memory
// round trip, and folds them into its running (M_w, L_w, o_w); the four waves' results
// combine through LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeChunk = 16;  // splits per wave and round of loads
constexpr int kMergeMaxSplits = 1024;

__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnParams p, float* out, uint16_t* pack,
                                                                   int kind, int nslices, int fused) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x;
  const int h = bh % p.n_q_heads, b = bh / p.n_q_heads;
  const int D = p.head_dim;  // 64 or 128: dims lane and lane + 64
  int seq, ctx;
  attn_row_place(p, b, seq, ctx);
  const int n_tok = fused ? ctx + 1 : ctx + p.self_in_pool;
  const int n_pages = (n_tok + kPage - 1) / kPage;
  const int S = min((n_pages + p.pages_per_split - 1) / p.pages_per_split, p.max_splits);
  const size_t base = ((size_t)b * p.n_q_heads + h) * p.max_splits;
  __shared__ float s_m[kMergeWaves], s_l[kMergeWaves];
  __shared__ float s_o[kMergeWaves][128];

  float Mw = -INFINITY, Lw = 0.f, ow[2] = {0.f, 0.f};
  for (int c0 = 0; c0 < S; c0 += kMergeWaves * kMergeChunk) {
    // lane j < kMergeChunk holds m and l of split c0 + wave + 4 j
    const int sl = c0 + wave + kMergeWaves * lane;
    float ml = -INFINITY, ll = 0.f;
    if (lane < kMergeChunk && sl < S) {
      ml = p.m_part[base + sl];
      ll = p.l_part[base + sl];
    }
    float ov[kMergeChunk][2];
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      const int sj = c0 + wave + kMergeWaves * j;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        ov[j][i] = (sj < S && 64 * i < D) ? p.o_part[(base + sj) * D + 64 * i + lane] : 0.f;
    }
    const float Mn = fmaxf(Mw, wave_max(ml));
    if (Mn == -INFINITY) continue;  // no split of this wave yet (wave-uniform)
    const float rs = exp2f(Mw - Mn);  // 0 while Mw is -inf
    const float e = exp2f(ml - Mn);   // 0 for lanes without a split
    Lw = __builtin_fmaf(Lw, rs, wave_sum(ll * e));
    ow[0] *= rs;
    ow[1] *= rs;
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      const float ej = __shfl(e, j, 64);
      ow[0] = __builtin_fmaf(ov[j][0], ej, ow[0]);
      ow[1] = __builtin_fmaf(ov[j][1], ej, ow[1]);
    }
    Mw = Mn;
  }
  if (lane == 0) {
    s_m[wave] = Mw;
    s_l[wave] = Lw;
  }
  s_o[wave][lane] = ow[0];
  s_o[wave][64 + lane] = ow[1];
  __syncthreads();
  if (tid < D) {
    float M = s_m[0];  // finite: wave 0 holds split 0
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, s_m[w]);
    float L = 0.f, v = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) {
      const float sc = s_m[w] == -INFINITY ? 0.f : exp2f(s_m[w] - M);
      L = __builtin_fmaf(s_l[w], sc, L);
      v = __builtin_fmaf(s_o[w][tid], sc, v);
    }
    v *= 1.0f / L;
    if (out) out[((size_t)b * p.n_q_heads + h) * D + tid] = v;
    if (pack) actpack_put(pack, kind, nslices, b, h * D + tid, v);
  }
}

// ------------------------------------------------------------------------ launch

// ------------------------------------------------------------ several tokens per row
//
// When a step carries several tokens of a sequence (tokens_per_seq > 1, or rows placed
// by row_seq / row_pos), a row's
// attention must see the tokens before it in the same step, so every row's K/V is
// stored first: one wave per (row, KV head) applies QK-norm and RoPE (the fused
// variant's set-up), stores K and V at the row's position and writes the roped query
// heads; the standalone attention kernel then runs with self_in_pool set.
template <int KVDT, int D>
__global__ __launch_bounds__(64) void attn_append_kernel(AttnParams p, float* q_out) {
  const int lane = threadIdx.x;
  const int g = blockIdx.x % p.n_kv_heads, b = blockIdx.x / p.n_kv_heads;
  const int R = p.n_q_heads / p.n_kv_heads;
  int seq, pos;
  attn_row_place(p, b, seq, pos);
  const bool act = lane < D / 2;
  int da = 0, db = 0;
  pair_dims(act ? lane : 0, D, p.rope_style, da, db);
  double cs = 1.0, sn = 0.0;
  if (act) {
    cs = p.rope[((size_t)b * (D / 2) + lane) * 2];
    sn = p.rope[((size_t)b * (D / 2) + lane) * 2 + 1];
  }
  __shared__ __attribute__((aligned(16))) float s_kv[2][128];
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[D * 4 + 64];
  const float* row = p.qkv + (size_t)b * p.qkv_ld;
  // query heads g*R .. g*R+R-1, then k, then v of head g
  for (int hh = 0; hh < R + 2; ++hh) {
    const int off = hh < R ? (g * R + hh) * D : hh == R ? p.q_dim + g * D : p.q_dim + p.kv_dim + g * D;
    float a = act ? row[off + da] : 0.f, bb = act ? row[off + db] : 0.f;
    if (hh <= R) norm_rope(a, bb, act, hh < R ? p.q_norm : p.k_norm, p.eps, D, da, db, cs, sn);
    if (hh < R) {
      if (act) {
        float* dst = q_out + ((size_t)b * p.n_q_heads + g * R + hh) * D;
        dst[da] = a;
        dst[db] = bb;
      }
    } else if (act) {
      s_kv[hh - R][da] = a;
      s_kv[hh - R][db] = bb;
    }
  }
  __syncthreads();
  const int HB = kv_head_bytes_t<KVDT>(D);
  const size_t page_bytes = (size_t)HB * p.n_kv_heads;
  const size_t pg = (size_t)p.block_table[(size_t)seq * p.max_blocks + pos / kPage];
  uint8_t* kdst = (uint8_t*)p.k_pages + pg * page_bytes + (size_t)g * HB;
  uint8_t* vdst = (uint8_t*)p.v_pages + pg * page_bytes + (size_t)g * HB;
  store_token<KVDT>(s_kv[0], s_stage, kdst, false, D, pos % kPage, lane);
  store_token<KVDT>(s_kv[1], s_stage, vdst, true, D, pos % kPage, lane);
}

hipError_t launch_attn_append(int kv_dtype, const AttnParams& p, float* q_out, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.B * p.n_kv_heads));
#define GR_AP(KV, DD) launch_kernel(attn_append_kernel<KV, DD>, grid, dim3(64), 0, st, p, q_out)
  if (kv_dtype == 0) {
    if (p.head_dim == 128) GR_AP(KV_F32_T, 128); else GR_AP(KV_F32_T, 64);
  } else if (kv_dtype == 1) {
    if (p.head_dim == 128) GR_AP(KV_F16_T, 128); else GR_AP(KV_F16_T, 64);
  } else {
    if (p.head_dim == 128) GR_AP(KV_Q8_T, 128); else GR_AP(KV_Q8_T, 64);
  }
#undef GR_AP
  return hipGetLastError();
}

AttnPlan plan_attn(int B, int n_kv_heads, int max_ctx_tokens) {
  // Enough (row, head, split) waves to fill the chip even when most rows are short:
  // about kAttnWaves waves at the longest context, at least kAttnMinPages pages per split.
  constexpr int kAttnWaves = 4096, kAttnMinPages = 4;  // measured: 2 or 8 pages per split are slower
  const int max_pages = (max_ctx_tokens + kPage - 1) / kPage;
  const long long units = (long long)B * n_kv_heads * (max_pages > 0 ? max_pages : 1);
  int pps = (int)((units + kAttnWaves - 1) / kAttnWaves);
  // many short rows (a prompt chunk) next to a few long ones (decode rows): the count
  // above assumes every row is as long as the longest and would leave the long rows a
  // handful of splits, each walking its pages alone; keep at least 16 splits for them
  const int long_rows_pps = (max_pages + 15) / 16;
  if (pps > long_rows_pps) pps = long_rows_pps;
  if (pps < kAttnMinPages) pps = kAttnMinPages;
  while ((max_pages + pps - 1) / pps > 1024) ++pps;  // the merge handles up to 1024 splits
  AttnPlan pl;
  pl.pages_per_split = pps;
  pl.max_splits = max_pages > 0 ? (max_pages + pps - 1) / pps : 1;
  return pl;
}

size_t attn_partial_floats(int B, int n_q_heads, int head_dim, const AttnPlan& pl) {
  return (size_t)B * n_q_heads * pl.max_splits * (head_dim + 2);
}

hipError_t launch_attn_split(int kv_dtype, bool fused, const AttnParams& p, hipStream_t st) {
  const int P = fused ? 1 : (p.rows_per_unit > 0 ? p.rows_per_unit : 1);
  if (P * (p.n_q_heads / p.n_kv_heads) > 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((size_t)p.B * p.n_kv_heads * p.max_splits));
#define GR_A(KV, DD, FU) launch_kernel(attn_split_kernel<KV, DD, FU>, grid, dim3(64), 0, st, p)
#define GR_AD(KV, FU)        \
  if (p.head_dim == 128)     \
    GR_A(KV, 128, FU);       \
  else                       \
    GR_A(KV, 64, FU);
#define GR_AK(FU)                  \
  if (kv_dtype == 0) {             \
    GR_AD(KV_F32_T, FU)            \
  } else if (kv_dtype == 1) {      \
    GR_AD(KV_F16_T, FU)            \
  } else {                         \
    GR_AD(KV_Q8_T, FU)             \
  }
  if (fused) {
    GR_AK(true)
  } else {
    GR_AK(false)
  }
#undef GR_AK
#undef GR_AD
#undef GR_A
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnParams& p, float* out, uint16_t* pack, int kind, int nslices, int fused,
                             hipStream_t st) {
  launch_kernel(attn_merge_kernel, dim3((unsigned)(p.B * p.n_q_heads)), dim3(kMergeThreads), 0, st, p, out, pack, kind,
                nslices, fused);
  return hipGetLastError();
}

}  // namespace gr
