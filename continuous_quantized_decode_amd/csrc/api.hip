// api.hip -- host side of libgr: argument validation, workspace carving, launch
// planning and the call sequences of the C ABI declared in include/gr.h.
//
// Every host-checkable condition is checked before the first launch, so a call
// that fails enqueues nothing.  The library keeps no per-row state: continuous
// batching (Leone, intro; tinyllm, Status: continuous admission, variable-length
// batched decode) is just a different B, block table and ctx_lens on the next call.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>

#include "gr_internal.h"
#include "attn_internal.h"

namespace gr {

thread_local ProbeEvents* probe_events = nullptr;


hipError_t launch_dequant(int kind, const void* blocks, int64_t n, float* out, hipStream_t st);
hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* out, hipStream_t st);
size_t sample_workspace_bytes(int B, int vocab);
hipError_t launch_spec_accept(const int32_t* sampled, const int32_t* draft, int B, int T, int32_t* n_accepted,
                              hipStream_t st);
int sample_max_vocab();
hipError_t launch_sample(const float* logits, int B, int vocab, const gr_sample_params* params, int32_t* tokens,
                         uint64_t* kept, void* ws, hipStream_t st);
hipError_t launch_gather(int kv_dtype, int D, const void* pool, int is_v, const int32_t* bt, const int32_t* ctx,
                         int B, int max_blocks, int n_kv_heads, int max_ctx, float* out, hipStream_t st);

namespace {

thread_local int t_last_hip_error = 0;
std::atomic<int> g_dev_state[64];  // 0 unknown, 1 gfx950, -1 other

gr_status check_launch(hipError_t e) {
  if (e != hipSuccess) {
    t_last_hip_error = (int)e;
    return GR_ERR_LAUNCH;
  }
  return GR_OK;
}

gr_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GR_ERR_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t pr;
    if (hipGetDeviceProperties(&pr, dev) != hipSuccess) return GR_ERR_DEVICE;
    st = std::strncmp(pr.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_dev_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? GR_OK : GR_ERR_DEVICE;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool wtype_ok(int t) { return t == GR_W_Q4_K || t == GR_W_Q6_K || t == GR_W_Q5_K || t == GR_W_Q8_0; }
bool kv_ok(int t) { return t == GR_KV_F32 || t == GR_KV_F16 || t == GR_KV_Q8_0; }

// Carves a caller-provided workspace into 256-byte aligned regions; with base ==
// nullptr it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <class T>
  T* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

// Both actpack kinds of B rows x K columns.
struct Pack2 {
  PackOut k32, k16;
  const PackOut& of(int wtype) const { return wtype == GR_W_Q6_K ? k16 : k32; }  // Q6_K: K=16 MFMA slices
};
Pack2 carve_pack2(Carver& c, int B, int K) {
  Pack2 p;
  p.k32.pack = c.take<u16>(actpack_bytes(B, K));
  p.k32.kind = kK32;
  p.k16.pack = c.take<u16>(actpack_bytes(B, K));
  p.k16.kind = kK16;
  return p;
}
const PackOut kNoPack{nullptr, 0};

int nslices_of(int kind, int K) { return kind == kK32 ? K / 32 : K / 16; }

// The kinds an input must be packed in for matrices of the given types.
struct Kinds {
  bool k32 = false, k16 = false;
  void add(int wtype) { (wtype == GR_W_Q6_K ? k16 : k32) = true; }
};

// GEMM epilogue parameters shared by one call of gemm_run.
struct Epi {
  int kind = kEpiStore;
  float* y = nullptr;
  int ldy = 0;
  const double* ss = nullptr;  // RMSNorm sum of squares of the input rows (NULL: none)
  float eps = 0.f;
  const float* gain = nullptr;
  PackOut out1 = kNoPack, out2 = kNoPack;
  int out_k = 0;  // K of the packed outputs (columns of y)
  double* ss_out = nullptr;
  double* zero_ptr = nullptr;
  int zero_n = 0;
  float* part = nullptr;  // many-row K-split partial sums (NULL: no split)
  size_t part_cap = 0;
};

// y (= the epilogue's destination) for up to three matrices sharing K and the input
// pack, split into one launch per weight type (outputs stay column-contiguous).
hipError_t gemm_run(const void* const* w, const int* types, const int* rows, int nmat, int K, int B,
                    const Pack2& xin, const Epi& ep, hipStream_t st) {
  int col = 0;
  int i = 0;
  bool zeroed = false;
  while (i < nmat) {
    GemmArgs a{};
    const int col_begin = col;
    int j = i, n = 0, tiles = 0, all_tiles = 0;
    for (int q = i; q < nmat && types[q] == types[i]; ++q) all_tiles += (rows[q] + 15) / 16;
    // many rows: the 2-D tiled kernel; many tiles and a plain store: the tile-loop
    // kernel (one tile per group)
    int type_cols = 0;
    for (int q = i; q < nmat && types[q] == types[i]; ++q) type_cols += rows[q];
    // (the whole-tile kernel also takes residual updates: Wo)
    const bool tl = !use_mm(types[i], B) &&
                    ((ep.kind == kEpiStore && use_tile_loop(types[i], all_tiles, K, B)) ||
                     ((ep.kind == kEpiStore || ep.kind == kEpiResidual) && use_tile_loop_whole(types[i], all_tiles, K, B)));
    const bool mm = !tl && (ep.kind == kEpiStore ? use_mm_store(types[i], B, type_cols) : use_mm(types[i], B));
    int n_of_type = 0;
    for (int q = i; q < nmat && types[q] == types[i]; ++q) ++n_of_type;
    // a Q6_K residual update (down) at one activation tile: K-chunk staging
    const bool kc = !tl && !mm && ep.kind == kEpiResidual && use_kcw(types[i], K, B, n_of_type);
    const int group = mm ? mm_group_tiles(false) : (tl || kc) ? 1 : gemm_group(all_tiles);
    while (j < nmat && types[j] == types[i]) {
      a.w[n] = (const uint8_t*)w[j];
      a.seg_rows[n] = rows[j];
      a.seg_tile_off[n] = tiles;
      a.seg_col_off[n] = col;
      tiles += ((rows[j] + 15) / 16 + group - 1) / group;  // workgroups of `group` tiles
      col += rows[j];
      ++n;
      ++j;
    }
    a.seg_tile_off[n] = tiles;
    a.nseg = n;
    const int wt = types[i];
    a.nsb = K / kQK;
    a.row_bytes = (size_t)(K / kQK) * sb_bytes(wt);
    const PackOut& pin = xin.of(wt);
    a.xpack = pin.pack;
    a.nslices = nslices_of(pin.kind, K);
    a.ss = ep.ss;
    a.ss_slots = ss_slots(B);
    a.inv_k = 1.0f / (float)K;
    a.eps = ep.eps;
    a.B = B;
    a.epi = ep.kind;
    a.y = ep.y;
    a.ldy = ep.ldy;
    a.gain = ep.gain;
    a.pack_out = ep.out1.pack;
    a.pack_kind = ep.out1.kind;
    a.pack_nslices = nslices_of(ep.out1.kind, ep.out_k);
    a.pack_out2 = ep.out2.pack;
    a.pack_kind2 = ep.out2.kind;
    a.pack_nslices2 = nslices_of(ep.out2.kind, ep.out_k);
    a.ss_out = ep.ss_out;
    if (!zeroed) {
      a.zero_ptr = ep.zero_ptr;
      a.zero_n = ep.zero_n;
      zeroed = true;
    }
    hipError_t e;
    if (mm) {
      a.part = ep.part;
      a.part_cap = ep.part_cap;
      a.ldp = col - col_begin;
      a.pcol0 = col_begin;
      e = launch_gemm_mm(wt, tiles, a, st);
    } else if (tl) {
      a.tl_groups = tiles;
      e = launch_gemm_tl(wt, 1, plan_gemm_tl(wt, 1, tiles, K, B), a, st);
    } else if (kc) {
      e = launch_gemm_kcw(tiles, a, st);
    } else {
      const GemmPlan pl = plan_gemm(wt, tiles, K, B, group);
      a.sb_per_wave = pl.sb_per_wave;
      e = launch_gemm(wt, pl, a, st);
    }
    if (e != hipSuccess) return e;
    i = j;
  }
  return hipSuccess;
}

// The SwiGLU GEMM: gate and up (same type, F rows each) paired per 16-column tile.
hipError_t gemm_swiglu(const void* wg, const void* wu, int wtype, int F, int K, int B, const Pack2& xin,
                       const double* ss, float eps, PackOut out, double* zero_ptr, int zero_n, hipStream_t st,
                       float* part = nullptr, size_t part_cap = 0, uint32_t* rb_cnt = nullptr, int rb_cnt_n = 0) {
  GemmArgs a{};
  a.w[0] = (const uint8_t*)wg;
  a.w[1] = (const uint8_t*)wu;
  a.seg_rows[0] = a.seg_rows[1] = F;
  a.nseg = 2;
  const int tiles = (F + 15) / 16;
  a.nsb = K / kQK;
  a.row_bytes = (size_t)(K / kQK) * sb_bytes(wtype);
  const PackOut& pin = xin.of(wtype);
  a.xpack = pin.pack;
  a.nslices = nslices_of(pin.kind, K);
  a.ss = ss;
  a.ss_slots = ss_slots(B);
  a.inv_k = 1.0f / (float)K;
  a.eps = eps;
  a.B = B;
  a.epi = kEpiSwiGLU;
  a.pack_out = out.pack;
  a.pack_kind = out.kind;
  a.pack_nslices = nslices_of(out.kind, F);
  a.zero_ptr = zero_ptr;
  a.zero_n = zero_n;
  if (use_mm(wtype, B)) return launch_gemm_mm(wtype, (tiles + mm_group_tiles(true) - 1) / mm_group_tiles(true), a, st);
  if (use_rb(wtype, K, B) && rb_fits(tiles, K, true, part_cap, rb_cnt_n)) {
    a.part = part;
    a.part_cap = part_cap;
    a.rb_cnt = rb_cnt;
    a.rb_cnt_n = rb_cnt_n;
    return launch_gemm_rb(tiles, a, st);
  }
  if (use_tile_loop(wtype, tiles, K, B) || use_tile_loop_whole(wtype, tiles, K, B)) {
    a.tl_groups = tiles;
    return launch_gemm_tl(wtype, 2, plan_gemm_tl(wtype, 2, tiles, K, B), a, st);
  }
  const GemmPlan pl = plan_gemm(wtype, tiles, K, B, 2);
  a.sb_per_wave = pl.sb_per_wave;
  return launch_gemm(wtype, pl, a, st);
}

struct LayerBufs {
  Pack2 xp;  // residual stream times the next RMSNorm gain (QKV / gate-up / head input)
  Pack2 op;  // attention output (Wo input)
  Pack2 ap;  // SwiGLU activation (down input)
  float* qkv;
  double *ss_attn, *ss_ffn;
  float *o_part, *m_part, *l_part;
  double* rope;  // [B][head_dim / 2][2]: RoPE of the step's positions
  float* qbuf;   // [B][Hq][D]: roped queries when a step carries several tokens per sequence
  float* part;   // many-row K-split partial sums (more than 64 rows), part_cap floats
  size_t part_cap;
  float* wg_part;     // decode attention: workgroup partial states
  uint32_t* wg_cnt;   // decode attention: arrival counters [B][Hkv], zeroed by the input pack
  int n_cnt;
  uint32_t* rb_cnt;   // row-block GEMM arrival counters, right after wg_cnt (zeroed with it)
  int rb_cnt_n;
  uint32_t* sched;    // decode attention: the step's work list, built by the input pack
};

// floats of the many-row K-split partial sums for `rows` rows and outputs of `cols`
// columns (no split above kMmSplitMaxCols columns or at 64 rows and below)
size_t mm_part_floats(int rows, int cols) {
  if (rows <= kMmMinRows) return 0;
  return (size_t)kMmMaxSplit * rows * (cols < kMmSplitMaxCols ? cols : kMmSplitMaxCols);
}

LayerBufs carve_layer(Carver& c, const gr_layer_cfg* cfg, int B, const AttnPlan& ap) {
  LayerBufs L;
  const int qd = cfg->n_q_heads * cfg->head_dim, kvd = cfg->n_kv_heads * cfg->head_dim;
  L.xp = carve_pack2(c, B, cfg->hidden);
  L.op = carve_pack2(c, B, qd);
  L.ap = carve_pack2(c, B, cfg->ffn);
  L.qkv = c.take<float>((size_t)B * (qd + 2 * kvd) * 4);
  L.ss_attn = c.take<double>(ss_count(B) * 8);  // [ss_slots(B)][B]
  L.ss_ffn = c.take<double>(ss_count(B) * 8);
  const size_t units = (size_t)B * cfg->n_q_heads * ap.max_splits;
  L.o_part = c.take<float>(units * cfg->head_dim * 4);
  L.m_part = c.take<float>(units * 4);
  L.l_part = c.take<float>(units * 4);
  L.rope = c.take<double>((size_t)B * cfg->head_dim * sizeof(double));
  L.qbuf = c.take<float>((size_t)B * qd * 4);
  L.part_cap = mm_part_floats(B, qd + 2 * kvd > cfg->hidden ? qd + 2 * kvd : cfg->hidden);
  // the row-block kernel's partials and counters: the gate/up pairs (Q4_K at 17 to 32 rows)
  const int gu = (cfg->ffn + 15) / 16;
  L.rb_cnt_n = 0;
  if (B > 16 && B <= 32) {
    L.part_cap = std::max(L.part_cap, rb_part_floats(gu, cfg->hidden, true));
    L.rb_cnt_n = gu;
  }
  L.part = L.part_cap ? c.take<float>(L.part_cap * 4) : nullptr;
  L.n_cnt = B * cfg->n_kv_heads;
  L.wg_cnt = c.take<uint32_t>((size_t)(L.n_cnt + L.rb_cnt_n) * 4);
  L.rb_cnt = L.wg_cnt + L.n_cnt;
  L.wg_part = c.take<float>(attn_dec_part_floats(B, cfg->n_q_heads, cfg->head_dim, ap.dec_wg_max > 1 ? ap.dec_wg_max : 1) * 4);
  L.sched = c.take<uint32_t>(attn_sched_words(B, ap.dec_wg_max > 1 ? ap.dec_wg_max : 1) * 4);
  return L;
}

gr_status check_layer_cfg(const gr_layer_cfg* c) {
  if (!c) return GR_ERR_NULL;
  if (!kv_ok(c->kv_dtype) || (c->rope_style != GR_ROPE_NEOX && c->rope_style != GR_ROPE_NORM)) return GR_ERR_DTYPE;
  if (c->page_size != GR_PAGE_SIZE) return GR_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return GR_ERR_SHAPE;
  if (c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->n_q_heads % c->n_kv_heads) return GR_ERR_SHAPE;
  if (c->n_q_heads / c->n_kv_heads > 8) return GR_ERR_SHAPE;
  if (c->hidden <= 0 || c->hidden % 256 || c->ffn <= 0 || c->ffn % 256) return GR_ERR_SHAPE;
  if ((c->n_q_heads * c->head_dim) % 256) return GR_ERR_SHAPE;
  if (c->hidden > 65536 || c->ffn > 65536 || c->n_q_heads * c->head_dim > 65536) return GR_ERR_SHAPE;
  if (!(c->rms_eps >= 0.0f) || !(c->rope_theta > 0.0)) return GR_ERR_SHAPE;
  return GR_OK;
}

gr_status check_layer_w(const gr_layer_cfg* c, const gr_layer_weights* w) {
  if (!w) return GR_ERR_NULL;
  if (!w->attn_norm || !w->ffn_norm || !w->wq || !w->wk || !w->wv || !w->wo || !w->w_gate || !w->w_up ||
      !w->w_down)
    return GR_ERR_NULL;
  if (c->qk_norm && (!w->q_norm || !w->k_norm)) return GR_ERR_NULL;
  const int ts[7] = {w->tq, w->tk, w->tv, w->to, w->tgate, w->tup, w->tdown};
  for (int t : ts)
    if (!wtype_ok(t)) return GR_ERR_DTYPE;
  if (w->tgate != w->tup) return GR_ERR_DTYPE;  // gate and up are streamed as pairs
  const void* ps[7] = {w->wq, w->wk, w->wv, w->wo, w->w_gate, w->w_up, w->w_down};
  for (const void* p : ps)
    if (!aligned(p, 16)) return GR_ERR_ALIGN;
  if (!aligned(w->attn_norm, 4) || !aligned(w->ffn_norm, 4)) return GR_ERR_ALIGN;
  return GR_OK;
}

// rows = B * T attention rows; a sequence holds at most max_ctx + T tokens after the step
AttnPlan layer_attn_plan(int rows, const gr_layer_cfg* c, int max_ctx, int T = 1) {
  AttnPlan pl = plan_attn(rows, c->n_kv_heads, max_ctx + T);
  const AttnDecPlan dp = plan_attn_dec(c->kv_dtype, max_ctx + T);
  pl.dec_wg_max = dp.wg_max;
  pl.dec_wg_pages = dp.wg_pages;
  pl.dec_slots = attn_dec_slots(c->kv_dtype);
  return pl;
}

// Optional timing probe: the launches of one stage (repeated `reps` times) carry the
// probe's start / stop events on their dispatches (see launch_kernel).
struct Probe {
  int stage = -1;
  int reps = 1;
  int layer = 0;
  void* const* ev_begin = nullptr;
  void* const* ev_end = nullptr;
};

// Runs body() once, or, for the probed stage, `reps` times with the layer's events
// armed on this thread.
template <class F>
gr_status probed(const Probe* p, int stage, hipStream_t st, F&& body) {
  (void)st;
  if (!p || p->stage != stage) return body();
  ProbeEvents pe;
  pe.start = (hipEvent_t)p->ev_begin[p->layer];
  pe.stop = (hipEvent_t)p->ev_end[p->layer];
  probe_events = &pe;
  gr_status s = GR_OK;
  for (int r = 0; r < p->reps && s == GR_OK; ++r) s = body();
  probe_events = nullptr;
  return s;
}

Kinds qkv_kinds(const gr_layer_weights* w) {
  Kinds k;
  k.add(w->tq);
  k.add(w->tk);
  k.add(w->tv);
  return k;
}

// Pack of the layer input: x * attn_norm and its sum of squares (and, for a decode
// step, the RoPE table of its positions).
gr_status run_input_pack(const float* x, int B, int H, const float* gain, Kinds k, const Pack2& xp, double* ss,
                         hipStream_t st, const Probe* probe, RopeTable rope = RopeTable{}, RowSel sel = RowSel{},
                         AttnSched sched = AttnSched{}) {
  return probed(probe, GR_STAGE_PACK, st, [&] {
    return check_launch(launch_pack_rows(x, H, B, H, gain, k.k32 ? xp.k32 : kNoPack, k.k16 ? xp.k16 : kNoPack, ss,
                                         st, rope, sel, sched));
  });
}

// The decode attention's work list and arrival counters, built and cleared by a decode
// step's first kernel (one token per row).
AttnSched attn_sched(const LayerBufs& L, const int32_t* ctx, int B, const AttnPlan& apl) {
  AttnSched z;
  z.ctx = ctx;
  z.B = B;
  z.self = 1;
  z.n_kv_heads = L.n_cnt / (B > 0 ? B : 1);
  z.slots = apl.dec_slots;
  z.group_pages = apl.dec_wg_pages;
  z.max_groups = kAttnDecMaxGroups;
  z.list = L.sched;
  z.cnt = L.wg_cnt;
  z.n_cnt = L.n_cnt + L.rb_cnt_n;
  return z;
}

// Steps without a decode work list: the input pack clears the arrival counters only.
AttnSched counters_only(const LayerBufs& L) {
  AttnSched z;
  z.cnt = L.wg_cnt;
  z.n_cnt = L.n_cnt + L.rb_cnt_n;
  return z;
}

RopeTable rope_table(const gr_layer_cfg* c, const int32_t* ctx, const LayerBufs& L, int T = 1,
                     const int32_t* row_pos = nullptr) {
  RopeTable r;
  r.ctx = ctx;
  r.theta = c->rope_theta;
  r.half_d = c->head_dim / 2;
  r.tokens_per_seq = T;
  r.row_pos = row_pos;
  r.out = L.rope;
  return r;
}

// Where a step's rows sit: row b is token b % T of sequence b / T at position
// ctx_lens[seq] + b % T (T = 1: a decode step), or, when pos is set, the token at
// position pos[b] of sequence seq[b].
struct RowMap {
  int T = 1;
  const int32_t* seq = nullptr;
  const int32_t* pos = nullptr;
  const int32_t* head_rows = nullptr;  // when set, the head runs on these n_head rows only
  int n_head = 0;
  bool fused() const { return T == 1 && !pos; }  // one token per sequence: append inside attention
};

// The launch sequence of one decode layer (arguments already validated).  B rows: row
// b is token b % T of sequence b / T (T = 1 for a decode step).  On entry L.xp holds
// x * attn_norm and L.ss_attn its per-row sum of squares.  On exit x is the layer output
// and, when next_gain is set, L.xp / L.ss_attn hold x * next_gain packed in the kinds
// `next`.
gr_status run_layer(const gr_layer_cfg* c, const gr_layer_weights* w, void* k_pages, void* v_pages, float* x,
                    const int32_t* bt, int max_blocks, const int32_t* ctx, int B, const AttnPlan& apl,
                    const LayerBufs& L, const float* next_gain, Kinds next, hipStream_t st, const Probe* probe,
                    RowMap rm = RowMap{}) {
  const int T = rm.T;
  const int H = c->hidden, D = c->head_dim, qd = c->n_q_heads * D, kvd = c->n_kv_heads * D, F = c->ffn;
  gr_status s;
  // 1. q, k, v = (W (x * g)) / rms(x); zero the FFN-norm accumulator for step 4
  s = probed(probe, GR_STAGE_QKV, st, [&] {
    const void* ws[3] = {w->wq, w->wk, w->wv};
    const int ts[3] = {w->tq, w->tk, w->tv};
    const int rs[3] = {qd, kvd, kvd};
    Epi ep;
    ep.kind = kEpiStore;
    ep.y = L.qkv;
    ep.ldy = qd + 2 * kvd;
    ep.ss = L.ss_attn;
    ep.eps = c->rms_eps;
    ep.zero_ptr = L.ss_ffn;
    ep.zero_n = ss_slots(B) * B;
    ep.part = L.part;
    ep.part_cap = L.part_cap;
    return check_launch(gemm_run(ws, ts, rs, 3, H, B, L.xp, ep, st));
  });
  if (s != GR_OK) return s;
  // 2. QK-norm, RoPE, KV append and split attention
  AttnParams ap{};
  ap.B = B;
  ap.tokens_per_seq = T;
  ap.self_in_pool = rm.fused() ? 0 : 1;
  // standalone: consecutive rows of one sequence (verification runs, prompt chunks) share
  // each page read, 8 / (Hq / Hkv) rows to a wave
  ap.rows_per_unit = rm.fused() ? 1 : 8 / (c->n_q_heads / c->n_kv_heads);
  ap.row_seq = rm.seq;
  ap.row_pos = rm.pos;
  ap.n_q_heads = c->n_q_heads;
  ap.n_kv_heads = c->n_kv_heads;
  ap.head_dim = D;
  ap.max_blocks = max_blocks;
  ap.pages_per_split = apl.pages_per_split;
  ap.max_splits = apl.max_splits;
  ap.scale = 1.0f / sqrtf((float)D);
  ap.block_table = bt;
  ap.ctx_lens = ctx;
  ap.k_pages = k_pages;
  ap.v_pages = v_pages;
  ap.qkv = L.qkv;
  ap.qkv_ld = qd + 2 * kvd;
  ap.q_dim = qd;
  ap.kv_dim = kvd;
  ap.q_norm = c->qk_norm ? w->q_norm : nullptr;
  ap.k_norm = c->qk_norm ? w->k_norm : nullptr;
  ap.eps = c->rms_eps;
  ap.rope_style = c->rope_style;
  ap.rope = L.rope;
  ap.o_part = L.o_part;
  ap.m_part = L.m_part;
  ap.l_part = L.l_part;
  if (rm.fused()) {
    // one token per sequence: the decode kernel stores the new K/V, attends, merges its
    // workgroups' partial states and writes the Wo input pack (no merge launch)
    const PackOut& op = L.op.of(w->to);
    ap.wg_part = L.wg_part;
    ap.wg_cnt = L.wg_cnt;
    ap.wg_max = apl.dec_wg_max;
    ap.wg_pages = apl.dec_wg_pages;
    ap.sched = L.sched;
    ap.pack = op.pack;
    ap.pack_kind = op.kind;
    ap.pack_nslices = nslices_of(op.kind, qd);
    s = probed(probe, GR_STAGE_ATTN, st, [&] { return check_launch(launch_attn_decode(c->kv_dtype, true, ap, st)); });
    if (s != GR_OK) return s;
  } else {
    // several tokens of a sequence: every row's K/V is stored before any row attends
    ap.q = L.qbuf;
    s = probed(probe, GR_STAGE_ATTN, st, [&] {
      const hipError_t e = launch_attn_append(c->kv_dtype, ap, L.qbuf, st);
      return check_launch(e != hipSuccess ? e : launch_attn_split(c->kv_dtype, false, ap, st));
    });
    if (s != GR_OK) return s;
    // 3. log-sum-exp merge -> Wo input pack
    s = probed(probe, GR_STAGE_ATTN_MERGE, st, [&] {
      const PackOut& op = L.op.of(w->to);
      return check_launch(launch_attn_merge(ap, nullptr, op.pack, op.kind, nslices_of(op.kind, qd), 0, st));
    });
    if (s != GR_OK) return s;
  }
  // 4. x += Wo o; pack x * ffn_norm and its sum of squares for the gate/up GEMM
  s = probed(probe, GR_STAGE_WO, st, [&] {
    const void* ws[1] = {w->wo};
    const int ts[1] = {w->to};
    const int rs[1] = {H};
    Epi ep;
    ep.kind = kEpiResidual;
    ep.y = x;
    ep.ldy = H;
    ep.gain = w->ffn_norm;
    ep.out1 = L.xp.of(w->tgate);
    ep.out_k = H;
    ep.ss_out = L.ss_ffn;
    ep.part = L.part;
    ep.part_cap = L.part_cap;
    return check_launch(gemm_run(ws, ts, rs, 1, qd, B, L.op, ep, st));
  });
  if (s != GR_OK) return s;
  // 5. a = silu(gate) * up (inputs divided by rms) -> down input pack; zero the
  //    attention-norm accumulator for step 6
  s = probed(probe, GR_STAGE_GATE_UP, st, [&] {
    return check_launch(gemm_swiglu(w->w_gate, w->w_up, w->tgate, F, H, B, L.xp, L.ss_ffn, c->rms_eps,
                                    L.ap.of(w->tdown), L.ss_attn, ss_slots(B) * B, st, L.part, L.part_cap, L.rb_cnt,
                                    L.rb_cnt_n));
  });
  if (s != GR_OK) return s;
  // 6. x += W_down a; pack x * next_gain for the next consumer
  return probed(probe, GR_STAGE_DOWN, st, [&] {
    const void* ws[1] = {w->w_down};
    const int ts[1] = {w->tdown};
    const int rs[1] = {H};
    Epi ep;
    ep.kind = kEpiResidual;
    ep.y = x;
    ep.ldy = H;
    if (next_gain) {
      ep.gain = next_gain;
      ep.out1 = next.k32 ? L.xp.k32 : kNoPack;
      ep.out2 = next.k16 ? L.xp.k16 : kNoPack;
      ep.out_k = H;
      ep.ss_out = L.ss_attn;
    }
    ep.part = L.part;
    ep.part_cap = L.part_cap;
    return check_launch(gemm_run(ws, ts, rs, 1, F, B, L.ap, ep, st));
  });
}

// Output head on a packed input (x * norm in xp, sum of squares in ss).
gr_status run_head(const void* w, int wtype, float* logits, int B, int H, int vocab, float eps, const Pack2& xp,
                   const double* ss, hipStream_t st, const Probe* probe) {
  return probed(probe, GR_STAGE_HEAD, st, [&] {
    const void* ws[1] = {w};
    const int ts[1] = {wtype};
    const int rs[1] = {vocab};
    Epi ep;
    ep.kind = kEpiStore;
    ep.y = logits;
    ep.ldy = vocab;
    ep.ss = ss;
    ep.eps = eps;
    return check_launch(gemm_run(ws, ts, rs, 1, H, B, xp, ep, st));
  });
}

}  // namespace
}  // namespace gr

using namespace gr;

extern "C" {

int gr_abi_version(void) { return GR_ABI_VERSION; }

const char* gr_status_str(int s) {
  switch (s) {
    case GR_OK: return "ok";
    case GR_ERR_NULL: return "required pointer is NULL";
    case GR_ERR_SHAPE: return "size or shape out of the supported range";
    case GR_ERR_DTYPE: return "unknown weight type, KV dtype or rope style";
    case GR_ERR_ALIGN: return "pointer lacks the required alignment";
    case GR_ERR_WORKSPACE: return "workspace missing or too small";
    case GR_ERR_CAPACITY: return "max_ctx + 1 tokens exceed the block table's pages";
    case GR_ERR_DEVICE: return "current device is not gfx950";
    case GR_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int gr_last_hip_error(void) { return t_last_hip_error; }

int64_t gr_kv_head_bytes(int kv_dtype, int head_dim) {
  if (head_dim <= 0 || head_dim % 32) return -1;
  if (kv_dtype == GR_KV_F32) return (int64_t)GR_PAGE_SIZE * head_dim * 4;
  if (kv_dtype == GR_KV_F16) return (int64_t)GR_PAGE_SIZE * head_dim * 2;
  if (kv_dtype == GR_KV_Q8_0) return (int64_t)GR_PAGE_SIZE * head_dim + GR_PAGE_SIZE * (head_dim / 32) * 2;
  return -1;
}

// ------------------------------------------------------------------ dequant
static gr_status dequant_common(int kind, const void* blocks, int64_t n, float* out, void* stream) {
  if (n < 0) return GR_ERR_SHAPE;
  if (n == 0) return GR_OK;
  if (!blocks || !out) return GR_ERR_NULL;
  if (!aligned(blocks, kind == 12 ? 16 : 2) || !aligned(out, 4)) return GR_ERR_ALIGN;
  gr_status s = check_device();
  if (s != GR_OK) return s;
  return check_launch(launch_dequant(kind, blocks, n, out, (hipStream_t)stream));
}
gr_status gr_stream_read(const void* p, size_t bytes, uint32_t* out, void* stream) {
  if (bytes == 0) return GR_OK;
  if (!p || !out) return GR_ERR_NULL;
  if (bytes % 16) return GR_ERR_SHAPE;
  if (!aligned(p, 16) || !aligned(out, 4)) return GR_ERR_ALIGN;
  gr_status s = check_device();
  if (s != GR_OK) return s;
  return check_launch(launch_stream_read(p, bytes, out, (hipStream_t)stream));
}
gr_status gr_q4k_dequant(const void* b, int64_t n, float* out, void* s) { return dequant_common(12, b, n, out, s); }
gr_status gr_q6k_dequant(const void* b, int64_t n, float* out, void* s) { return dequant_common(14, b, n, out, s); }
gr_status gr_q8_0_dequant(const void* b, int64_t n, float* out, void* s) { return dequant_common(8, b, n, out, s); }

// --------------------------------------------------------------------- GEMM
size_t gr_gemm_workspace_size(int B, int N, int K) {
  if (B <= 0 || K <= 0 || N < 0) return 0;
  Carver c(nullptr);
  carve_pack2(c, B, K);
  c.take<float>(mm_part_floats(B, N) * 4);
  return c.off + 256;
}

gr_status gr_gemm_launch_shape(int wtype, int rows, int K, int B, int epi, int* tile_loop, int* nt, int* btn,
                               int* maxt, int* grid_threads, int* block_threads) {
  if (!tile_loop || !nt || !btn || !maxt || !grid_threads || !block_threads) return GR_ERR_NULL;
  if (!wtype_ok(wtype)) return GR_ERR_DTYPE;
  if (rows <= 0 || K <= 0 || K % kQK || B <= 0 || B > kMaxRows || epi < 0 || epi > 2) return GR_ERR_SHAPE;
  if (mm_required(B) && !mm_supported(wtype)) return GR_ERR_DTYPE;
  const int tiles = (rows + 15) / 16;
  const bool pair = epi == 2;
  // the choices gemm_run and gemm_swiglu make (given the workspace the layer and the
  // standalone GEMM provide)
  if (pair && !use_mm(wtype, B) && use_rb(wtype, K, B)) {  // row-block kernel (gate/up pairs)
    const int nkr = rb_ranges(K / kQK), W = K / kQK / nkr;
    *tile_loop = 6;
    *nt = 2;
    *btn = 4;
    *maxt = 512;
    *block_threads = W * 64;
    *grid_threads = rb_grid(K / kQK) * W * 64;
    return GR_OK;
  }
  if ((pair || epi == 0) && !use_mm(wtype, B) &&
      (use_tile_loop(wtype, tiles, K, B) || use_tile_loop_whole(wtype, tiles, K, B))) {
    const TlPlan tp = plan_gemm_tl(wtype, pair ? 2 : 1, tiles, K, B);
    *tile_loop = tp.whole ? 3 : 1;
    *nt = pair ? 2 : 1;
    *btn = tl_btn(B);
    *maxt = tp.whole ? 1024 : 512;
    *grid_threads = tp.grid * tp.waves * 64;
    *block_threads = tp.waves * 64;
    return GR_OK;
  }
  if (epi == 1 && !use_mm(wtype, B) && use_tile_loop_whole(wtype, tiles, K, B)) {  // whole tiles (Wo)
    const TlPlan tp = plan_gemm_tl(wtype, 1, tiles, K, B);
    *tile_loop = 5;
    *nt = 1;
    *btn = 1;
    *maxt = 1024;
    *grid_threads = tp.grid * tp.waves * 64;
    *block_threads = tp.waves * 64;
    return GR_OK;
  }
  if (epi == 1 && !use_mm(wtype, B) && use_kcw(wtype, K, B, 1)) {  // K-chunk staging (gemm_kcw_kernel)
    const int C = kcw_waves(K / kQK);
    *tile_loop = 4;
    *nt = 1;
    *btn = 1;
    *maxt = 1024;
    *grid_threads = tiles * C * 64;
    *block_threads = C * 64;
    return GR_OK;
  }
  if (epi == 0 ? use_mm_store(wtype, B, rows) : use_mm(wtype, B)) {  // the many-row kernel: 512 threads, activation tile groups x weight tile groups
    const int gt = mm_group_tiles(pair);
    const int mb = wtype == GR_W_Q4_K ? 4 : 2;
    *tile_loop = 2;
    *nt = 2;
    *btn = mb;
    *maxt = 512;
    *block_threads = 512;
    const int groups = (tiles + gt - 1) / gt;
    const int split = mm_split(wtype, B, rows, K / kQK, groups, epi, mm_part_floats(B, rows));
    *grid_threads = (actpack_tiles(B) / mb) * groups * split * 512;  // a split adds a finishing pass
    return GR_OK;
  }
  *tile_loop = 0;
  const int group = gemm_group(tiles);
  const GemmPlan pl = pair ? plan_gemm(wtype, tiles, K, B, 2)
                           : plan_gemm(wtype, (tiles + group - 1) / group, K, B, group);
  *nt = pl.nt;
  *btn = pl.btn;
  *maxt = pl.maxt;
  *grid_threads = pl.tiles * pl.waves * 64;
  *block_threads = pl.waves * 64;
  return GR_OK;
}

static gr_status gemm_api(int wtype, const void* w, const float* x, float* y, int B, int N, int K, void* ws,
                          size_t ws_bytes, void* stream) {
  if (B < 0 || N < 0 || K < 0) return GR_ERR_SHAPE;
  if (B == 0 || N == 0) return GR_OK;
  if (!w || !x || !y) return GR_ERR_NULL;
  if (B > kMaxRows || K == 0 || K % 256 || K > 65536) return GR_ERR_SHAPE;
  if (mm_required(B) && !mm_supported(wtype)) return GR_ERR_DTYPE;
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return GR_ERR_ALIGN;
  if (!ws || ws_bytes < gr_gemm_workspace_size(B, N, K) || !aligned(ws, 256)) return GR_ERR_WORKSPACE;
  gr_status s = check_device();
  if (s != GR_OK) return s;
  Carver c(ws);
  const Pack2 xp = carve_pack2(c, B, K);
  const size_t part_cap = mm_part_floats(B, N);
  float* part = part_cap ? c.take<float>(part_cap * 4) : nullptr;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_pack_rows(x, K, B, K, nullptr, xp.of(wtype), kNoPack, nullptr, st);
  if (e != hipSuccess) return check_launch(e);
  const void* ws1[1] = {w};
  const int ts[1] = {wtype};
  const int rs[1] = {N};
  Epi ep;
  ep.kind = kEpiStore;
  ep.y = y;
  ep.ldy = N;
  ep.part = part;
  ep.part_cap = part_cap;
  return check_launch(gemm_run(ws1, ts, rs, 1, K, B, xp, ep, st));
}

gr_status gr_q4k_gemm(const void* w, const float* x, float* y, int B, int N, int K, void* ws, size_t wsb, void* s) {
  return gemm_api(GR_W_Q4_K, w, x, y, B, N, K, ws, wsb, s);
}
gr_status gr_q6k_gemm(const void* w, const float* x, float* y, int B, int N, int K, void* ws, size_t wsb, void* s) {
  return gemm_api(GR_W_Q6_K, w, x, y, B, N, K, ws, wsb, s);
}
gr_status gr_q5k_gemm(const void* w, const float* x, float* y, int B, int N, int K, void* ws, size_t wsb, void* s) {
  return gemm_api(GR_W_Q5_K, w, x, y, B, N, K, ws, wsb, s);
}
gr_status gr_q8_0_gemm(const void* w, const float* x, float* y, int B, int N, int K, void* ws, size_t wsb, void* s) {
  return gemm_api(GR_W_Q8_0, w, x, y, B, N, K, ws, wsb, s);
}

// ---------------------------------------------------------------- attention
static gr_status check_meta(const gr_attn_meta* m) {
  if (!m) return GR_ERR_NULL;
  if (!kv_ok(m->kv_dtype)) return GR_ERR_DTYPE;
  if (m->page_size != GR_PAGE_SIZE) return GR_ERR_SHAPE;
  if (m->head_dim != 64 && m->head_dim != 128) return GR_ERR_SHAPE;
  if (m->n_q_heads <= 0 || m->n_kv_heads <= 0 || m->n_q_heads % m->n_kv_heads) return GR_ERR_SHAPE;
  if (m->n_q_heads / m->n_kv_heads > 8) return GR_ERR_SHAPE;
  if (m->num_pages <= 0 || m->max_blocks_per_row <= 0 || m->max_ctx <= 0) return GR_ERR_SHAPE;
  if ((int64_t)m->max_ctx > (int64_t)GR_PAGE_SIZE * m->max_blocks_per_row) return GR_ERR_CAPACITY;
  if (plan_attn_dec(m->kv_dtype, m->max_ctx).wg_max == 0) return GR_ERR_CAPACITY;
  return GR_OK;
}

// Standalone decode attention workspace: arrival counters [B][Hkv], then the workgroup
// partial states.
static void carve_attn_ws(Carver& c, const gr_attn_meta* m, int B, AttnParams& ap, uint32_t** list) {
  const AttnDecPlan dp = plan_attn_dec(m->kv_dtype, m->max_ctx);
  ap.wg_max = dp.wg_max;
  ap.wg_pages = dp.wg_pages;
  ap.wg_cnt = c.take<uint32_t>((size_t)B * m->n_kv_heads * 4);
  ap.wg_part = c.take<float>(attn_dec_part_floats(B, m->n_q_heads, m->head_dim, ap.wg_max) * 4);
  *list = c.take<uint32_t>(attn_sched_words(B, ap.wg_max) * 4);
  ap.sched = *list;
}

size_t gr_paged_decode_attn_workspace_size(const gr_attn_meta* m, int B) {
  if (check_meta(m) != GR_OK || B <= 0) return 0;
  Carver c(nullptr);
  AttnParams ap{};
  uint32_t* list;
  carve_attn_ws(c, m, B, ap, &list);
  return c.off + 256;
}

// The decode attention call with its workspace at ws (device memory, 256-byte aligned,
// at least gr_paged_decode_attn_workspace_size bytes, checked by the caller).
static gr_status paged_decode_attn_ws(const float* q, const void* k_pages, const void* v_pages,
                                      const int32_t* block_table, const int32_t* ctx_lens, float* out, int B,
                                      const gr_attn_meta* m, void* ws, void* stream);

static gr_status check_attn_call(const float* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                                 const int32_t* ctx_lens, float* out, int B, const gr_attn_meta* m) {
  if (B < 0) return GR_ERR_SHAPE;
  gr_status s = check_meta(m);
  if (s != GR_OK) return s;
  if (B == 0) return GR_OK;
  if (B > 4096) return GR_ERR_SHAPE;
  if (!q || !k_pages || !v_pages || !block_table || !ctx_lens || !out) return GR_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 4) ||
      !aligned(block_table, 4) || !aligned(ctx_lens, 4))
    return GR_ERR_ALIGN;
  return GR_OK;
}

gr_status gr_paged_decode_attn(const float* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                               const int32_t* ctx_lens, float* out, int B, const gr_attn_meta* m, void* ws,
                               size_t ws_bytes, void* stream) {
  gr_status s = check_attn_call(q, k_pages, v_pages, block_table, ctx_lens, out, B, m);
  if (s != GR_OK || B == 0) return s;
  if (!ws || ws_bytes < gr_paged_decode_attn_workspace_size(m, B) || !aligned(ws, 256)) return GR_ERR_WORKSPACE;
  s = check_device();
  if (s != GR_OK) return s;
  return paged_decode_attn_ws(q, k_pages, v_pages, block_table, ctx_lens, out, B, m, ws, stream);
}

static gr_status paged_decode_attn_ws(const float* q, const void* k_pages, const void* v_pages,
                                      const int32_t* block_table, const int32_t* ctx_lens, float* out, int B,
                                      const gr_attn_meta* m, void* ws, void* stream) {
  Carver c(ws);
  AttnParams ap{};
  uint32_t* list;
  carve_attn_ws(c, m, B, ap, &list);
  ap.tokens_per_seq = 1;
  ap.B = B;
  ap.n_q_heads = m->n_q_heads;
  ap.n_kv_heads = m->n_kv_heads;
  ap.head_dim = m->head_dim;
  ap.max_blocks = m->max_blocks_per_row;
  ap.scale = m->scale;
  ap.block_table = block_table;
  ap.ctx_lens = ctx_lens;
  ap.k_pages = k_pages;
  ap.v_pages = v_pages;
  ap.q = q;
  ap.out = out;
  hipStream_t st = (hipStream_t)stream;
  AttnSched sc;
  sc.ctx = ctx_lens;
  sc.B = B;
  sc.self = 0;
  sc.n_kv_heads = m->n_kv_heads;
  sc.slots = attn_dec_slots(m->kv_dtype);
  sc.group_pages = ap.wg_pages;
  sc.max_groups = kAttnDecMaxGroups;
  sc.list = list;
  sc.cnt = ap.wg_cnt;
  sc.n_cnt = B * m->n_kv_heads;
  hipError_t e = launch_attn_sched(sc, st);
  if (e != hipSuccess) return check_launch(e);
  return check_launch(launch_attn_decode(m->kv_dtype, false, ap, st));
}

// ------------------------------------------- decode attention without allocation
// The allocation-free variant keeps its workspace (arrival counters, workgroup partial
// states, work list) in this file-scope array: one copy per device, held until the
// process ends.  Host code never passes the array's name to a kernel (on the host it is
// a stand-in, not a device address): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[GR_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static gr_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GR_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return check_launch(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GR_OK;
}

gr_status gr_paged_decode_attn_noalloc(const float* q, const void* k_pages, const void* v_pages,
                                       const int32_t* block_table, const int32_t* ctx_lens, float* out, int B,
                                       const gr_attn_meta* m, void* stream) {
  gr_status s = check_attn_call(q, k_pages, v_pages, block_table, ctx_lens, out, B, m);
  if (s != GR_OK || B == 0) return s;
  if (gr_paged_decode_attn_workspace_size(m, B) > (size_t)GR_NOALLOC_SCRATCH_BYTES) return GR_ERR_WORKSPACE;
  s = check_device();
  if (s != GR_OK) return s;
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != GR_OK) return s;
  return paged_decode_attn_ws(q, k_pages, v_pages, block_table, ctx_lens, out, B, m, ws, stream);
}

gr_status gr_attn_launch_shape(int kv_dtype, int B, int n_kv_heads, int max_tokens, int* waves_per_wg,
                               int* pages_per_wave, int* wg_per_row, long long* grid_threads) {
  if (!waves_per_wg || !pages_per_wave || !wg_per_row || !grid_threads) return GR_ERR_NULL;
  if (!kv_ok(kv_dtype)) return GR_ERR_DTYPE;
  if (B <= 0 || n_kv_heads <= 0 || max_tokens <= 0) return GR_ERR_SHAPE;
  const AttnDecPlan dp = plan_attn_dec(kv_dtype, max_tokens);
  if (dp.wg_max == 0) return GR_ERR_CAPACITY;
  *waves_per_wg = kAttnDecWaves;
  *pages_per_wave = dp.wg_pages / kAttnDecWaves;
  *wg_per_row = dp.wg_max;
  *grid_threads = (long long)B * n_kv_heads * dp.wg_max * kAttnDecWaves * 64;
  return GR_OK;
}

gr_status gr_paged_gather_kv(const void* pages, int is_v, const int32_t* block_table, const int32_t* ctx_lens, int B,
                             const gr_attn_meta* m, float* out, void* stream) {
  if (B < 0) return GR_ERR_SHAPE;
  gr_status s = check_meta(m);
  if (s != GR_OK) return s;
  if (B == 0) return GR_OK;
  if (!pages || !block_table || !ctx_lens || !out) return GR_ERR_NULL;
  if (!aligned(pages, 16) || !aligned(out, 4)) return GR_ERR_ALIGN;
  if (B > 65535 || m->n_kv_heads > 65535) return GR_ERR_SHAPE;
  s = check_device();
  if (s != GR_OK) return s;
  return check_launch(launch_gather(m->kv_dtype, m->head_dim, pages, is_v ? 1 : 0, block_table, ctx_lens, B,
                                    m->max_blocks_per_row, m->n_kv_heads, m->max_ctx, out, (hipStream_t)stream));
}

// --------------------------------------------------------------- decode layer
static size_t layer_ws_bytes(const gr_layer_cfg* c, int B, int T, int max_ctx) {
  if (check_layer_cfg(c) != GR_OK || B <= 0 || T <= 0 || max_ctx < 0) return 0;
  Carver cv(nullptr);
  carve_layer(cv, c, B * T, layer_attn_plan(B * T, c, max_ctx, T));
  return cv.off + 256;
}

size_t gr_decode_layer_workspace_size(const gr_layer_cfg* c, int B, int max_ctx) {
  return layer_ws_bytes(c, B, 1, max_ctx);
}

// B sequences of T tokens each (B * T rows through the GEMMs).
static gr_status check_layer_call(const gr_layer_cfg* c, const gr_layer_weights* w, const void* k_pages,
                                  const void* v_pages, int num_pages, const float* x, const int32_t* bt,
                                  int max_blocks, const int32_t* ctx, int max_ctx, int B, int T = 1,
                                  const int32_t* row_seq = nullptr, const int32_t* row_pos = nullptr) {
  gr_status s = check_layer_cfg(c);
  if (s != GR_OK) return s;
  s = check_layer_w(c, w);
  if (s != GR_OK) return s;
  if (B < 0 || T < 1 || (int64_t)B * T > kMaxRows) return GR_ERR_SHAPE;
  if (mm_required(B * T)) {
    const int ts[7] = {w->tq, w->tk, w->tv, w->to, w->tgate, w->tup, w->tdown};
    for (int t : ts)
      if (!mm_supported(t)) return GR_ERR_DTYPE;
  }
  if (!k_pages || !v_pages || !x || !bt) return GR_ERR_NULL;
  if (row_pos ? !row_seq : !ctx) return GR_ERR_NULL;
  if (num_pages <= 0 || max_blocks <= 0 || max_ctx < 0) return GR_ERR_SHAPE;
  if ((int64_t)max_ctx + T > (int64_t)GR_PAGE_SIZE * max_blocks) return GR_ERR_CAPACITY;
  // one token per sequence: the decode attention kernel's longest context
  if (T == 1 && !row_pos && plan_attn_dec(c->kv_dtype, max_ctx + 1).wg_max == 0)
    return GR_ERR_CAPACITY;
  if (!aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(x, 16) || !aligned(bt, 4) || !aligned(ctx, 4) ||
      !aligned(row_seq, 4) || !aligned(row_pos, 4))
    return GR_ERR_ALIGN;
  return GR_OK;
}

gr_status gr_decode_layer(const gr_layer_cfg* c, const gr_layer_weights* w, void* k_pages, void* v_pages,
                          int num_pages, float* x, const int32_t* bt, int max_blocks, const int32_t* ctx, int max_ctx,
                          int B, void* ws, size_t ws_bytes, void* stream) {
  gr_status s = check_layer_call(c, w, k_pages, v_pages, num_pages, x, bt, max_blocks, ctx, max_ctx, B);
  if (s != GR_OK) return s;
  if (B == 0) return GR_OK;
  if (!ws || ws_bytes < gr_decode_layer_workspace_size(c, B, max_ctx) || !aligned(ws, 256)) return GR_ERR_WORKSPACE;
  s = check_device();
  if (s != GR_OK) return s;
  const AttnPlan apl = layer_attn_plan(B, c, max_ctx);
  Carver cv(ws);
  const LayerBufs L = carve_layer(cv, c, B, apl);
  hipStream_t st = (hipStream_t)stream;
  s = run_input_pack(x, B, c->hidden, w->attn_norm, qkv_kinds(w), L.xp, L.ss_attn, st, nullptr, rope_table(c, ctx, L),
                     RowSel{}, attn_sched(L, ctx, B, apl));
  if (s != GR_OK) return s;
  return run_layer(c, w, k_pages, v_pages, x, bt, max_blocks, ctx, B, apl, L, nullptr, Kinds{}, st, nullptr);
}

size_t gr_output_head_workspace_size(int B, int hidden, int vocab) {
  if (B <= 0 || hidden <= 0) return 0;
  (void)vocab;
  Carver c(nullptr);
  carve_pack2(c, B, hidden);
  c.take<double>(ss_count(B) * 8);
  return c.off + 256;
}

gr_status gr_output_head(const float* x, const float* norm, float eps, const void* w, int wtype, float* logits, int B,
                         int hidden, int vocab, void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || hidden < 0 || vocab < 0) return GR_ERR_SHAPE;
  if (!wtype_ok(wtype)) return GR_ERR_DTYPE;
  if (B == 0 || vocab == 0) return GR_OK;
  if (!x || !norm || !w || !logits) return GR_ERR_NULL;
  if (B > kMaxRows || hidden % 256 || hidden > 65536) return GR_ERR_SHAPE;
  if (mm_required(B) && !mm_supported(wtype)) return GR_ERR_DTYPE;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(logits, 4) || !aligned(norm, 4)) return GR_ERR_ALIGN;
  if (!ws || ws_bytes < gr_output_head_workspace_size(B, hidden, vocab) || !aligned(ws, 256)) return GR_ERR_WORKSPACE;
  gr_status s = check_device();
  if (s != GR_OK) return s;
  Carver c(ws);
  const Pack2 xp = carve_pack2(c, B, hidden);
  double* ss = c.take<double>(ss_count(B) * 8);
  hipStream_t st = (hipStream_t)stream;
  Kinds k;
  k.add(wtype);
  s = run_input_pack(x, B, hidden, norm, k, xp, ss, st, nullptr);
  if (s != GR_OK) return s;
  return run_head(w, wtype, logits, B, hidden, vocab, eps, xp, ss, st, nullptr);
}

size_t gr_sample_workspace_size(int B, int vocab) {
  if (B <= 0 || vocab <= 0 || vocab > sample_max_vocab() || B > 65535) return 0;
  return sample_workspace_bytes(B, vocab) + 256;
}

gr_status gr_sample(const float* logits, int B, int vocab, const gr_sample_params* params, int32_t* tokens,
                    uint64_t* kept_weight, void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || vocab < 1 || vocab > sample_max_vocab() || B > 65535) return GR_ERR_SHAPE;
  if (B == 0) return GR_OK;
  if (!logits || !params || !tokens) return GR_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(params, 8) || !aligned(tokens, 4) || !aligned(kept_weight, 8))
    return GR_ERR_ALIGN;
  if (!ws || ws_bytes < gr_sample_workspace_size(B, vocab) || !aligned(ws, 256)) return GR_ERR_WORKSPACE;
  gr_status s = check_device();
  if (s != GR_OK) return s;
  return check_launch(launch_sample(logits, B, vocab, params, tokens, kept_weight, ws, (hipStream_t)stream));
}

size_t gr_decode_stack_workspace_size(const gr_layer_cfg* c, int B, int max_ctx, int vocab) {
  (void)vocab;
  return gr_decode_layer_workspace_size(c, B, max_ctx);
}

static gr_status decode_stack_impl(const gr_layer_cfg* c, const gr_layer_weights* weights, int n_layers,
                                   void* const* k_pages, void* const* v_pages, int num_pages, float* x,
                                   const int32_t* bt, int max_blocks, const int32_t* ctx, int max_ctx, int B,
                                   const float* head_norm, const void* head_w, int head_wtype, int vocab,
                                   float* logits, void* ws, size_t ws_bytes, void* stream, Probe* probe,
                                   RowMap rm = RowMap{}) {
  const int T = rm.T;
  if (n_layers < 0) return GR_ERR_SHAPE;
  if (n_layers > 0 && (!weights || !k_pages || !v_pages)) return GR_ERR_NULL;
  for (int l = 0; l < n_layers; ++l) {
    gr_status s = check_layer_call(c, &weights[l], k_pages[l], v_pages[l], num_pages, x, bt, max_blocks, ctx,
                                   max_ctx, B, T, rm.seq, rm.pos);
    if (s != GR_OK) return s;
  }
  if (rm.head_rows && (rm.n_head < 1 || (int64_t)rm.n_head > (int64_t)B * T)) return GR_ERR_SHAPE;
  if (rm.head_rows && !aligned(rm.head_rows, 4)) return GR_ERR_ALIGN;
  const int head_b = rm.head_rows ? rm.n_head : B * T;
  if (head_w) {
    if (!wtype_ok(head_wtype)) return GR_ERR_DTYPE;
    if (mm_required(head_b) && !mm_supported(head_wtype)) return GR_ERR_DTYPE;
    if (!head_norm || !logits) return GR_ERR_NULL;
    if (vocab <= 0) return GR_ERR_SHAPE;
    if (!aligned(head_w, 16) || !aligned(head_norm, 4) || !aligned(logits, 4)) return GR_ERR_ALIGN;
  }
  if (n_layers == 0) {
    gr_status s = check_layer_cfg(c);
    if (s != GR_OK) return s;
    if (B < 0 || T < 1 || (int64_t)B * T > kMaxRows) return GR_ERR_SHAPE;
  }
  if (probe && probe->stage >= 0) {
    if (!probe->ev_begin || !probe->ev_end) return GR_ERR_NULL;
    if (probe->stage > GR_STAGE_HEAD) return GR_ERR_SHAPE;
  }
  if (B == 0) return GR_OK;
  if (!ws || ws_bytes < layer_ws_bytes(c, B, T, max_ctx) || !aligned(ws, 256)) return GR_ERR_WORKSPACE;
  gr_status s = check_device();
  if (s != GR_OK) return s;
  const int rows = B * T;
  const AttnPlan apl = layer_attn_plan(rows, c, max_ctx, T);
  Carver cv(ws);
  const LayerBufs L = carve_layer(cv, c, rows, apl);
  hipStream_t st = (hipStream_t)stream;
  if (probe) probe->layer = 0;
  if (n_layers > 0) {
    s = run_input_pack(x, rows, c->hidden, weights[0].attn_norm, qkv_kinds(&weights[0]), L.xp, L.ss_attn, st, probe,
                       rope_table(c, ctx, L, T, rm.pos), RowSel{},
                       rm.fused() ? attn_sched(L, ctx, rows, apl) : counters_only(L));
  } else if (head_w) {
    Kinds k;
    k.add(head_wtype);
    RowSel sel;
    sel.idx = rm.head_rows;
    sel.src_rows = rows;
    s = run_input_pack(x, head_b, c->hidden, head_norm, k, L.xp, L.ss_attn, st, probe, RopeTable{}, sel);
  }
  if (s != GR_OK) return s;
  for (int l = 0; l < n_layers; ++l) {
    if (probe) probe->layer = l;
    const float* next_gain = nullptr;
    Kinds next;
    if (l + 1 < n_layers) {
      next_gain = weights[l + 1].attn_norm;
      next = qkv_kinds(&weights[l + 1]);
    } else if (head_w && !rm.head_rows) {
      next_gain = head_norm;
      next.add(head_wtype);
    }
    s = run_layer(c, &weights[l], k_pages[l], v_pages[l], x, bt, max_blocks, ctx, rows, apl, L, next_gain, next, st,
                  probe, rm);
    if (s != GR_OK) return s;
  }
  if (probe) probe->layer = 0;
  if (head_w && rm.head_rows && n_layers > 0) {
    // the selected rows' final states, gathered into the pack with the head's norm
    Kinds k;
    k.add(head_wtype);
    RowSel sel;
    sel.idx = rm.head_rows;
    sel.src_rows = rows;
    s = run_input_pack(x, head_b, c->hidden, head_norm, k, L.xp, L.ss_attn, st, probe, RopeTable{}, sel);
    if (s != GR_OK) return s;
  }
  if (head_w)
    return run_head(head_w, head_wtype, logits, head_b, c->hidden, vocab, c->rms_eps, L.xp, L.ss_attn, st, probe);
  return GR_OK;
}

gr_status gr_decode_stack(const gr_layer_cfg* c, const gr_layer_weights* weights, int n_layers,
                          void* const* k_pages, void* const* v_pages, int num_pages, float* x, const int32_t* bt,
                          int max_blocks, const int32_t* ctx, int max_ctx, int B, const float* head_norm,
                          const void* head_w, int head_wtype, int vocab, float* logits, void* ws, size_t ws_bytes,
                          void* stream) {
  return decode_stack_impl(c, weights, n_layers, k_pages, v_pages, num_pages, x, bt, max_blocks, ctx, max_ctx, B,
                           head_norm, head_w, head_wtype, vocab, logits, ws, ws_bytes, stream, nullptr);
}

gr_status gr_decode_stack_probed(const gr_layer_cfg* c, const gr_layer_weights* weights, int n_layers,
                                 void* const* k_pages, void* const* v_pages, int num_pages, float* x,
                                 const int32_t* bt, int max_blocks, const int32_t* ctx, int max_ctx, int B,
                                 const float* head_norm, const void* head_w, int head_wtype, int vocab,
                                 float* logits, void* ws, size_t ws_bytes, void* stream, int probe_stage,
                                 int probe_reps, void* const* ev_begin, void* const* ev_end) {
  if (probe_reps < 1 || probe_reps > 1000) return GR_ERR_SHAPE;
  Probe pr;
  pr.stage = probe_stage;
  pr.reps = probe_reps;
  pr.ev_begin = ev_begin;
  pr.ev_end = ev_end;
  return decode_stack_impl(c, weights, n_layers, k_pages, v_pages, num_pages, x, bt, max_blocks, ctx, max_ctx, B,
                           head_norm, head_w, head_wtype, vocab, logits, ws, ws_bytes, stream, &pr);
}

size_t gr_verify_stack_workspace_size(const gr_layer_cfg* c, int B, int T, int max_ctx, int vocab) {
  (void)vocab;
  if (B <= 0 || T <= 0 || (int64_t)B * T > kMaxRows) return 0;
  return layer_ws_bytes(c, B, T, max_ctx);
}

gr_status gr_verify_stack(const gr_layer_cfg* c, const gr_layer_weights* weights, int n_layers,
                          void* const* k_pages, void* const* v_pages, int num_pages, float* x, const int32_t* bt,
                          int max_blocks, const int32_t* ctx, int max_ctx, int B, int T, const float* head_norm,
                          const void* head_w, int head_wtype, int vocab, float* logits, void* ws, size_t ws_bytes,
                          void* stream) {
  if (T < 1) return GR_ERR_SHAPE;
  RowMap rm;
  rm.T = T;
  return decode_stack_impl(c, weights, n_layers, k_pages, v_pages, num_pages, x, bt, max_blocks, ctx, max_ctx, B,
                           head_norm, head_w, head_wtype, vocab, logits, ws, ws_bytes, stream, nullptr, rm);
}

size_t gr_mixed_stack_workspace_size(const gr_layer_cfg* c, int rows, int max_pos, int vocab) {
  (void)vocab;
  if (rows <= 0 || rows > kMaxRows || max_pos < 0) return 0;
  return layer_ws_bytes(c, rows, 1, max_pos);
}

gr_status gr_mixed_stack(const gr_layer_cfg* c, const gr_layer_weights* weights, int n_layers, void* const* k_pages,
                         void* const* v_pages, int num_pages, float* x, const int32_t* bt, int max_blocks,
                         const int32_t* row_seq, const int32_t* row_pos, int rows, int max_pos,
                         const float* head_norm, const void* head_w, int head_wtype, int vocab,
                         const int32_t* head_rows, int n_head_rows, float* logits, void* ws, size_t ws_bytes,
                         void* stream) {
  if (n_layers > 0 && (!row_seq || !row_pos) && rows > 0) return GR_ERR_NULL;
  RowMap rm;
  rm.seq = row_seq;
  rm.pos = row_pos;
  rm.head_rows = head_w ? head_rows : nullptr;
  rm.n_head = n_head_rows;
  return decode_stack_impl(c, weights, n_layers, k_pages, v_pages, num_pages, x, bt, max_blocks, nullptr, max_pos,
                           rows, head_norm, head_w, head_wtype, vocab, logits, ws, ws_bytes, stream, nullptr, rm);
}

gr_status gr_spec_accept(const int32_t* sampled, const int32_t* draft, int B, int T, int32_t* n_accepted,
                         void* stream) {
  if (B < 0 || T < 1 || T > 1024) return GR_ERR_SHAPE;
  if (B == 0) return GR_OK;
  if (!sampled || !draft || !n_accepted) return GR_ERR_NULL;
  if (!aligned(sampled, 4) || !aligned(draft, 4) || !aligned(n_accepted, 4)) return GR_ERR_ALIGN;
  gr_status s = check_device();
  if (s != GR_OK) return s;
  return check_launch(launch_spec_accept(sampled, draft, B, T, n_accepted, (hipStream_t)stream));
}

}  // extern "C"
