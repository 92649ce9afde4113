/*
 * gr.h -- C ABI of the continuous-batched, quantized decode step on MI355X (gfx950).
 *
 * The operations follow the problem as the pages state it:
 *  - Leone, intro: the server batches active decode rows into shared matrix
 *    operations while each request keeps separate attention; "What ships": Q4_K and
 *    Q6_K weights, f32 / f16 / q8 KV storage, graph-replayed decode.
 *  - tinyllm, Status: a physical KV page pool, a logical block table per sequence,
 *    variable-length batched decode; Roadmap item 6: paged KV blocks behind a typed
 *    attention metadata boundary; Known limitations: 16-token pages.
 *  - LeatEngine, Run: a q8_0 KV cache as llama.cpp keeps it (32-element blocks,
 *    fp16 scale) in about half the memory of f16.
 *
 * Conventions for every call:
 *  - Pointers are device memory owned by the caller (weights, pools, activations,
 *    block tables, workspaces).  The library never allocates, frees or
 *    synchronizes; calls enqueue work on `stream` (a hipStream_t, NULL = the null
 *    stream) and return.  Results are valid once the stream reaches them.
 *  - Every check the host can make runs before anything is enqueued; a call that
 *    returns an error enqueued nothing.  Unknown enum values are rejected
 *    (GR_ERR_DTYPE), never ignored.  Capacity errors are returned before the
 *    capacity would be exceeded (GR_ERR_CAPACITY).
 *  - Device-resident preconditions are documented, not checked: block-table
 *    entries of the pages a row uses lie in [0, num_pages); ctx_lens[b] <= max_ctx.
 *  - B == 0 returns GR_OK and enqueues nothing.
 *  - Weight matrices are GGUF rows: row n of an N x K matrix is K/256 consecutive
 *    super-blocks (Q4_K: 144 B, Q5_K: 176 B, Q6_K: 210 B), or K/32 consecutive q8_0
 *    blocks (34 B: fp16 d, 32 int8), rows back to back.
 *    y[b][n] = sum_k W[n][k] * x[b][k].  K must be a multiple of 256.
 *  - KV pools (one K pool and one V pool per layer): page p holds 16 tokens of all
 *    KV heads; head g occupies bytes [g*HB, (g+1)*HB) of the page with
 *    HB = gr_kv_head_bytes(kv_dtype, head_dim).  K heads are token-major [16][D],
 *    V heads are dim-major [D][16].  f32 / f16 heads hold plain elements; q8_0 heads
 *    hold the 16*D int8 codes in that order followed by fp16 scales [16][D/32]
 *    (token t, block j covers elements 32j..32j+31 of that token).
 *  - The block table is int32 [B][max_blocks_per_row]; entry j of row b is the
 *    physical page holding that row's logical tokens 16j..16j+15.
 */
#ifndef GR_H_
#define GR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GR_ABI_VERSION 10

typedef enum {
  GR_OK = 0,
  GR_ERR_NULL = -1,      /* a required pointer is NULL */
  GR_ERR_SHAPE = -2,     /* a size or shape is out of the supported range */
  GR_ERR_DTYPE = -3,     /* unknown weight type, KV dtype or rope style */
  GR_ERR_ALIGN = -4,     /* a pointer lacks the stated alignment */
  GR_ERR_WORKSPACE = -5, /* workspace missing or smaller than the size query returns */
  GR_ERR_CAPACITY = -6,  /* max_ctx + 1 tokens do not fit max_blocks_per_row pages */
  GR_ERR_DEVICE = -7,    /* the current device is not gfx950 */
  GR_ERR_LAUNCH = -8     /* a kernel launch failed; see gr_last_hip_error() */
} gr_status;

typedef enum { GR_KV_F32 = 0, GR_KV_F16 = 1, GR_KV_Q8_0 = 2 } gr_kv_dtype;
/* values are the GGUF tensor type ids */
/* GGUF type ids.  Q4_K / Q6_K are the decode step's formats (Leone, What ships); Q5_K
 * and Q8_0 weight rows are accepted by every GEMM (the tile-loop kernel stays Q4_K /
 * Q6_K). */
typedef enum { GR_W_Q8_0 = 8, GR_W_Q4_K = 12, GR_W_Q5_K = 13, GR_W_Q6_K = 14 } gr_wtype;
/* NEOX rotates (v[i], v[i+D/2]); NORM rotates (v[2i], v[2i+1]) */
typedef enum { GR_ROPE_NEOX = 0, GR_ROPE_NORM = 1 } gr_rope_style;

#define GR_PAGE_SIZE 16

int gr_abi_version(void);
const char* gr_status_str(int status);
/* hipError_t of the most recent GR_ERR_LAUNCH on the calling thread (0 if none). */
int gr_last_hip_error(void);
/* Bytes of one KV head's block inside a page, or -1 for an unknown dtype. */
int64_t gr_kv_head_bytes(int kv_dtype, int head_dim);

/* ---------------------------------------------------------------- dequant --
 * Test exports (bit-exactness).  Leone, "What ships": Q4_K and Q6_K weights; the
 * block layouts are the public GGUF formats.  out receives 256 (Q4_K, Q6_K) or 32
 * (q8_0, 34-byte GGUF blocks) fp32 values per block.  Q4_K values are
 * fp32(d*sc)*q - fp32(dmin*m) rounded once (one fused multiply-add); Q6_K and
 * q8_0 values are exact in fp32.  blocks: 2-byte aligned; out: 4-byte aligned. */
gr_status gr_q4k_dequant(const void* blocks, int64_t n_blocks, float* out, void* stream);
gr_status gr_q6k_dequant(const void* blocks, int64_t n_blocks, float* out, void* stream);
gr_status gr_q8_0_dequant(const void* blocks, int64_t n_blocks, float* out, void* stream);

/* ------------------------------------------------------------------ GEMM --
 * Fused-dequant skinny GEMM (Leone, intro: shared matrix operations over the
 * active rows).  x: f32 [B][K], y: f32 [B][N], both row-major, 16-byte aligned;
 * wblocks 16-byte aligned.  1 <= B <= 512, N >= 1, K % 256 == 0, K <= 65536.  Above
 * 64 rows (prompt chunks; Leone, What ships: chunked prefill) a 2-D tiled kernel runs,
 * for Q4_K and Q6_K only: Q5_K and Q8_0 above 64 rows return GR_ERR_DTYPE.
 * The workspace (16-byte aligned) holds the packed activations; size it with
 * gr_gemm_workspace_size.  Up to 64 rows the weights are streamed once; above, once
 * per group of 32 (Q4_K) or 16 (Q6_K) rows, from L2 after the first. */
size_t gr_gemm_workspace_size(int B, int N, int K);
gr_status gr_q4k_gemm(const void* wblocks, const float* x, float* y, int B, int N, int K, void* workspace,
                      size_t ws_bytes, void* stream);
gr_status gr_q6k_gemm(const void* wblocks, const float* x, float* y, int B, int N, int K, void* workspace,
                      size_t ws_bytes, void* stream);
gr_status gr_q5k_gemm(const void* wblocks, const float* x, float* y, int B, int N, int K, void* workspace,
                      size_t ws_bytes, void* stream);
gr_status gr_q8_0_gemm(const void* wblocks, const float* x, float* y, int B, int N, int K, void* workspace,
                       size_t ws_bytes, void* stream);

/* Measurement aid: one read-only pass over `bytes` bytes at p (16-byte aligned, a
 * multiple of 16) by a plain streaming kernel of GR_STREAM_READ_WORDS workgroups
 * (grid-stride, 16-byte loads, eight 1 KB loads in flight per wave).  out[w] (uint32,
 * GR_STREAM_READ_WORDS of them) receives workgroup w's XOR of the first and last dword
 * of every 16-byte unit it read; the XOR of all out[w] covers the whole buffer.  Its
 * rate is the practical read ceiling the decode step's kernels are compared with. */
#define GR_STREAM_READ_WORDS 2048
gr_status gr_stream_read(const void* p, size_t bytes, uint32_t* out, void* stream);

/* Launch shape of one fused-dequant GEMM launch (a profiling aid: it names the
 * dispatch a counter or trace row belongs to).  rows: output rows of the launch (for
 * several matrices sharing one launch, the sum of each one's rows rounded up to 16;
 * for a gate/up pair, rows = F).  epi: 0 plain store, 1 residual update, 2 gate/up
 * pair with SwiGLU.  Returns which kernel runs (tile_loop 0: the split-K kernel
 * gemm_kernel<type, nt, btn, maxt, aligned>; 1: the tile-loop kernel
 * gemm_tl_kernel<type, nt, aligned, ring, btn> with maxt = 512; 2: the many-row
 * kernel gemm_mm_kernel<type, aligned>, 512 threads, nt = 2 tiles per wave and btn = 4
 * (Q4_K) or 2 (Q6_K) activation tiles per workgroup; 3: the whole-tile tile loop
 * gemm_tlw_kernel<mode>, Q4_K gate/up pairs (mode 2) or plain stores (mode 0) at one
 * activation tile, one wave per 256 of K, maxt = 1024; 5: the same for a Q4_K residual
 * update (mode 1); 4: the K-chunk kernel gemm_kcw_kernel, a Q6_K residual update at one
 * activation tile, K a multiple of 2048), its template
 * parameters (16-row tiles per workgroup or group nt, 8-row batch tiles btn, launch
 * bound maxt) and the grid and workgroup sizes in threads, as launched by every entry
 * point above for these sizes.  GR_ERR_NULL for a null output pointer, GR_ERR_DTYPE for
 * an unknown type, GR_ERR_SHAPE for rows, K, B or epi out of range. */
gr_status gr_gemm_launch_shape(int wtype, int rows, int K, int B, int epi, int* tile_loop, int* nt, int* btn,
                               int* maxt, int* grid_threads, int* block_threads);

/* ------------------------------------------------------------- attention --
 * Typed attention metadata (tinyllm, Roadmap item 6). */
typedef struct {
  int n_q_heads, n_kv_heads, head_dim; /* head_dim in {64, 128}; n_q_heads % n_kv_heads == 0, ratio <= 8 */
  int page_size;                       /* must be 16 */
  int kv_dtype;                        /* gr_kv_dtype */
  int num_pages, max_blocks_per_row, max_ctx;
  float scale;                         /* softmax scale, normally 1/sqrt(head_dim) */
} gr_attn_meta;

/* Per-row GQA decode attention over paged KV (Leone, intro: each request keeps
 * its own attention; tinyllm: pages addressed through a logical block table).
 * q, out: f32 [B][n_q_heads][head_dim]; row b attends its first ctx_lens[b] tokens
 * (1 <= ctx_lens[b] <= max_ctx, all already in the pools); query head h uses KV head
 * h / (n_q_heads / n_kv_heads).  out[b][h] = sum_t softmax_t(scale * q.k_t) v_t.
 * The context is cut into page-aligned ranges processed by separate workgroups whose
 * softmax states the last one to finish merges by log-sum-exp.  Pools and q 16-byte
 * aligned.  GR_ERR_CAPACITY when max_ctx needs more ranges than one merge takes
 * (see gr_attn_launch_shape).  The workspace holds per-row arrival counters that
 * the call clears first: calls that share a workspace must not overlap. */
size_t gr_paged_decode_attn_workspace_size(const gr_attn_meta* m, int B);
gr_status gr_paged_decode_attn(const float* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                               const int32_t* ctx_lens, float* out, int B, const gr_attn_meta* m, void* workspace,
                               size_t ws_bytes, void* stream);

/* gr_paged_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments, kernels and results, without the workspace arguments.  Its
 * workspace lives in a static array of GR_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each device it runs on until the process ends; the call allocates nothing
 * (the array's device address is looked up once per device, on the first call with
 * that device current).  GR_ERR_WORKSPACE when the call needs more than the array
 * (gr_paged_decode_attn_workspace_size(m, B) > GR_NOALLOC_SCRATCH_BYTES); the other
 * errors as gr_paged_decode_attn.  Every call on a device shares that device's array,
 * which keeps the last call's contents (the call clears its arrival counters itself):
 * calls that overlap on one device race, whatever their streams. */
#define GR_NOALLOC_SCRATCH_BYTES (16u << 20)
gr_status gr_paged_decode_attn_noalloc(const float* q, const void* k_pages, const void* v_pages,
                                       const int32_t* block_table, const int32_t* ctx_lens, float* out, int B,
                                       const gr_attn_meta* m, void* stream);

/* Launch shape of the decode attention for rows of up to max_tokens attended tokens
 * (profiling aid and test of the page walk): waves per workgroup, pages per wave, the
 * most workgroups one (row, KV head) takes, and the grid in threads for B rows and
 * n_kv_heads heads.  GR_ERR_CAPACITY when max_tokens needs more workgroups than the
 * merging workgroup takes (the decode layer then rejects max_ctx + 1 as well). */
gr_status gr_attn_launch_shape(int kv_dtype, int B, int n_kv_heads, int max_tokens, int* waves_per_wg,
                               int* pages_per_wave, int* wg_per_row, long long* grid_threads);

/* Test export (bit-exactness of the page walk): decode the first ctx_lens[b] tokens
 * of each row of one pool (is_v selects the V layout) into out f32
 * [B][max_ctx][n_kv_heads][head_dim]; slots at or beyond ctx_lens[b] are untouched. */
gr_status gr_paged_gather_kv(const void* pages, int is_v, const int32_t* block_table, const int32_t* ctx_lens, int B,
                             const gr_attn_meta* m, float* out, void* stream);

/* ----------------------------------------------------------- decode layer --
 * One decode layer of a dense Qwen3 / Llama-3 stack (tinyllm, Status: RMSNorm,
 * RoPE, GQA, SwiGLU MLP; Leone: Q4_K / Q6_K weights, f32 / f16 / q8 KV). */
typedef struct {
  int hidden, n_q_heads, n_kv_heads, head_dim, ffn;
  float rms_eps;
  double rope_theta;
  int rope_style; /* gr_rope_style */
  int qk_norm;    /* 1: per-head RMSNorm of q and k before RoPE (Qwen3) */
  int kv_dtype;   /* gr_kv_dtype */
  int page_size;  /* must be 16 */
} gr_layer_cfg;

typedef struct {
  const float *attn_norm, *ffn_norm; /* f32 [hidden] */
  const float *q_norm, *k_norm;      /* f32 [head_dim]; NULL unless qk_norm */
  const void *wq, *wk, *wv;          /* [Hq*D x hidden], [Hkv*D x hidden], [Hkv*D x hidden] */
  const void* wo;                    /* [hidden x Hq*D] */
  const void *w_gate, *w_up;         /* [ffn x hidden] */
  const void* w_down;                /* [hidden x ffn] */
  int tq, tk, tv, to, tgate, tup, tdown; /* gr_wtype of each matrix */
} gr_layer_weights;

/* x: f32 [B][hidden], the residual stream, read and overwritten with the layer
 * output.  ctx_lens[b] = tokens already cached for row b (0 <= ctx_lens[b] <=
 * max_ctx); the step computes the new token's k and v, stores them at logical
 * position ctx_lens[b] (page block_table[b][ctx_lens[b]/16], slot ctx_lens[b]%16;
 * f32 / f16 round to nearest even; q8_0 per 32-element block: amax, d = amax/127,
 * codes round(x/d) half away from zero, scale fp16(d)), and attends ctx_lens[b]+1
 * tokens.  ctx_lens is not advanced (the caller does that).  Requires
 * max_ctx + 1 <= 16 * max_blocks_per_row (else GR_ERR_CAPACITY). */
size_t gr_decode_layer_workspace_size(const gr_layer_cfg* c, int B, int max_ctx);
gr_status gr_decode_layer(const gr_layer_cfg* c, const gr_layer_weights* w, void* k_pages, void* v_pages,
                          int num_pages, float* x, const int32_t* block_table, int max_blocks_per_row,
                          const int32_t* ctx_lens, int max_ctx, int B, void* workspace, size_t ws_bytes,
                          void* stream);

/* Final RMSNorm and output head (Leone: sampling follows the logits):
 * logits f32 [B][vocab] = W (rms(x_b) * norm), W [vocab x hidden]. */
size_t gr_output_head_workspace_size(int B, int hidden, int vocab);
gr_status gr_output_head(const float* x, const float* norm, float eps, const void* w, int wtype, float* logits,
                         int B, int hidden, int vocab, void* workspace, size_t ws_bytes, void* stream);

/* Token sampling after the output head (Leone, "What ships": greedy and stochastic
 * sampling).  The pages fix no formula; this call defines one in which every decision is
 * an integer one, so a result is reproducible bit for bit:
 *  - order: a row's logits by value, largest first, equal values by index ascending;
 *    NaN sorts last and -0 equals +0;
 *  - greedy rows (temperature <= 0 or NaN, 1/temperature not finite, top_k == 1, or a
 *    largest logit that is not finite) take the first element of the order;
 *  - otherwise element i weighs W_i = floor(2^31 e^d), d = (l_i - l_max) * (1/temperature)
 *    in fp64 (W_i = 0 for d < -22 or NaN), e^d evaluated by Cody-Waite reduction and a
 *    degree-13 Taylor polynomial with fused multiply-adds;
 *  - top_k = k with 1 < k < vocab: Wk = running weight of the k-th element of the order,
 *    else the row's total weight;
 *  - top_p = p < 1: P = ceil(p * Wk) (fp64 product) clamped to [1, Wk]; Wp = running
 *    weight of the first element whose running weight reaches P, else Wp = Wk;
 *  - draw: U = floor(u * Wp) clamped to [0, Wp - 1]; the token is the first element of
 *    the order whose running weight exceeds U.
 * params: device array [B] of gr_sample_params (8-byte aligned).  u is the caller's
 * uniform random number for the row (a seeded generator of the caller's choice).
 * logits: f32 [B][vocab], 1 <= vocab <= 262144.  tokens: int32 [B].  kept_weight: NULL
 * or uint64 [B][2] receiving (Wk, Wp), (0, 0) for greedy rows.  The workspace holds
 * per-row weights and histograms; the call issues three kernels and no host
 * synchronization (capturable in a HIP graph).  B > 65535 is GR_ERR_SHAPE. */
typedef struct {
  double temperature;
  double top_p;
  double u;
  int32_t top_k;
  int32_t reserved;
} gr_sample_params;

size_t gr_sample_workspace_size(int B, int vocab);
gr_status gr_sample(const float* logits, int B, int vocab, const gr_sample_params* params, int32_t* tokens,
                    uint64_t* kept_weight, void* workspace, size_t ws_bytes, void* stream);

/* Whole decode step: n_layers layers in order (layer l uses weights[l], k_pages[l],
 * v_pages[l]; host arrays of device pointers), then, when head_w is not NULL, the
 * final norm and output head into logits.  One workspace of
 * gr_decode_stack_workspace_size bytes serves every layer.  Suitable for capture
 * into one HIP graph (a fixed sequence of kernel launches, no host syncs). */
size_t gr_decode_stack_workspace_size(const gr_layer_cfg* c, int B, int max_ctx, int vocab);
gr_status gr_decode_stack(const gr_layer_cfg* c, const gr_layer_weights* weights, int n_layers, void* const* k_pages,
                          void* const* v_pages, int num_pages, float* x, const int32_t* block_table,
                          int max_blocks_per_row, const int32_t* ctx_lens, int max_ctx, int B,
                          const float* head_norm, const void* head_w, int head_wtype, int vocab, float* logits,
                          void* workspace, size_t ws_bytes, void* stream);

/* Exact speculative verification (Leone, "What ships": exact speculative verification).
 * gr_verify_stack is the decode stack for T tokens per row in one step: x [B*T][hidden]
 * (row b*T + j is token j of sequence b, at position ctx_lens[b] + j) holds the inputs
 * (the sequence's last accepted token, then T-1 proposed tokens); every token's K/V is
 * appended at its position and every token attends to the sequence's cached tokens and
 * to the step's tokens at or before it, exactly as T decode steps would.  Returns the
 * outputs in x and, with a head, logits [B*T][vocab].  B*T <= 512 (above 64, Q4_K / Q6_K
 * weights only, else GR_ERR_DTYPE);
 * max_ctx + T <= 16 * max_blocks_per_row (else GR_ERR_CAPACITY).  T = 1 is gr_decode_stack.
 * gr_spec_accept: sampled [B][T] holds the target's token after each position (for
 * example gr_sample over the verify logits, one uniform per position), draft [B][T] the
 * step's input tokens; n_accepted[b] = the number of leading j < T-1 with
 * sampled[b][j] == draft[b][j+1].  The sequence then emits sampled[b][0..n_accepted[b]].
 * With deterministic proposals every emitted token follows the target's own
 * distribution, so the acceptance is exact. */
size_t gr_verify_stack_workspace_size(const gr_layer_cfg* c, int B, int T, int max_ctx, int vocab);
gr_status gr_verify_stack(const gr_layer_cfg* c, const gr_layer_weights* weights, int n_layers, void* const* k_pages,
                          void* const* v_pages, int num_pages, float* x, const int32_t* block_table,
                          int max_blocks_per_row, const int32_t* ctx_lens, int max_ctx, int B, int T,
                          const float* head_norm, const void* head_w, int head_wtype, int vocab, float* logits,
                          void* workspace, size_t ws_bytes, void* stream);
gr_status gr_spec_accept(const int32_t* sampled, const int32_t* draft, int B, int T, int32_t* n_accepted,
                         void* stream);

/* Mixed step (continuous batching with chunked prefill; Leone, What ships: chunked
 * prefill, continuous decode batching; Leone, intro: decode rows and prompt chunks in one
 * schedule).  Row r of x [rows][hidden] is the token at position row_pos[r] of sequence
 * row_seq[r] (device int32 arrays; block_table row row_seq[r]).  Every row's K/V is stored
 * at its position, then every row attends to positions 0..row_pos[r] of its sequence.  A
 * step can hold decode rows (one token at the cached length), verification runs and
 * prompt chunks (consecutive positions), in any row order.  Device-resident
 * preconditions (documented, not checked): the positions of a sequence's rows in one step
 * are distinct and, together with the tokens cached before the step, cover 0..max of them;
 * row_pos[r] <= max_pos.  1 <= rows <= 512 (above 64, Q4_K / Q6_K weights only, else
 * GR_ERR_DTYPE); max_pos + 1 <= 16 * max_blocks_per_row (else
 * GR_ERR_CAPACITY).  With a head: logits [rows][vocab], or, when head_rows (device int32
 * [n_head_rows], 1 <= n_head_rows <= rows) is set, logits [n_head_rows][vocab] of rows
 * head_rows[i] only (a prompt chunk needs the logits of its last token alone; indices
 * are clamped to [0, rows)). */
size_t gr_mixed_stack_workspace_size(const gr_layer_cfg* c, int rows, int max_pos, int vocab);
gr_status gr_mixed_stack(const gr_layer_cfg* c, const gr_layer_weights* weights, int n_layers, void* const* k_pages,
                         void* const* v_pages, int num_pages, float* x, const int32_t* block_table,
                         int max_blocks_per_row, const int32_t* row_seq, const int32_t* row_pos, int rows, int max_pos,
                         const float* head_norm, const void* head_w, int head_wtype, int vocab,
                         const int32_t* head_rows, int n_head_rows, float* logits, void* workspace, size_t ws_bytes,
                         void* stream);

/* Timing probe (profiling hook): the same launches as gr_decode_stack, except that
 * the launches of stage `probe_stage` are issued `probe_reps` times (1..1000) in a
 * row with events attached to their dispatches (hipExtLaunchKernel): ev_begin[l] is
 * recorded when the stage's first kernel of layer l starts and ev_end[l] when its last
 * one ends (ev_*[0] for the pack and head stages), so the interval is the kernels'
 * execution alone.  Repeating a stage recomputes the same outputs, except that the
 * residual stages (Wo, down) add their product to x once per repetition, so x is
 * meaningful only with probe_reps == 1.  ev_begin / ev_end are host arrays of
 * hipEvent_t with n_layers entries (1 for GR_STAGE_HEAD and GR_STAGE_PACK), created by
 * the caller.  Not for use under stream capture.  Errors as gr_decode_stack;
 * GR_ERR_SHAPE for a stage or repetition count out of range. */
typedef enum {
  GR_STAGE_PACK = 0,       /* RMSNorm input pack of the first layer (or of the head) */
  GR_STAGE_QKV = 1,        /* q, k, v GEMM */
  GR_STAGE_ATTN = 2,       /* QK-norm, RoPE, KV append, split attention */
  GR_STAGE_ATTN_MERGE = 3, /* log-sum-exp merge + pack of the Wo input */
  GR_STAGE_WO = 4,         /* output projection + residual + pack of the FFN input */
  GR_STAGE_GATE_UP = 5,    /* gate and up GEMM + SwiGLU + pack of the down input */
  GR_STAGE_DOWN = 6,       /* down projection + residual + pack of the next input */
  GR_STAGE_HEAD = 7        /* output head GEMM */
} gr_stage;

gr_status gr_decode_stack_probed(const gr_layer_cfg* c, const gr_layer_weights* weights, int n_layers,
                                 void* const* k_pages, void* const* v_pages, int num_pages, float* x,
                                 const int32_t* block_table, int max_blocks_per_row, const int32_t* ctx_lens,
                                 int max_ctx, int B, const float* head_norm, const void* head_w, int head_wtype,
                                 int vocab, float* logits, void* workspace, size_t ws_bytes, void* stream,
                                 int probe_stage, int probe_reps, void* const* ev_begin,
                                 void* const* ev_end);

#ifdef __cplusplus
}
#endif

#endif /* GR_H_ */
