/*
 * oracle.c -- plain, slow fp64 CPU oracle of one continuous-batched, quantized
 * decode step of a dense Qwen3 / Llama-3 style layer stack.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * bench's CPU-baseline leg load this library.  It shares no code, header, table
 * or constant generator with the HIP path under continuous_quantized_decode_amd/.
 *
 * What it computes, and where the pages state it:
 *   - Leone, intro: active decode rows share matrix operations, each request keeps
 *     its own attention; "What ships": Q4_K and Q6_K weights; f32, f16 and q8 KV;
 *     an FP64 CPU oracle; each kernel has a scalar reference path.
 *   - tinyllm, Status feature list: RMSNorm, RoPE, GQA, SwiGLU MLP, causal
 *     attention; a physical KV page pool with a logical block table per sequence,
 *     and a retained contiguous comparison path; paged-reference decode gathers
 *     logical pages (Known limitations), 16-token pages.
 *   - LeatEngine, Run: the q8_0 cache as llama.cpp keeps it (32-element blocks with
 *     an fp16 scale).
 *   - Q5_K and Q8_0 weight rows (further GGUF weight formats; public layouts).
 *   - Leone, "What ships": greedy and stochastic sampling (temperature, top-k, top-p)
 *     after the output head, with fixed-point weights so every decision is an
 *     integer one (the readings sit with orc_sample below).
 * The byte layouts of Q4_K, Q6_K and q8_0 are not printed on the pages; they are
 * the public GGUF block formats.  Everything runs in fp64 on exactly decoded
 * inputs, with contiguous (gathered) K/V and one softmax over the whole context.
 * Sums run in index order.  Rows are independent, so a batch and its rows run
 * one at a time give identical results.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (see build.py).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q8_0 8
#define ORC_Q4_K 12
#define ORC_Q5_K 13
#define ORC_Q6_K 14
#define ORC_KV_F32 0
#define ORC_KV_F16 1
#define ORC_KV_Q8_0 2
#define ORC_ROPE_NEOX 0
#define ORC_ROPE_NORM 1
#define ORC_PAGE 16
#define ORC_QK 256
#define ORC_Q8B 32

/* ------------------------------------------------------------------ fp16 -- */

/* IEEE binary16 -> double, exact. */
double orc_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return sign ? -v : v;
}

/* double -> IEEE binary16, round to nearest, ties to even. */
uint16_t orc_f64_to_f16(double x) {
  if (isnan(x)) return 0x7E00;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a >= 65520.0) return sign | 0x7C00; /* halfway to 2^16 and above round to inf */
  if (a < ldexp(1.0, -14)) {              /* subnormal range, step 2^-24 */
    double q = nearbyint(ldexp(a, 24));   /* exact scaling; rint = ties-to-even */
    return sign | (uint16_t)q;            /* q == 1024 is the smallest normal */
  }
  int e2;
  frexp(a, &e2);      /* a = f * 2^e2, f in [0.5, 1) */
  int E = e2 - 1;     /* a = 1.x * 2^E */
  double r = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
  if (r >= 2048.0) { r = 1024.0; E += 1; }
  if (E + 15 >= 31) return sign | 0x7C00;
  return sign | (uint16_t)(((E + 15) << 10) | ((int)r - 1024));
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* --------------------------------------------------------- block decoders -- */

/* Q4_K super-block (GGUF): 256 weights in 144 bytes.
 *   [0,2) d (fp16), [2,4) dmin (fp16), [4,16) twelve bytes holding eight 6-bit
 *   scales and eight 6-bit mins, [16,144) 128 bytes of 4-bit quants.
 *   Sub-block j (32 weights) has weight w = d*sc[j]*q - dmin*m[j].
 *   Byte 32c+l of the quants holds weight 64c+l (low nibble, sub-block 2c) and
 *   weight 64c+32+l (high nibble, sub-block 2c+1). */
void orc_q4k_block(const uint8_t* blk, double* w) {
  double d = orc_f16_to_f64(rd16(blk)), dmin = orc_f16_to_f64(rd16(blk + 2));
  const uint8_t* s = blk + 4;
  const uint8_t* qs = blk + 16;
  int sc[8], mn[8];
  for (int j = 0; j < 4; ++j) {
    sc[j] = s[j] & 63;
    mn[j] = s[j + 4] & 63;
  }
  for (int j = 4; j < 8; ++j) {
    sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
    mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
  for (int c = 0; c < 4; ++c) {
    for (int l = 0; l < 32; ++l) {
      int lo = qs[32 * c + l] & 15, hi = qs[32 * c + l] >> 4;
      w[64 * c + l] = d * sc[2 * c] * lo - dmin * mn[2 * c];
      w[64 * c + 32 + l] = d * sc[2 * c + 1] * hi - dmin * mn[2 * c + 1];
    }
  }
}

/* Q5_K super-block (GGUF): 256 weights in 176 bytes.
 *   [0,2) d (fp16), [2,4) dmin (fp16), [4,16) the Q4_K packing of eight 6-bit scales
 *   and mins, [16,48) 32 bytes of high bits, [48,176) 128 bytes of low 4 bits.
 *   Sub-block j (32 weights) has w = d*sc[j]*q - dmin*m[j], q in [0,32).  Byte 32c+l
 *   of the low bits holds weight 64c+l (low nibble) and 64c+32+l (high nibble); their
 *   fifth bits are bits 2c and 2c+1 of high-bit byte l. */
void orc_q5k_block(const uint8_t* blk, double* w) {
  double d = orc_f16_to_f64(rd16(blk)), dmin = orc_f16_to_f64(rd16(blk + 2));
  const uint8_t* s = blk + 4;
  const uint8_t* qh = blk + 16;
  const uint8_t* qs = blk + 48;
  int sc[8], mn[8];
  for (int j = 0; j < 4; ++j) {
    sc[j] = s[j] & 63;
    mn[j] = s[j + 4] & 63;
  }
  for (int j = 4; j < 8; ++j) {
    sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
    mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
  for (int c = 0; c < 4; ++c) {
    for (int l = 0; l < 32; ++l) {
      int lo = (qs[32 * c + l] & 15) | (((qh[l] >> (2 * c)) & 1) << 4);
      int hi = (qs[32 * c + l] >> 4) | (((qh[l] >> (2 * c + 1)) & 1) << 4);
      w[64 * c + l] = d * sc[2 * c] * lo - dmin * mn[2 * c];
      w[64 * c + 32 + l] = d * sc[2 * c + 1] * hi - dmin * mn[2 * c + 1];
    }
  }
}

/* Q6_K super-block (GGUF): 256 weights in 210 bytes.
 *   [0,128) low 4 bits, [128,192) high 2 bits, [192,208) sixteen int8 scales,
 *   [208,210) d (fp16).  Weight i = d * scale[i/16] * (q_i - 32), q_i in [0,64).
 *   For half h and l in [0,32): the low-bit byte L=ql[64h+l] / L2=ql[64h+32+l] and
 *   the high-bit byte Q=qh[32h+l] give
 *     weight 128h+l    : (L  & 15) | ((Q >> 0) & 3) << 4
 *     weight 128h+l+32 : (L2 & 15) | ((Q >> 2) & 3) << 4
 *     weight 128h+l+64 : (L  >> 4) | ((Q >> 4) & 3) << 4
 *     weight 128h+l+96 : (L2 >> 4) | ((Q >> 6) & 3) << 4 */
void orc_q6k_block(const uint8_t* blk, double* w) {
  const uint8_t* ql = blk;
  const uint8_t* qh = blk + 128;
  const int8_t* sc = (const int8_t*)(blk + 192);
  double d = orc_f16_to_f64(rd16(blk + 208));
  for (int h = 0; h < 2; ++h) {
    for (int l = 0; l < 32; ++l) {
      int L = ql[64 * h + l], L2 = ql[64 * h + 32 + l], Q = qh[32 * h + l];
      int q[4] = {(L & 15) | (((Q >> 0) & 3) << 4), (L2 & 15) | (((Q >> 2) & 3) << 4),
                  (L >> 4) | (((Q >> 4) & 3) << 4), (L2 >> 4) | (((Q >> 6) & 3) << 4)};
      for (int r = 0; r < 4; ++r) {
        int i = 128 * h + l + 32 * r;
        w[i] = d * sc[i / 16] * (q[r] - 32);
      }
    }
  }
}

/* q8_0 block (GGUF): 32 values in 34 bytes, d (fp16) then 32 int8; x = d*q. */
void orc_q8_0_block(const uint8_t* blk, double* w) {
  double d = orc_f16_to_f64(rd16(blk));
  for (int i = 0; i < ORC_Q8B; ++i) w[i] = d * (double)(int8_t)blk[2 + i];
}

void orc_q4k_dequant(const uint8_t* blocks, int64_t n_blocks, double* out) {
  for (int64_t i = 0; i < n_blocks; ++i) orc_q4k_block(blocks + 144 * i, out + 256 * i);
}
void orc_q6k_dequant(const uint8_t* blocks, int64_t n_blocks, double* out) {
  for (int64_t i = 0; i < n_blocks; ++i) orc_q6k_block(blocks + 210 * i, out + 256 * i);
}
void orc_q8_0_dequant(const uint8_t* blocks, int64_t n_blocks, double* out) {
  for (int64_t i = 0; i < n_blocks; ++i) orc_q8_0_block(blocks + 34 * i, out + 32 * i);
}
void orc_q5k_dequant(const uint8_t* blocks, int64_t n_blocks, double* out) {
  for (int64_t i = 0; i < n_blocks; ++i) orc_q5k_block(blocks + 176 * i, out + 256 * i);
}

/* Bytes per 256 weights of a matrix row (Q8_0 rows are K/32 consecutive q8_0 blocks). */
static int wtype_block_bytes(int wtype) {
  return wtype == ORC_Q4_K ? 144 : wtype == ORC_Q6_K ? 210 : wtype == ORC_Q5_K ? 176 : wtype == ORC_Q8_0 ? 272 : 0;
}

static void decode_row(int wtype, const uint8_t* row, int K, double* w) {
  int nb = K / ORC_QK, bb = wtype_block_bytes(wtype);
  for (int j = 0; j < nb; ++j) {
    const uint8_t* blk = row + (size_t)bb * j;
    double* out = w + ORC_QK * j;
    if (wtype == ORC_Q4_K)
      orc_q4k_block(blk, out);
    else if (wtype == ORC_Q5_K)
      orc_q5k_block(blk, out);
    else if (wtype == ORC_Q8_0)
      for (int b = 0; b < ORC_QK / ORC_Q8B; ++b) orc_q8_0_block(blk + 34 * b, out + ORC_Q8B * b);
    else
      orc_q6k_block(blk, out);
  }
}

/* ------------------------------------------------------------------ GEMM -- */

/* y[b,n] = sum_k W[n,k] * x[b,k] with W decoded exactly from N rows of K/256
 * super-blocks each (row-major), summed in k order.  Returns 0, or -1 for an
 * unknown weight type or K not a multiple of 256. */
int orc_gemm(int wtype, const uint8_t* w, const double* x, double* y, int B, int N, int K) {
  int bb = wtype_block_bytes(wtype);
  if (!bb || K % ORC_QK) return -1;
  size_t row_bytes = (size_t)bb * (K / ORC_QK);
#pragma omp parallel
  {
    double* wr = (double*)malloc(sizeof(double) * K);
#pragma omp for schedule(dynamic, 8)
    for (int n = 0; n < N; ++n) {
      decode_row(wtype, w + row_bytes * n, K, wr);
      for (int b = 0; b < B; ++b) {
        const double* xb = x + (size_t)b * K;
        double s = 0.0;
        for (int k = 0; k < K; ++k) s += wr[k] * xb[k];
        y[(size_t)b * N + n] = s;
      }
    }
    free(wr);
  }
  return 0;
}

/* ------------------------------------------------------------- elementwise -- */

/* RMSNorm (tinyllm feature list): out = x / sqrt(mean(x^2) + eps) * g. */
void orc_rmsnorm(const double* x, const float* g, double eps, int n, double* out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * r * (double)g[i];
}

/* RoPE at position p: pair i in [0, D/2) has angle p * theta^(-2i/D); NeoX style
 * rotates (v[i], v[i+D/2]), "norm" style rotates (v[2i], v[2i+1]). */
void orc_rope(double* v, int D, int p, double theta, int style) {
  for (int i = 0; i < D / 2; ++i) {
    double phi = (double)p * pow(theta, -2.0 * i / D);
    double c = cos(phi), s = sin(phi);
    int ia = style == ORC_ROPE_NEOX ? i : 2 * i;
    int ib = style == ORC_ROPE_NEOX ? i + D / 2 : 2 * i + 1;
    double a = v[ia], b = v[ib];
    v[ia] = a * c - b * s;
    v[ib] = a * s + b * c;
  }
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* -------------------------------------------------------------- KV pages -- */
/* One pool per layer and per K/V.  A page holds 16 tokens of every KV head:
 * head g occupies bytes [g*HB, (g+1)*HB) of the page.  K heads are token-major
 * [16][D]; V heads are dim-major [D][16].  f32/f16 heads hold plain elements;
 * q8_0 heads hold 16*D int8 codes in that order, then fp16 scales [16][D/32]
 * (one per token per 32-element block along D). */

int64_t orc_head_bytes(int kv_dtype, int D) {
  if (kv_dtype == ORC_KV_F32) return (int64_t)ORC_PAGE * D * 4;
  if (kv_dtype == ORC_KV_F16) return (int64_t)ORC_PAGE * D * 2;
  if (kv_dtype == ORC_KV_Q8_0) return (int64_t)ORC_PAGE * D + ORC_PAGE * (D / ORC_Q8B) * 2;
  return -1;
}

/* exact value of element d of token `slot` in head block `hb` */
static double kv_read(const uint8_t* hb, int kv_dtype, int is_v, int D, int slot, int d) {
  size_t e = is_v ? (size_t)d * ORC_PAGE + slot : (size_t)slot * D + d;
  if (kv_dtype == ORC_KV_F32) {
    float f;
    memcpy(&f, hb + 4 * e, 4);
    return (double)f;
  }
  if (kv_dtype == ORC_KV_F16) return orc_f16_to_f64(rd16(hb + 2 * e));
  double sc = orc_f16_to_f64(rd16(hb + (size_t)ORC_PAGE * D + 2 * ((size_t)slot * (D / ORC_Q8B) + d / ORC_Q8B)));
  return sc * (double)(int8_t)hb[e];
}

/* q8_0 quantizer of one 32-element block, taken in fp32 as a kernel takes it:
 * amax = max|x|, d = amax/127, q = round-half-away(x/d) clamped to +-127,
 * stored scale = fp16(d); amax == 0 gives d = 0 and q = 0. */
void orc_q8_0_quantize_block(const float* x, int8_t* q, uint16_t* d16) {
  float amax = 0.0f;
  for (int i = 0; i < ORC_Q8B; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float d = amax / 127.0f;
  for (int i = 0; i < ORC_Q8B; ++i) {
    float r = d != 0.0f ? roundf(x[i] / d) : 0.0f;
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    q[i] = (int8_t)r;
  }
  *d16 = orc_f64_to_f16((double)d);
}

/* Store one token (all KV heads, vector v[Hkv*D]) at logical position pos of a row. */
void orc_kv_append(uint8_t* pool, int kv_dtype, int is_v, int Hkv, int D, const int32_t* bt_row, int pos,
                   const double* v) {
  int64_t HB = orc_head_bytes(kv_dtype, D);
  uint8_t* page = pool + (size_t)bt_row[pos / ORC_PAGE] * (size_t)(HB * Hkv);
  int slot = pos % ORC_PAGE;
  for (int g = 0; g < Hkv; ++g) {
    uint8_t* hb = page + (size_t)g * HB;
    const double* vg = v + (size_t)g * D;
    if (kv_dtype == ORC_KV_Q8_0) {
      for (int blk = 0; blk < D / ORC_Q8B; ++blk) {
        float xf[ORC_Q8B];
        int8_t q[ORC_Q8B];
        uint16_t d16;
        for (int i = 0; i < ORC_Q8B; ++i) xf[i] = (float)vg[blk * ORC_Q8B + i];
        orc_q8_0_quantize_block(xf, q, &d16);
        for (int i = 0; i < ORC_Q8B; ++i) {
          int d = blk * ORC_Q8B + i;
          size_t e = is_v ? (size_t)d * ORC_PAGE + slot : (size_t)slot * D + d;
          hb[e] = (uint8_t)q[i];
        }
        uint8_t* sp = hb + (size_t)ORC_PAGE * D + 2 * ((size_t)slot * (D / ORC_Q8B) + blk);
        sp[0] = (uint8_t)(d16 & 255);
        sp[1] = (uint8_t)(d16 >> 8);
      }
    } else {
      for (int d = 0; d < D; ++d) {
        size_t e = is_v ? (size_t)d * ORC_PAGE + slot : (size_t)slot * D + d;
        if (kv_dtype == ORC_KV_F32) {
          float f = (float)vg[d];
          memcpy(hb + 4 * e, &f, 4);
        } else {
          uint16_t h = orc_f64_to_f16(vg[d]);
          hb[2 * e] = (uint8_t)(h & 255);
          hb[2 * e + 1] = (uint8_t)(h >> 8);
        }
      }
    }
  }
}

/* Paged -> logical gather (tinyllm, Known limitations: the reference decode gathers
 * logical pages): tokens [0, n_tok) of one row into out[n_tok][Hkv][D], exact. */
void orc_gather_row(const uint8_t* pool, int kv_dtype, int is_v, int Hkv, int D, const int32_t* bt_row, int n_tok,
                    double* out) {
  int64_t HB = orc_head_bytes(kv_dtype, D);
  for (int t = 0; t < n_tok; ++t) {
    const uint8_t* page = pool + (size_t)bt_row[t / ORC_PAGE] * (size_t)(HB * Hkv);
    for (int g = 0; g < Hkv; ++g)
      for (int d = 0; d < D; ++d)
        out[((size_t)t * Hkv + g) * D + d] = kv_read(page + (size_t)g * HB, kv_dtype, is_v, D, t % ORC_PAGE, d);
  }
}

/* Gather for a batch: rows concatenated, row b contributes ctx_lens[b] tokens. */
void orc_gather_kv(const uint8_t* pool, int kv_dtype, int is_v, int Hkv, int D, const int32_t* block_table,
                   int max_blocks, const int32_t* ctx_lens, int B, double* out) {
  size_t off = 0;
  for (int b = 0; b < B; ++b) {
    orc_gather_row(pool, kv_dtype, is_v, Hkv, D, block_table + (size_t)b * max_blocks, ctx_lens[b], out + off);
    off += (size_t)ctx_lens[b] * Hkv * D;
  }
}

/* ------------------------------------------------------------- attention -- */

/* GQA decode attention of one query head over contiguous K/V of n_tok tokens
 * (layout [t][Hkv][D]) using KV head g: s_t = q.K_t / sqrt(D), softmax over all
 * t, o = sum_t w_t V_t. */
void orc_attend_head(const double* q, const double* K, const double* V, int n_tok, int Hkv, int D, int g, double* o) {
  double* s = (double*)malloc(sizeof(double) * (n_tok > 0 ? n_tok : 1));
  double scale = 1.0 / sqrt((double)D), mx = -INFINITY;
  for (int t = 0; t < n_tok; ++t) {
    const double* k = K + ((size_t)t * Hkv + g) * D;
    double a = 0.0;
    for (int d = 0; d < D; ++d) a += q[d] * k[d];
    s[t] = a * scale;
    if (s[t] > mx) mx = s[t];
  }
  double z = 0.0;
  for (int t = 0; t < n_tok; ++t) {
    s[t] = exp(s[t] - mx);
    z += s[t];
  }
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  for (int t = 0; t < n_tok; ++t) {
    const double* v = V + ((size_t)t * Hkv + g) * D;
    double w = s[t] / z;
    for (int d = 0; d < D; ++d) o[d] += w * v[d];
  }
  free(s);
}

/* Unnormalised partial over tokens [t0, t1): m = max s, l = sum e^(s-m),
 * o = sum e^(s-m) V.  (Used by the tests of the log-sum-exp merge.) */
void orc_attend_partial(const double* q, const double* K, const double* V, int t0, int t1, int Hkv, int D, int g,
                        double* o, double* m_out, double* l_out) {
  double scale = 1.0 / sqrt((double)D), mx = -INFINITY;
  int n = t1 - t0;
  double* s = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
  for (int t = t0; t < t1; ++t) {
    const double* k = K + ((size_t)t * Hkv + g) * D;
    double a = 0.0;
    for (int d = 0; d < D; ++d) a += q[d] * k[d];
    s[t - t0] = a * scale;
    if (s[t - t0] > mx) mx = s[t - t0];
  }
  double l = 0.0;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  for (int t = t0; t < t1; ++t) {
    double e = exp(s[t - t0] - mx);
    l += e;
    const double* v = V + ((size_t)t * Hkv + g) * D;
    for (int d = 0; d < D; ++d) o[d] += e * v[d];
  }
  *m_out = mx;
  *l_out = l;
  free(s);
}

/* Log-sum-exp merge of S partials: M = max m_s, L = sum l_s e^(m_s-M),
 * o = sum o_s e^(m_s-M) / L. */
void orc_lse_merge(const double* o_s, const double* m_s, const double* l_s, int S, int D, double* o) {
  double M = -INFINITY;
  for (int s = 0; s < S; ++s)
    if (m_s[s] > M) M = m_s[s];
  double L = 0.0;
  for (int s = 0; s < S; ++s) L += l_s[s] * exp(m_s[s] - M);
  for (int d = 0; d < D; ++d) {
    double a = 0.0;
    for (int s = 0; s < S; ++s) a += o_s[(size_t)s * D + d] * exp(m_s[s] - M);
    o[d] = a / L;
  }
}

/* Paged decode attention for a batch: gather each row's ctx_lens[b] tokens from
 * the pools, then attend every query head (q, out: [B][Hq][D]). */
void orc_paged_attention(const double* q, const uint8_t* k_pool, const uint8_t* v_pool, int kv_dtype,
                         const int32_t* block_table, int max_blocks, const int32_t* ctx_lens, int B, int Hq, int Hkv,
                         int D, double* out) {
  for (int b = 0; b < B; ++b) {
    int n = ctx_lens[b];
    double* K = (double*)malloc(sizeof(double) * ((size_t)n * Hkv * D + 1));
    double* V = (double*)malloc(sizeof(double) * ((size_t)n * Hkv * D + 1));
    const int32_t* bt = block_table + (size_t)b * max_blocks;
    orc_gather_row(k_pool, kv_dtype, 0, Hkv, D, bt, n, K);
    orc_gather_row(v_pool, kv_dtype, 1, Hkv, D, bt, n, V);
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < Hq; ++h)
      orc_attend_head(q + ((size_t)b * Hq + h) * D, K, V, n, Hkv, D, h / (Hq / Hkv), out + ((size_t)b * Hq + h) * D);
    free(K);
    free(V);
  }
}

/* ------------------------------------------------------------ the layer -- */

typedef struct {
  int hidden, n_q_heads, n_kv_heads, head_dim, ffn;
  double rms_eps, rope_theta;
  int rope_style, qk_norm, kv_dtype;
} orc_layer_cfg;

typedef struct {
  const float *attn_norm, *ffn_norm, *q_norm, *k_norm;
  const uint8_t *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
  int tq, tk, tv, to, tgate, tup, tdown;
} orc_layer_w;

/* Optional intermediates (any pointer may be NULL):
 *   q [B][Hq*D] after QK-norm and RoPE, k/v [B][Hkv*D] before storage rounding,
 *   attn [B][Hq*D] attention output, h1 [B][H] residual after attention,
 *   act [B][F] SwiGLU activation. */
typedef struct {
  double *q, *k, *v, *attn, *h1, *act;
} orc_layer_taps;

/* One decode layer for B rows; x [B][H] is read and overwritten with the layer
 * output.  ctx_lens[b] = tokens cached before this step; the new token is
 * appended at that position (pools modified), then attention covers ctx+1 tokens.
 * Returns 0, or -1 on an unsupported weight type. */
int orc_decode_layer(const orc_layer_cfg* c, const orc_layer_w* w, uint8_t* k_pool, uint8_t* v_pool, double* x,
                     const int32_t* block_table, int max_blocks, const int32_t* ctx_lens, int B,
                     const orc_layer_taps* taps) {
  int H = c->hidden, Hq = c->n_q_heads, Hkv = c->n_kv_heads, D = c->head_dim, F = c->ffn;
  int QD = Hq * D, KVD = Hkv * D;
  double* xn = (double*)malloc(sizeof(double) * (size_t)B * H);
  double* q = (double*)malloc(sizeof(double) * (size_t)B * QD);
  double* k = (double*)malloc(sizeof(double) * (size_t)B * KVD);
  double* v = (double*)malloc(sizeof(double) * (size_t)B * KVD);
  double* o = (double*)malloc(sizeof(double) * (size_t)B * QD);
  double* y = (double*)malloc(sizeof(double) * (size_t)B * (H > F ? H : F));
  double* g = (double*)malloc(sizeof(double) * (size_t)B * F);
  double* u = (double*)malloc(sizeof(double) * (size_t)B * F);
  int rc = 0;

  /* attention RMSNorm, then q = Wq xn, k = Wk xn, v = Wv xn (no biases) */
  for (int b = 0; b < B; ++b) orc_rmsnorm(x + (size_t)b * H, w->attn_norm, c->rms_eps, H, xn + (size_t)b * H);
  rc |= orc_gemm(w->tq, w->wq, xn, q, B, QD, H);
  rc |= orc_gemm(w->tk, w->wk, xn, k, B, KVD, H);
  rc |= orc_gemm(w->tv, w->wv, xn, v, B, KVD, H);
  if (rc) goto done;

  for (int b = 0; b < B; ++b) {
    int p = ctx_lens[b];
    double tmp[1024];
    /* QK-RMSNorm per head (Qwen3-shaped layers), then RoPE at position p */
    for (int h = 0; h < Hq; ++h) {
      double* qh = q + (size_t)b * QD + (size_t)h * D;
      if (c->qk_norm) {
        orc_rmsnorm(qh, w->q_norm, c->rms_eps, D, tmp);
        memcpy(qh, tmp, sizeof(double) * D);
      }
      orc_rope(qh, D, p, c->rope_theta, c->rope_style);
    }
    for (int h = 0; h < Hkv; ++h) {
      double* kh = k + (size_t)b * KVD + (size_t)h * D;
      if (c->qk_norm) {
        orc_rmsnorm(kh, w->k_norm, c->rms_eps, D, tmp);
        memcpy(kh, tmp, sizeof(double) * D);
      }
      orc_rope(kh, D, p, c->rope_theta, c->rope_style);
    }
    if (taps && taps->k) memcpy(taps->k + (size_t)b * KVD, k + (size_t)b * KVD, sizeof(double) * KVD);
    if (taps && taps->v) memcpy(taps->v + (size_t)b * KVD, v + (size_t)b * KVD, sizeof(double) * KVD);

    /* append the new token in storage precision, then read it back with the rest */
    const int32_t* bt = block_table + (size_t)b * max_blocks;
    orc_kv_append(k_pool, c->kv_dtype, 0, Hkv, D, bt, p, k + (size_t)b * KVD);
    orc_kv_append(v_pool, c->kv_dtype, 1, Hkv, D, bt, p, v + (size_t)b * KVD);
  }
  if (taps && taps->q) memcpy(taps->q, q, sizeof(double) * (size_t)B * QD);

  {
    int32_t* n_tok = (int32_t*)malloc(sizeof(int32_t) * B);
    for (int b = 0; b < B; ++b) n_tok[b] = ctx_lens[b] + 1;
    orc_paged_attention(q, k_pool, v_pool, c->kv_dtype, block_table, max_blocks, n_tok, B, Hq, Hkv, D, o);
    free(n_tok);
  }
  if (taps && taps->attn) memcpy(taps->attn, o, sizeof(double) * (size_t)B * QD);

  /* x1 = x + Wo o */
  rc |= orc_gemm(w->to, w->wo, o, y, B, H, QD);
  if (rc) goto done;
  for (size_t i = 0; i < (size_t)B * H; ++i) x[i] += y[i];
  if (taps && taps->h1) memcpy(taps->h1, x, sizeof(double) * (size_t)B * H);

  /* a = silu(Wg xn2) * (Wu xn2), out = x1 + Wd a */
  for (int b = 0; b < B; ++b) orc_rmsnorm(x + (size_t)b * H, w->ffn_norm, c->rms_eps, H, xn + (size_t)b * H);
  rc |= orc_gemm(w->tgate, w->w_gate, xn, g, B, F, H);
  rc |= orc_gemm(w->tup, w->w_up, xn, u, B, F, H);
  if (rc) goto done;
  for (size_t i = 0; i < (size_t)B * F; ++i) g[i] = orc_silu(g[i]) * u[i];
  if (taps && taps->act) memcpy(taps->act, g, sizeof(double) * (size_t)B * F);
  rc |= orc_gemm(w->tdown, w->w_down, g, y, B, H, F);
  if (rc) goto done;
  for (size_t i = 0; i < (size_t)B * H; ++i) x[i] += y[i];

done:
  free(xn); free(q); free(k); free(v); free(o); free(y); free(g); free(u);
  return rc ? -1 : 0;
}

/* Final RMSNorm and output head: logits[b] = Wout (rms(x_b) * g). */
int orc_output_head(const double* x, const float* norm, double eps, const uint8_t* w, int wtype, double* logits, int B,
                    int H, int vocab) {
  double* xn = (double*)malloc(sizeof(double) * (size_t)B * H);
  for (int b = 0; b < B; ++b) orc_rmsnorm(x + (size_t)b * H, norm, eps, H, xn + (size_t)b * H);
  int rc = orc_gemm(wtype, w, xn, logits, B, vocab, H);
  free(xn);
  return rc;
}

/* Threads the parallel loops above use (bookkeeping for timing reports; no arithmetic). */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------------------------------------
 * Sampling after the output head (Leone, "What ships": greedy and stochastic sampling with an
 * FP64 CPU oracle).  The pages name the feature and nothing of its arithmetic; the readings
 * taken here make every decision an integer one:
 *   - order: logits sorted by value, largest first, equal values by index ascending; NaN sorts
 *     last and -0 equals +0;
 *   - greedy (temperature <= 0 or NaN, 1/temperature not finite, top_k == 1, or a largest logit
 *     that is not finite): the first element of the order;
 *   - weight of element i: W_i = floor(2^31 e^d) with d = (l_i - l_max) * (1/T) in fp64, and
 *     W_i = 0 when d < -22 or d is NaN (e^-22 < 2^-31, so the floor is 0 there anyway);
 *   - top_k = k in [2, vocab): the first k elements of the order are kept, Wk their weight sum;
 *     otherwise Wk is the sum over the whole row;
 *   - top_p = p < 1: P = ceil(p Wk) clamped to [1, Wk]; the kept prefix ends at the first element
 *     whose running weight reaches P, Wp that running weight; otherwise Wp = Wk;
 *   - draw: U = floor(u Wp) clamped to [0, Wp - 1] for the caller's uniform u in [0, 1); the token
 *     is the first element of the order whose running weight exceeds U.
 * ------------------------------------------------------------------------------------------- */

/* e^d for -22 <= d <= 0 in fp64.  Cody and Waite's reduction d = k ln2 + r, k = rint(d / ln2),
 * with ln2 split into a high part whose low bits are zero (so k ln2_hi is exact) and a low part
 * (the fdlibm split); e^r from the Taylor series of the exponential to degree 13 in Horner form,
 * one fused multiply-add per step; then e^d = 2^k e^r. */
double orc_exp_neg(double d) {
  static const double ln2_hi = 0x1.62e42fee00000p-1, ln2_lo = 0x1.a39ef35793c76p-33;
  static const double inv_ln2 = 0x1.71547652b82fep+0;
  double c[14], f = 1.0;
  c[0] = 1.0;
  for (int n = 1; n <= 13; ++n) {
    f *= n; /* n! is exact in fp64 up to 22! */
    c[n] = 1.0 / f;
  }
  const double k = rint(d * inv_ln2);
  double r = fma(-k, ln2_hi, d);
  r = fma(-k, ln2_lo, r);
  double p = c[13];
  for (int n = 12; n >= 0; --n) p = fma(p, r, c[n]);
  return ldexp(p, (int)k);
}

/* Fixed-point weight of an element whose scaled logit difference is d. */
uint32_t orc_sample_weight(double d) {
  if (!(d >= -22.0)) return 0;
  return (uint32_t)floor(ldexp(orc_exp_neg(d), 31));
}

typedef struct {
  double l;
  int i, nan;
} OrcRank;

static int orc_rank_cmp(const void* a, const void* b) {
  const OrcRank* x = (const OrcRank*)a;
  const OrcRank* y = (const OrcRank*)b;
  if (x->nan != y->nan) return x->nan ? 1 : -1;
  if (!x->nan && x->l != y->l) return x->l > y->l ? -1 : 1;
  return (x->i > y->i) - (x->i < y->i);
}

/* One token per row.  temperature, top_p, u: B doubles; top_k: B ints.  wk_out and wp_out (may
 * be NULL) receive Wk and Wp (0 for a greedy row). */
int orc_sample(const float* logits, int B, int vocab, const double* temperature, const double* top_p,
               const int* top_k, const double* u, int32_t* tokens, uint64_t* wk_out, uint64_t* wp_out) {
  if (B < 0 || vocab < 1) return -1;
  OrcRank* e = (OrcRank*)malloc(sizeof(OrcRank) * (size_t)vocab);
  uint32_t* w = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)vocab);
  for (int b = 0; b < B; ++b) {
    const float* row = logits + (size_t)b * vocab;
    for (int i = 0; i < vocab; ++i) {
      e[i].l = (double)row[i];
      e[i].i = i;
      e[i].nan = isnan(row[i]) ? 1 : 0;
    }
    qsort(e, (size_t)vocab, sizeof(OrcRank), orc_rank_cmp);
    const double T = temperature[b], inv_t = 1.0 / T, lmax = e[0].l;
    if (wk_out) wk_out[b] = 0;
    if (wp_out) wp_out[b] = 0;
    if (!(T > 0.0) || !isfinite(inv_t) || top_k[b] == 1 || e[0].nan || !isfinite(lmax)) {
      tokens[b] = e[0].i;
      continue;
    }
    for (int j = 0; j < vocab; ++j) w[j] = orc_sample_weight((e[j].l - lmax) * inv_t);
    const int kk = (top_k[b] <= 0 || top_k[b] >= vocab) ? vocab : top_k[b];
    uint64_t wk = 0;
    for (int j = 0; j < kk; ++j) wk += w[j];
    uint64_t wp = wk;
    if (top_p[b] < 1.0) {
      const double pd = ceil(top_p[b] * (double)wk);
      const uint64_t P = !(pd > 1.0) ? 1 : (pd >= (double)wk ? wk : (uint64_t)pd);
      uint64_t cum = 0;
      for (int j = 0; j < vocab; ++j) {
        cum += w[j];
        if (cum >= P) {
          wp = cum;
          break;
        }
      }
    }
    const double x = floor(u[b] * (double)wp);
    const uint64_t U = x >= (double)wp ? wp - 1 : (x > 0.0 ? (uint64_t)x : 0);
    uint64_t cum = 0;
    int tok = e[0].i;
    for (int j = 0; j < vocab; ++j) {
      cum += w[j];
      if (cum > U) {
        tok = e[j].i;
        break;
      }
    }
    tokens[b] = tok;
    if (wk_out) wk_out[b] = wk;
    if (wp_out) wp_out[b] = wp;
  }
  free(e);
  free(w);
  return 0;
}
