// sample.hip -- token sampling after the output head: greedy argmax and seeded
// temperature / top-k / top-p draws (Leone, "What ships": greedy and stochastic
// sampling with an FP64 CPU oracle).
//
// The pages give no formula, so the operation is defined with integer decisions only:
//   order   logits by value, largest first, equal values by index ascending (NaN last,
//           -0 == +0), encoded as the 50-bit composite (order_key << 18) | (2^18-1 - i),
//           larger composite first;
//   weight  W_i = floor(2^31 e^d), d = (l_i - l_max) * (1/T) in fp64 (0 for d < -22 or NaN);
//   top-k   Wk = running weight of the k-th element of the order (the row total when off);
//   top-p   P = ceil(p Wk) clamped to [1, Wk]; Wp = running weight of the first element
//           whose running weight reaches P (Wk when off);
//   draw    U = floor(u Wp) clamped to [0, Wp-1]; the token is the first element whose
//           running weight exceeds U.
// Every cut is "the first element of the order whose running count or weight reaches a
// target", so all three are one select over the whole order, never restricted to a set.
//
// Kernels, launched back to back on the caller's stream:
//   1. sample_max    (row chunks of 4096, 256 threads): per-chunk packed (key, index)
//                    maximum; clears the row's level-1 histogram.
//   2. sample_hist   (row chunks of 4096, 512 threads): row maximum from the chunk maxima;
//                    greedy rows write their token and stop.  Otherwise the weight of every
//                    element goes into a 4096-bin histogram of the key's top 12 bits (count
//                    and weight packed in one LDS word per bin, then added to the row's
//                    histogram), and every 256-element segment records its largest composite
//                    and the largest key among its other elements.
//   3. sample_select (one 512-thread workgroup per row).  The three cuts all fall in the
//                    order's prefix that ends in the level-1 bin where the first cut that
//                    applies (top-k count, else top-p weight, else the draw) lands; the
//                    histogram's running sums name that bin exactly.  A prefix of at most
//                    8192 elements is gathered into LDS: a segment whose second key lies below
//                    the bin gives its top element from its record, the other segments that
//                    reach the bin are read, and weights are recomputed for what was gathered.
//                    Up to 256 gathered elements are ranked against each other once and every
//                    cut is a lookup; more go through 10-bit LDS histogram levels until the
//                    cut's bucket holds at most 256 members, which are then ranked.  A longer
//                    prefix takes the general route: each cut gathers its own bin with a row
//                    pass, after 8-bit row-pass histogram levels while the bin exceeds 8192.
#include <hip/hip_runtime.h>

#include "gr_internal.h"

namespace gr {
namespace {

constexpr int kChunk = 4096;      // elements per workgroup of the max kernel (<= 64 chunks per row)
constexpr int kHistChunk = 4096;  // elements per workgroup of the histogram kernel
constexpr int kHistThreads = 512;
constexpr int kWideThreads = 256;
constexpr int kSeg = 256;         // elements per segment: one wave of the histogram kernel, 4 per lane
constexpr int kSegTop = 4;        // largest composites each segment records
constexpr int kBins1 = 4096;      // level 1: top 12 bits of the order key
constexpr int kSelThreads = 512;
constexpr int kCap = 8192;        // elements a select can hold in LDS
constexpr int kIdxBits = 18;      // vocab <= 2^18
constexpr int kCompBits = 32 + kIdxBits;
constexpr uint32_t kIdxMask = (1u << kIdxBits) - 1u;
constexpr int kMaxSegs = (1 << kIdxBits) / kSeg;  // two per select thread

struct SampleWs {
  uint64_t* cmax;  // [B][nch]  packed (key, 2^32-1 - index) chunk maxima
  uint32_t* hcnt;  // [B][kBins1]
  uint64_t* hsum;  // [B][kBins1]
  uint64_t* segtop;  // [B][nseg][kSegTop] largest composites of each 256-element segment, descending
  uint32_t* segsec;  // [B][nseg] largest key of the segment's other elements (0 if none)
};

// Monotone map of a float to an unsigned key: larger float, larger key; -0 maps as +0;
// NaN maps below everything.
__device__ inline uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (f != f) return 0u;
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline uint64_t composite(uint32_t key, uint32_t i) {
  return ((uint64_t)key << kIdxBits) | (uint64_t)(kIdxMask - i);
}

constexpr double inv_fact(int n) {
  double f = 1.0;
  for (int i = 2; i <= n; ++i) f *= i;
  return 1.0 / f;
}

// Fixed-point weight floor(2^31 e^d) of a scaled logit difference d <= 0, in fp64: Cody and
// Waite's reduction d = k ln2 + r with k = rint(d / ln2) and ln2 in two parts (the high
// part's low 21 bits are zero, the fdlibm split), the Taylor series of e^r to degree 13 in
// Horner form, one fused multiply-add per step, then the exact scaling by 2^(k + 31).
// Below d = -22 the weight is 0 (e^-22 < 2^-31).
__device__ inline uint32_t sample_weight(double d) {
#pragma clang fp contract(off)
  if (!(d >= -22.0)) return 0u;
  const double ln2_hi = 0x1.62e42fee00000p-1, ln2_lo = 0x1.a39ef35793c76p-33;
  const double inv_ln2 = 0x1.71547652b82fep+0;
  const double k = __builtin_rint(d * inv_ln2);
  double r = __builtin_fma(-k, ln2_hi, d);
  r = __builtin_fma(-k, ln2_lo, r);
  double p = inv_fact(13);
#pragma unroll
  for (int n = 12; n >= 0; --n) p = __builtin_fma(p, r, inv_fact(n));
  return (uint32_t)__builtin_floor(__builtin_ldexp(p, (int)k + 31));
}

// Wave scans and reductions use DPP lane shifts (row shifts inside 16-lane rows, then the
// row broadcasts of lanes 15 and 31): no LDS round trips.
template <int kCtrl, int kRowMask>
__device__ inline uint64_t dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, kCtrl, kRowMask, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), kCtrl, kRowMask, 0xF, true);
  return ((uint64_t)hi << 32) | lo;
}

__device__ inline uint64_t lane63(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ inline uint64_t wave_scan_dpp(uint64_t v) {
  v += dpp64<0x111, 0xF>(v);  // row_shr:1
  v += dpp64<0x112, 0xF>(v);  // row_shr:2
  v += dpp64<0x114, 0xF>(v);  // row_shr:4
  v += dpp64<0x118, 0xF>(v);  // row_shr:8
  v += dpp64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the 64 lanes (every lane receives it).
__device__ inline uint64_t wave_max_dpp(uint64_t v) {
  v = umax64(v, dpp64<0x111, 0xF>(v));
  v = umax64(v, dpp64<0x112, 0xF>(v));
  v = umax64(v, dpp64<0x114, 0xF>(v));
  v = umax64(v, dpp64<0x118, 0xF>(v));
  v = umax64(v, dpp64<0x142, 0xA>(v));
  v = umax64(v, dpp64<0x143, 0xC>(v));
  return lane63(v);
}

struct RowHead {
  uint32_t argmax;
  bool greedy;
  double lmax, inv_t;
};

// Row maximum from the chunk maxima (every wave computes it; nch <= 64) and the greedy test.
__device__ inline RowHead row_head(const float* row, const uint64_t* cmax, int nch, const gr_sample_params& pr) {
  const int lane = threadIdx.x & 63;
  const uint64_t m = wave_max_dpp(lane < nch ? cmax[lane] : 0ull);
  RowHead h;
  h.argmax = 0xFFFFFFFFu - (uint32_t)m;
  h.lmax = (double)row[h.argmax];
  h.inv_t = 1.0 / pr.temperature;
  h.greedy = !(pr.temperature > 0.0) || !__builtin_isfinite(h.inv_t) || pr.top_k == 1 || !__builtin_isfinite(h.lmax);
  return h;
}

__device__ inline uint32_t weight_of(float l, const RowHead& h) { return sample_weight(((double)l - h.lmax) * h.inv_t); }

// The four elements i0 .. i0+3 of a row (those at or past vocab read as 0 and are skipped by
// the callers); one 16-byte load when rows are 16-byte aligned.
__device__ inline float4 load4(const float* row, int i0, int vocab) {
  if ((vocab & 3) == 0) return i0 < vocab ? *(const float4*)(row + i0) : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 v;
  v.x = i0 < vocab ? row[i0] : 0.f;
  v.y = i0 + 1 < vocab ? row[i0 + 1] : 0.f;
  v.z = i0 + 2 < vocab ? row[i0 + 2] : 0.f;
  v.w = i0 + 3 < vocab ? row[i0 + 3] : 0.f;
  return v;
}

__device__ inline float elem(const float4& v, int q) { return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w; }

// ---------------------------------------------------------------- kernel 1
__global__ __launch_bounds__(kWideThreads) void sample_max_kernel(const float* __restrict__ logits, int vocab, int nch,
                                                                  SampleWs ws) {
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const float* row = logits + (size_t)b * vocab;
  for (int i = c * kWideThreads + t; i < kBins1; i += nch * kWideThreads) {
    ws.hcnt[(size_t)b * kBins1 + i] = 0u;
    ws.hsum[(size_t)b * kBins1 + i] = 0ull;
  }
  uint64_t m = 0ull;
  float4 v[kChunk / (4 * kWideThreads)];
#pragma unroll
  for (int j = 0; j < kChunk / (4 * kWideThreads); ++j) v[j] = load4(row, c * kChunk + j * 4 * kWideThreads + 4 * t, vocab);
#pragma unroll
  for (int j = 0; j < kChunk / (4 * kWideThreads); ++j) {
    const int i0 = c * kChunk + j * 4 * kWideThreads + 4 * t;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (i0 + q < vocab) {
        const uint64_t x = ((uint64_t)order_key(elem(v[j], q)) << 32) | (0xFFFFFFFFu - (uint32_t)(i0 + q));
        m = x > m ? x : m;
      }
    }
  }
  m = wave_max_dpp(m);
  __shared__ uint64_t s_m[kWideThreads / 64];
  if ((t & 63) == 0) s_m[t >> 6] = m;
  __syncthreads();
  if (t == 0) {
    uint64_t r = s_m[0];
    for (int w = 1; w < kWideThreads / 64; ++w) r = s_m[w] > r ? s_m[w] : r;
    ws.cmax[(size_t)b * nch + c] = r;
  }
}

// ---------------------------------------------------------------- kernel 2
__global__ __launch_bounds__(kHistThreads) void sample_hist_kernel(const float* __restrict__ logits,
                                                                   const gr_sample_params* __restrict__ params,
                                                                   int vocab, int nch, int nseg, SampleWs ws,
                                                                   int32_t* __restrict__ tokens,
                                                                   uint64_t* __restrict__ kept) {
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const float* row = logits + (size_t)b * vocab;
  constexpr int kJ = kHistChunk / (4 * kHistThreads);
  // the chunk's loads go out before the row maximum's
  float4 v[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) v[j] = load4(row, c * kHistChunk + j * 4 * kHistThreads + 4 * t, vocab);
  const gr_sample_params pr = params[b];
  const RowHead h = row_head(row, ws.cmax + (size_t)b * nch, nch, pr);
  if (h.greedy) {
    if (c == 0 && t == 0) {
      tokens[b] = (int32_t)h.argmax;
      if (kept) kept[2 * b] = kept[2 * b + 1] = 0ull;
    }
    return;
  }
  // per bin: count in bits 44..63, weight sum in bits 0..43 (a chunk's weights sum below 2^43)
  __shared__ uint64_t s_bin[kBins1];
  static_assert((uint64_t)kHistChunk << 31 < (1ull << 44), "weight sum fits below the count");
  for (int i = t; i < kBins1; i += kHistThreads) s_bin[i] = 0ull;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int i0 = c * kHistChunk + j * 4 * kHistThreads + 4 * t;
    uint64_t cq[4];  // the lane's composites, 0 for positions past the row
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      cq[q] = 0ull;
      if (i0 + q < vocab) {
        const float l = elem(v[j], q);
        const uint32_t key = order_key(l);
        const uint32_t w = weight_of(l, h);
        atomicAdd((unsigned long long*)&s_bin[key >> 20], (1ull << 44) | (unsigned long long)w);
        cq[q] = composite(key, (uint32_t)(i0 + q));
      }
    }
    // wave wv covers the 256 consecutive elements of one segment: its kSegTop largest
    // composites (each round the lane holding the winner moves to its next), then the largest
    // key of the rest
    auto cx = [](uint64_t& a, uint64_t& b2) {
      const uint64_t hi = a > b2 ? a : b2, lo = a > b2 ? b2 : a;
      a = hi;
      b2 = lo;
    };
    cx(cq[0], cq[1]);
    cx(cq[2], cq[3]);
    cx(cq[0], cq[2]);
    cx(cq[1], cq[3]);
    cx(cq[1], cq[2]);
    int head = 0;
    uint64_t tops[kSegTop];
#pragma unroll
    for (int r = 0; r <= kSegTop; ++r) {
      const uint64_t cur = head == 0 ? cq[0] : head == 1 ? cq[1] : head == 2 ? cq[2] : head == 3 ? cq[3] : 0ull;
      const uint64_t m = wave_max_dpp(cur);
      if (r < kSegTop) {
        tops[r] = m;
        if (m != 0ull && cur == m) ++head;
      } else {
        const int seg = (c * kHistChunk + j * 4 * kHistThreads) / kSeg + wv;
        if (lane == 0 && seg < nseg) {
          ulonglong2* dst = (ulonglong2*)(ws.segtop + ((size_t)b * nseg + seg) * kSegTop);
          dst[0] = make_ulonglong2(tops[0], tops[1]);
          dst[1] = make_ulonglong2(tops[2], tops[3]);
          ws.segsec[(size_t)b * nseg + seg] = (uint32_t)(m >> kIdxBits);
        }
      }
    }
  }
  __syncthreads();
  // add the non-empty bins to the row's histogram; thread t owns bins t + 256 k, so each wave's
  // atomics cover consecutive addresses
  uint32_t* gc = ws.hcnt + (size_t)b * kBins1;
  uint64_t* gs = ws.hsum + (size_t)b * kBins1;
  constexpr int kPer = kBins1 / kHistThreads;
  uint64_t x[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) x[k] = s_bin[t + kHistThreads * k];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int bin = t + kHistThreads * k;
    if (x[k]) atomicAdd(&gc[bin], (uint32_t)(x[k] >> 44));
    if (x[k] & ((1ull << 44) - 1)) atomicAdd((unsigned long long*)&gs[bin], (unsigned long long)(x[k] & ((1ull << 44) - 1)));
  }
}

// ---------------------------------------------------------------- kernel 3
constexpr int kBins2 = 1024;  // LDS levels: 10 composite bits at a time
constexpr int kMembers = 256; // bucket size resolved by ranking the members against each other

struct alignas(16) SelShared {
  uint32_t cc[kBins1];   // level-1 running count from the highest bin down, through this bin
  uint64_t cw[kBins1];   // and running weight
  uint64_t lc[kCap];     // gathered composites
  uint32_t lw[kCap];     // and their weights
  uint32_t h2c[kBins2];  // LDS level histogram (also the members' staging area)
  uint64_t h2s[kBins2];
  uint16_t segs[kMaxSegs];
  uint64_t wave_a[kSelThreads / 64], wave_b[kSelThreads / 64];
  int r_bin;
  uint32_t r_idx, n_list, n_segs, n_mem;
  uint64_t r_cum, r_c_above, r_w_above, r_cnt;
};
static_assert(sizeof(SelShared) <= 160 * 1024, "fits one CU's LDS");

// Block-wide inclusive scan of two quantities in thread order (one barrier pair).
__device__ inline void block_scan2(SelShared& s, uint64_t a, uint64_t b, uint64_t& ia, uint64_t& ib) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  ia = wave_scan_dpp(a);
  ib = wave_scan_dpp(b);
  if (lane == 63) {
    s.wave_a[wv] = ia;
    s.wave_b[wv] = ib;
  }
  __syncthreads();
  uint64_t pa = 0, pb = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const uint64_t xa = s.wave_a[w], xb = s.wave_b[w];
    pa += w < wv ? xa : 0ull;
    pb += w < wv ? xb : 0ull;
  }
  __syncthreads();
  ia += pa;
  ib += pb;
}

__device__ inline uint64_t nucleus_target(double p, uint64_t wk) {
  const double pd = __builtin_ceil(p * (double)wk);
  return !(pd > 1.0) ? 1ull : (pd >= (double)wk ? wk : (uint64_t)pd);
}

__device__ inline uint64_t draw_target(double u, uint64_t wp) {
  const double x = __builtin_floor(u * (double)wp);
  return x >= (double)wp ? wp - 1 : (x > 0.0 ? (uint64_t)x : 0ull);
}

// Inverse of order_key (NaN comes back as a NaN, -0 as +0, which weigh the same).
__device__ inline float key_value(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

// Reserves n_mine list slots for this lane (one LDS atomic per wave) and returns the first.
__device__ inline uint32_t wave_reserve(SelShared& s, uint32_t n_mine) {
  const uint64_t inc = wave_scan_dpp((uint64_t)n_mine);
  const uint32_t total = (uint32_t)lane63(inc);
  uint32_t base = 0;
  if (total != 0u) {
    if ((threadIdx.x & 63) == 0) base = atomicAdd(&s.n_list, total);
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
  }
  return base + (uint32_t)inc - n_mine;
}

// Visits every element of the row: f(i, key, valid) for 32 elements per thread per round
// (uniform control flow: invalid positions are visited with valid == false).
template <class F>
__device__ inline void row_pass(const float* row, int vocab, F&& f) {
  const int t = threadIdx.x;
  constexpr int kU = 8;  // float4 loads per thread and round
  for (int i00 = 0; i00 < vocab; i00 += 4 * kU * kSelThreads) {
    float4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = load4(row, i00 + 4 * (u * kSelThreads + t), vocab);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i0 = i00 + 4 * (u * kSelThreads + t);
#pragma unroll
      for (int q = 0; q < 4; ++q) f(i0 + q, order_key(elem(v[u], q)), i0 + q < vocab);
    }
  }
}

// Weights of the list entries [0, n_list).
__device__ inline void list_weights(SelShared& s, const RowHead& h) {
  const int n = (int)min(s.n_list, (uint32_t)kCap);
  for (int j = threadIdx.x; j < n; j += kSelThreads)
    s.lw[j] = weight_of(key_value((uint32_t)(s.lc[j] >> kIdxBits)), h);
  __syncthreads();
}

// Per-thread copy of the segment summaries (segments t and t + kSelThreads).
static_assert(kMaxSegs <= 2 * kSelThreads, "two segment summaries per select thread");
struct SegSummary {
  uint64_t top[2][kSegTop];
  uint32_t sec[2];
};

// Gathers every element whose level-1 bin is at least b_low.  A segment whose top element is
// the only one reaching the bin contributes it straight from its summary; only segments with
// more candidates are read.
__device__ void gather_top(SelShared& s, const float* row, int vocab, const SegSummary& sum, int nseg, int b_low,
                           const RowHead& h) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  if (t == 0) {
    s.n_list = 0u;
    s.n_segs = 0u;
  }
  __syncthreads();
  // a segment whose key below its recorded top ones misses the bin gives those of its top
  // ones that reach it; the others that reach it are read
  int nd[2] = {0, 0};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int seg = t + k * kSelThreads;
    if (seg < nseg && (int)(sum.top[k][0] >> (kIdxBits + 20)) >= b_low) {
      if ((int)(sum.sec[k] >> 20) < b_low) {
        const int valid = min(kSegTop, vocab - seg * kSeg);
#pragma unroll
        for (int r = 0; r < kSegTop; ++r) nd[k] += (r < valid && (int)(sum.top[k][r] >> (kIdxBits + 20)) >= b_low) ? 1 : 0;
      } else {
        s.segs[atomicAdd(&s.n_segs, 1u)] = (uint16_t)seg;
      }
    }
  }
  uint32_t slot = wave_reserve(s, (uint32_t)(nd[0] + nd[1]));
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int r = 0; r < kSegTop; ++r)
      if (r < nd[k]) {
        if (slot < (uint32_t)kCap) s.lc[slot] = sum.top[k][r];
        ++slot;
      }
  __syncthreads();
  const int nq = (int)s.n_segs;
  constexpr int kWaves = kSelThreads / 64, kInFlight = 8;
  for (int q0 = wv; q0 < nq; q0 += kWaves * kInFlight) {
    float4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int q = q0 + kWaves * u;
      v[u] = q < nq ? load4(row, (int)s.segs[q] * kSeg + 4 * lane, vocab) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    uint32_t mine = 0u;  // bit 4u+e: element e of segment u is taken
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int q = q0 + kWaves * u;
      const int i0 = (q < nq ? (int)s.segs[q] : 0) * kSeg + 4 * lane;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool take = q < nq && i0 + e < vocab && (int)(order_key(elem(v[u], e)) >> 20) >= b_low;
        mine |= take ? 1u << (4 * u + e) : 0u;
      }
    }
    slot = wave_reserve(s, (uint32_t)__popc(mine));
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int q = q0 + kWaves * u;
      const int i0 = (q < nq ? (int)s.segs[q] : 0) * kSeg + 4 * lane;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((mine >> (4 * u + e)) & 1u) {
          if (slot < (uint32_t)kCap) s.lc[slot] = composite(order_key(elem(v[u], e)), (uint32_t)(i0 + e));
          ++slot;
        }
      }
    }
  }
  __syncthreads();
  list_weights(s, h);
}

// Gathers every element whose composite starts with prefix (plen bits) with one row pass.
__device__ void gather_prefix(SelShared& s, const float* row, int vocab, uint64_t prefix, int plen, const RowHead& h) {
  const int t = threadIdx.x;
  if (t == 0) s.n_list = 0u;
  __syncthreads();
  const int sh = kCompBits - plen;
  constexpr int kU = 8;  // float4 loads per thread and round
  for (int i00 = 0; i00 < vocab; i00 += 4 * kU * kSelThreads) {
    float4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = load4(row, i00 + 4 * (u * kSelThreads + t), vocab);
    uint32_t mine = 0u;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i0 = i00 + 4 * (u * kSelThreads + t);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool take = i0 + q < vocab && (composite(order_key(elem(v[u], q)), (uint32_t)(i0 + q)) >> sh) == prefix;
        mine |= take ? 1u << (4 * u + q) : 0u;
      }
    }
    uint32_t slot = wave_reserve(s, (uint32_t)__popc(mine));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i0 = i00 + 4 * (u * kSelThreads + t);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if ((mine >> (4 * u + q)) & 1u) {
          if (slot < (uint32_t)kCap) s.lc[slot] = composite(order_key(elem(v[u], q)), (uint32_t)(i0 + q));
          ++slot;
        }
      }
    }
  }
  __syncthreads();
  list_weights(s, h);
}

// What the LDS list holds: nothing, every element whose level-1 bin is at least min_bin, or
// every element whose composite starts with prefix (plen bits).
struct ListTag {
  int mode;  // 0 empty, 1 min_bin, 2 prefix
  int min_bin, plen;
  uint64_t prefix;
  __device__ bool covers(uint64_t pre, int len) const {
    if (mode == 1) return (int)(pre >> (len - 12)) >= min_bin;
    if (mode == 2) return len >= plen && (pre >> (len - plen)) == prefix;
    return false;
  }
};

struct Selected {
  uint32_t idx;
  uint64_t cum_w;  // running weight through the selected element
};

// Level-1 bin where the running count (count_mode) or weight reaches target.
__device__ inline int find_bin1(SelShared& s, bool count_mode, uint64_t target) {
  const int t = threadIdx.x;
  constexpr int kPer = kBins1 / kSelThreads;
  // thread t owns bins hi-kPer+1 .. hi, hi = kBins1-1-kPer*t; it needs the running values of
  // those bins and of the bin above them
  const int hi = kBins1 - 1 - kPer * t;
  uint64_t run[kPer + 1];
#pragma unroll
  for (int j = 0; j <= kPer; ++j) {
    const int bin = hi + 1 - j;  // j == 0: the bin above (none for thread 0)
    const int bc = bin < kBins1 ? bin : kBins1 - 1;
    const uint64_t v = count_mode ? (uint64_t)s.cc[bc] : s.cw[bc];
    run[j] = bin < kBins1 ? v : 0ull;
  }
  int found = -1;
#pragma unroll
  for (int j = 1; j <= kPer; ++j)
    if (run[j] >= target && run[j - 1] < target) found = hi + 1 - j;
  if (t == 0) s.r_bin = 0;
  __syncthreads();
  if (found >= 0) s.r_bin = found;
  __syncthreads();
  const int r = s.r_bin;
  __syncthreads();
  return r;
}

// Members of one bucket: the list entries whose composite starts with prefix (plen bits; all
// entries when plen == 0), at most kMembers of them, staged in the level histogram's space
// with, for each, the count and weight of the members at or above it in the order.
struct Members {
  uint64_t* c;
  uint32_t* w;
  uint32_t* cge;
  uint64_t* wge;
  int n;
};

__device__ Members rank_members(SelShared& s, uint64_t prefix, int plen) {
  const int t = threadIdx.x;
  Members m;
  m.c = (uint64_t*)s.h2s;
  m.wge = (uint64_t*)s.h2s + kMembers;
  m.w = s.h2c;
  m.cge = s.h2c + kMembers;
  if (t == 0) s.n_mem = 0u;
  __syncthreads();
  const int n = (int)min(s.n_list, (uint32_t)kCap), sh = kCompBits - plen;
  for (int j0 = 0; j0 < n; j0 += kSelThreads) {
    const int j = j0 + t;
    const bool take = j < n && (plen == 0 || (s.lc[j] >> sh) == prefix);
    const uint64_t bm = __ballot(take);
    if (bm != 0ull) {
      const int lane = t & 63, leader = __ffsll((long long)bm) - 1;
      uint32_t base = 0;
      if (lane == leader) base = atomicAdd(&s.n_mem, (uint32_t)__popcll(bm));
      base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
      const uint32_t slot = base + (uint32_t)__popcll(bm & ((1ull << lane) - 1ull));
      if (take && slot < (uint32_t)kMembers) {
        m.c[slot] = s.lc[j];
        m.w[slot] = s.lw[j];
      }
    }
  }
  __syncthreads();
  m.n = (int)min(s.n_mem, (uint32_t)kMembers);
  // pad to a multiple of 16 with composite 0 and weight 0 (never larger than a member)
  const int n16 = (m.n + 15) & ~15;
  if (t >= m.n && t < n16) {
    m.c[t] = 0ull;
    m.w[t] = 0u;
  }
  __syncthreads();
  if (t < m.n) {
    const uint64_t c = m.c[t];
    const uint32_t w_self = m.w[t];
    uint32_t gt = 0;
    uint64_t wgt = 0;
    for (int j0 = 0; j0 < n16; j0 += 16) {
      ulonglong2 c2[8];
      uint4 w4[4];
#pragma unroll
      for (int u = 0; u < 8; ++u) c2[u] = *(const ulonglong2*)&m.c[j0 + 2 * u];
#pragma unroll
      for (int u = 0; u < 4; ++u) w4[u] = *(const uint4*)&m.w[j0 + 4 * u];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint64_t cj = (u & 1) ? c2[u / 2].y : c2[u / 2].x;
        const uint32_t wj = (u & 3) == 0 ? w4[u / 4].x : (u & 3) == 1 ? w4[u / 4].y : (u & 3) == 2 ? w4[u / 4].z : w4[u / 4].w;
        const bool g = cj > c;
        gt += g ? 1u : 0u;
        wgt += g ? (uint64_t)wj : 0ull;
      }
    }
    m.cge[t] = gt + 1u;  // members at or above this one (composites are distinct)
    m.wge[t] = wgt + w_self;
  }
  __syncthreads();
  return m;
}

// The member whose running count (count_mode) or weight, from the bucket's top, reaches t_rem.
__device__ Selected find_member(SelShared& s, const Members& m, bool count_mode, uint64_t t_rem, uint64_t w_above) {
  const int t = threadIdx.x;
  if (t == 0) {
    s.r_idx = 0u;
    s.r_cum = 0ull;
  }
  __syncthreads();
  if (t < m.n) {
    const uint64_t cge = m.cge[t], wge = m.wge[t];
    const uint64_t q = count_mode ? cge : wge, q_prev = count_mode ? cge - 1 : wge - m.w[t];
    if (q >= t_rem && q_prev < t_rem) {
      s.r_idx = kIdxMask - (uint32_t)(m.c[t] & kIdxMask);
      s.r_cum = w_above + wge;
    }
  }
  __syncthreads();
  Selected r;
  r.idx = s.r_idx;
  r.cum_w = s.r_cum;
  __syncthreads();
  return r;
}

// First element of the order whose running count (count_mode) or weight reaches target
// (1 <= target <= the row's total).
__device__ Selected select(SelShared& s, ListTag& tag, const float* row, int vocab, const RowHead& h,
                           bool count_mode, uint64_t target) {
  const int t = threadIdx.x;
  const int b1 = find_bin1(s, count_mode, target);
  const uint64_t c_above = b1 == kBins1 - 1 ? 0ull : s.cc[b1 + 1], w_above0 = b1 == kBins1 - 1 ? 0ull : s.cw[b1 + 1];
  uint64_t prefix = (uint64_t)b1;
  int plen = 12;
  uint64_t t_rem = target - (count_mode ? c_above : w_above0), w_above = w_above0;
  uint64_t cnt = (uint64_t)s.cc[b1] - c_above;
  for (int guard = 0; guard < 24; ++guard) {
    const bool covered = tag.covers(prefix, plen);
    if (covered && cnt <= (uint64_t)kMembers)
      return find_member(s, rank_members(s, prefix, plen), count_mode, t_rem, w_above);
    if (!covered && cnt <= (uint64_t)kCap) {
      gather_prefix(s, row, vocab, prefix, plen, h);
      tag.mode = 2;
      tag.prefix = prefix;
      tag.plen = plen;
      continue;
    }
    // one more histogram level: 10 bits from the list, 8 bits from a row pass
    const int dw = min(covered ? 10 : 8, kCompBits - plen);
    const int sh = kCompBits - plen, shd = sh - dw, nb = 1 << dw;
    const uint64_t dmask = (uint64_t)(nb - 1);
    for (int i = t; i < kBins2; i += kSelThreads) {
      s.h2c[i] = 0u;
      s.h2s[i] = 0ull;
    }
    __syncthreads();
    if (covered) {
      const int n = (int)min(s.n_list, (uint32_t)kCap);
      for (int j = t; j < n; j += kSelThreads) {
        const uint64_t c = s.lc[j];
        if ((c >> sh) == prefix) {
          const int dg = (int)((c >> shd) & dmask);
          atomicAdd(&s.h2c[dg], 1u);
          if (s.lw[j]) atomicAdd((unsigned long long*)&s.h2s[dg], (unsigned long long)s.lw[j]);
        }
      }
    } else {
      row_pass(row, vocab, [&](int i, uint32_t key, bool valid) {
        const uint64_t c = composite(key, (uint32_t)i);
        if (valid && (c >> sh) == prefix) {
          const int dg = (int)((c >> shd) & dmask);
          atomicAdd(&s.h2c[dg], 1u);
          const uint32_t w = weight_of(key_value(key), h);
          if (w) atomicAdd((unsigned long long*)&s.h2s[dg], (unsigned long long)w);
        }
      });
    }
    __syncthreads();
    // scan the level's bins from the highest down; thread t owns bins nb-1-per*t .. nb-per*(t+1)
    const int per = nb > kSelThreads ? nb / kSelThreads : 1;
    const bool active = t * per < nb;
    uint64_t own_c = 0, own_w = 0;
    if (active)
      for (int j = 0; j < per; ++j) {
        own_c += s.h2c[nb - 1 - (t * per + j)];
        own_w += s.h2s[nb - 1 - (t * per + j)];
      }
    uint64_t inc_c, inc_w;
    block_scan2(s, own_c, own_w, inc_c, inc_w);
    if (t == 0) {
      s.r_bin = 0;
      s.r_c_above = s.r_w_above = s.r_cnt = 0;
    }
    __syncthreads();
    uint64_t ex_c = inc_c - own_c, ex_w = inc_w - own_w;
    const uint64_t ex_m = count_mode ? ex_c : ex_w, own_m = count_mode ? own_c : own_w;
    if (active && ex_m < t_rem && t_rem <= ex_m + own_m) {
      for (int j = 0; j < per; ++j) {
        const int bin = nb - 1 - (t * per + j);
        const uint64_t bc = s.h2c[bin], bw = s.h2s[bin];
        if (t_rem <= (count_mode ? ex_c + bc : ex_w + bw)) {
          s.r_bin = bin;
          s.r_c_above = ex_c;  // count and weight above the bin inside the prefix
          s.r_w_above = ex_w;
          s.r_cnt = bc;
          break;
        }
        ex_c += bc;
        ex_w += bw;
      }
    }
    __syncthreads();
    const uint64_t ca = s.r_c_above, wa = s.r_w_above;
    prefix = (prefix << dw) | (uint64_t)s.r_bin;
    plen += dw;
    t_rem -= count_mode ? ca : wa;
    w_above += wa;
    cnt = s.r_cnt;
    __syncthreads();
  }
  Selected r;
  r.idx = 0;
  r.cum_w = 0;
  return r;
}

__global__ __launch_bounds__(kSelThreads) void sample_select_kernel(const float* __restrict__ logits,
                                                                    const gr_sample_params* __restrict__ params,
                                                                    int vocab, int nch, int nseg, SampleWs ws,
                                                                    int32_t* __restrict__ tokens,
                                                                    uint64_t* __restrict__ kept) {
  const int b = blockIdx.x, t = threadIdx.x;
  const float* row = logits + (size_t)b * vocab;
  // the level-1 histogram's loads go out first: thread t owns bins kPer*t' .. kPer*t'+kPer-1
  // with t' = kSelThreads-1-t (thread 0 the highest bins)
  constexpr int kPer = kBins1 / kSelThreads;
  static_assert(kPer == 8, "two 16-byte count loads and four weight loads per thread");
  const int bin0 = kBins1 - kPer * (t + 1);
  const uint4 hc_lo = *(const uint4*)(ws.hcnt + (size_t)b * kBins1 + bin0);
  const uint4 hc_hi = *(const uint4*)(ws.hcnt + (size_t)b * kBins1 + bin0 + 4);
  ulonglong2 hs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) hs[j] = *(const ulonglong2*)(ws.hsum + (size_t)b * kBins1 + bin0 + 2 * j);
  SegSummary sum;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int seg = t + k * kSelThreads;
    const bool in = seg < nseg;
    const ulonglong2* src = (const ulonglong2*)(ws.segtop + ((size_t)b * nseg + (in ? seg : 0)) * kSegTop);
    const ulonglong2 p0 = src[0], p1 = src[1];
    sum.top[k][0] = in ? p0.x : 0ull;
    sum.top[k][1] = in ? p0.y : 0ull;
    sum.top[k][2] = in ? p1.x : 0ull;
    sum.top[k][3] = in ? p1.y : 0ull;
    sum.sec[k] = in ? ws.segsec[(size_t)b * nseg + seg] : 0u;
  }
  const gr_sample_params pr = params[b];
  const RowHead h = row_head(row, ws.cmax + (size_t)b * nch, nch, pr);
  if (h.greedy) return;  // the histogram kernel wrote the token
  __shared__ SelShared s;
  // running count and weight from the top bin down
  const uint32_t c4[kPer] = {hc_lo.x, hc_lo.y, hc_lo.z, hc_lo.w, hc_hi.x, hc_hi.y, hc_hi.z, hc_hi.w};
  const uint64_t w4[kPer] = {hs[0].x, hs[0].y, hs[1].x, hs[1].y, hs[2].x, hs[2].y, hs[3].x, hs[3].y};
  uint64_t own_c = 0, own_w = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    own_c += c4[j];
    own_w += w4[j];
  }
  uint64_t inc_c, inc_w;
  block_scan2(s, own_c, own_w, inc_c, inc_w);
  {
    uint64_t rc = inc_c - own_c, rw = inc_w - own_w;
#pragma unroll
    for (int j = kPer - 1; j >= 0; --j) {  // highest bin first
      rc += c4[j];
      rw += w4[j];
      s.cc[bin0 + j] = (uint32_t)rc;
      s.cw[bin0 + j] = rw;
    }
  }
  __syncthreads();
  const uint64_t total = s.cw[0];
  const bool topk = pr.top_k > 1 && pr.top_k < vocab, topp = pr.top_p < 1.0;
  // the level-1 bin where the first cut that applies lands: every cut lies at or above it
  const int b_low = topk   ? find_bin1(s, true, (uint64_t)pr.top_k)
                    : topp ? find_bin1(s, false, nucleus_target(pr.top_p, total))
                           : find_bin1(s, false, draw_target(pr.u, total) + 1);
  const uint64_t n_top = s.cc[b_low];
  uint64_t wk = total, wp = total;
  uint32_t token = 0;
  ListTag tag;
  tag.mode = 0;
  tag.min_bin = 0;
  tag.plen = 0;
  tag.prefix = 0;
  if (n_top <= (uint64_t)kCap) {
    gather_top(s, row, vocab, sum, nseg, b_low, h);
    tag.mode = 1;
    tag.min_bin = b_low;
  }
  // the three cuts in turn (one code path, so each routine is instantiated once); a prefix
  // of at most kMembers elements is ranked once and every cut is a lookup in it
  Members top;
  top.n = 0;
  const bool ranked = n_top <= (uint64_t)kMembers;
  if (ranked) top = rank_members(s, 0, 0);
  for (int ph = 0; ph < 3; ++ph) {
    if ((ph == 0 && !topk) || (ph == 1 && !topp)) {
      if (ph == 1) wp = wk;
      continue;
    }
    const uint64_t target = ph == 0 ? (uint64_t)pr.top_k : ph == 1 ? nucleus_target(pr.top_p, wk) : draw_target(pr.u, wp) + 1;
    const Selected r = ranked ? find_member(s, top, ph == 0, target, 0) : select(s, tag, row, vocab, h, ph == 0, target);
    if (ph == 0) wk = r.cum_w;
    else if (ph == 1) wp = r.cum_w;
    else token = r.idx;
  }
  if (t == 0) {
    tokens[b] = (int32_t)token;
    if (kept) {
      kept[2 * b] = wk;
      kept[2 * b + 1] = wp;
    }
  }
}


SampleWs carve_sample(void* base, int B, int vocab, size_t* bytes) {
  const int nch = (vocab + kChunk - 1) / kChunk;
  const int nseg = (vocab + kSeg - 1) / kSeg;
  size_t off = 0;
  auto take = [&](size_t n) {
    off = (off + 255) & ~(size_t)255;
    const size_t o = off;
    off += n;
    return base ? (char*)base + o : nullptr;
  };
  SampleWs w;
  w.cmax = (uint64_t*)take((size_t)B * nch * 8);
  w.hcnt = (uint32_t*)take((size_t)B * kBins1 * 4);
  w.hsum = (uint64_t*)take((size_t)B * kBins1 * 8);
  w.segtop = (uint64_t*)take((size_t)B * nseg * kSegTop * 8);
  w.segsec = (uint32_t*)take((size_t)B * nseg * 4);
  if (bytes) *bytes = off;
  return w;
}

}  // namespace

size_t sample_workspace_bytes(int B, int vocab) {
  size_t n = 0;
  carve_sample(nullptr, B, vocab, &n);
  return n;
}

int sample_max_vocab() { return 1 << kIdxBits; }

hipError_t launch_sample(const float* logits, int B, int vocab, const gr_sample_params* params, int32_t* tokens,
                         uint64_t* kept, void* ws, hipStream_t st) {
  const SampleWs w = carve_sample(ws, B, vocab, nullptr);
  const int nch = (vocab + kChunk - 1) / kChunk;
  const int nseg = (vocab + kSeg - 1) / kSeg;
  const dim3 wide(nch, B);
  launch_kernel(sample_max_kernel, wide, dim3(kWideThreads), 0, st, logits, vocab, nch, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_kernel(sample_hist_kernel, dim3((vocab + kHistChunk - 1) / kHistChunk, B), dim3(kHistThreads), 0, st, logits,
                params, vocab, nch, nseg, w, tokens, kept);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_kernel(sample_select_kernel, dim3(B), dim3(kSelThreads), 0, st, logits, params, vocab, nch, nseg, w, tokens,
                kept);
  return hipGetLastError();
}

}  // namespace gr

// ------------------------------------------------------------ speculative acceptance
namespace gr {
namespace {

// Row b accepts its proposals while the target's token after each position equals the
// proposal that follows it.
__global__ void spec_accept_kernel(const int32_t* __restrict__ sampled, const int32_t* __restrict__ draft, int B,
                                   int T, int32_t* __restrict__ n_accepted) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int n = 0;
  while (n < T - 1 && sampled[(size_t)b * T + n] == draft[(size_t)b * T + n + 1]) ++n;
  n_accepted[b] = n;
}

}  // namespace

hipError_t launch_spec_accept(const int32_t* sampled, const int32_t* draft, int B, int T, int32_t* n_accepted,
                              hipStream_t st) {
  launch_kernel(spec_accept_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, st, sampled, draft, B, T,
                n_accepted);
  return hipGetLastError();
}

}  // namespace gr
