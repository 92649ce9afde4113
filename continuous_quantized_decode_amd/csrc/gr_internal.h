// gr_internal.h -- internal declarations shared by the translation units of libgr.
#pragma once

#include <hip/hip_ext.h>

#include "gr_common.h"
#include "../../include/gr.h"

namespace gr {

// ------------------------------------------------------------------ launches
//
// Every kernel of the library is launched through launch_kernel.  While a timing
// probe is armed on this thread (probe_events non-null), the launch attaches the
// probe's events to the dispatch itself (hipExtLaunchKernelGGL): the start event of
// the first launch and the stop event of every launch, so the events span exactly
// the kernels' execution, with no marker or dispatch latency in between.
struct ProbeEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool first = true;
};
extern thread_local ProbeEvents* probe_events;

template <class K, class... A>
inline void launch_kernel(K kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t st, A... args) {
  if (ProbeEvents* pe = probe_events) {
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)shmem, st, pe->first ? pe->start : nullptr, pe->stop, 0,
                          args...);
    pe->first = false;
  } else {
    kernel<<<grid, block, shmem, st>>>(args...);
  }
}

// The same for a kernel chosen at run time (host pointer of a __global__ function and
// its packed argument pointers).
inline hipError_t launch_fn(const void* fn, dim3 grid, dim3 block, size_t shmem, hipStream_t st, void** args) {
  if (ProbeEvents* pe = probe_events) {
    const hipError_t e = hipExtLaunchKernel(fn, grid, block, args, shmem, st, pe->first ? pe->start : nullptr, pe->stop, 0);
    pe->first = false;
    return e;
  }
  return hipLaunchKernel(fn, grid, block, args, shmem, st);
}

// ------------------------------------------------------------------------ GEMM
//
// One workgroup per output tile: 16 weight rows (or, for the SwiGLU GEMM, 16 gate
// rows and the 16 up rows of the same FFN columns), all B activation rows, the whole
// K range.  The workgroup's waves split K into contiguous super-block ranges, each
// stream their weights once, and reduce through LDS before the epilogue.

enum GemmEpi {
  kEpiStore = 0,     // y[b][col] = r_b * acc
  kEpiResidual = 1,  // x[b][col] += r_b * acc; then pack x * gain, accumulate sum x^2
  kEpiSwiGLU = 2,    // a = silu(r_b * gate) * (r_b * up); pack a
};

struct GemmArgs {
  const uint8_t* w[3];
  int seg_rows[3];
  int seg_tile_off[4];  // first workgroup of each matrix; [nseg] = total workgroups
  int seg_col_off[3];   // first output column of each matrix
  int nseg;
  int nsb;              // super-blocks per row (K/256)
  size_t row_bytes;
  const void* xpack;    // actpack of the input, kind by weight type
  int nslices;
  const double* ss;     // per-row sum of squares of the input (RMSNorm) in ss_slots
                        // partial slots [slot][B], or NULL: r = 1
  int ss_slots;
  float inv_k, eps;
  int B;
  int sb_per_wave;
  int tl_groups, tl_groups_per_wg;  // tile-loop kernel: tile groups in all, per workgroup
  int mm_mtiles, mm_groups;         // many-row kernel: activation tile groups, weight tile groups
  int epi;
  float* y;             // store: output; residual: the residual stream x
  int ldy;
  const float* gain;    // residual: next norm gain (per column); NULL = 1
  u16* pack_out;        // residual / swiglu: actpack written by the epilogue (NULL: none)
  int pack_kind, pack_nslices;
  u16* pack_out2;       // residual: a second actpack kind of the same values (NULL: none)
  int pack_kind2, pack_nslices2;
  double* ss_out;       // residual: sum of squares accumulator of the packed rows, [ss_slots][B]
  double* zero_ptr;     // optional: workgroup 0 zeroes zero_n values (a sum-of-squares buffer)
  int zero_n;
  // many-row kernel split over K (store and residual epilogues): the K ranges' partial
  // sums part[split][B][ldp] (launch-local columns, the launch's first output column
  // pcol0), summed and finished by a second kernel; part NULL: no split
  float* part;
  size_t part_cap;      // floats available at part
  int ldp, pcol0;
  // row-block kernel (17 to 32 rows) over several K ranges: the ranges' partial sums at
  // part, and one arrival counter per gate/up pair (zero between launches), rb_cnt_n of them
  uint32_t* rb_cnt;
  int rb_cnt_n;
};

// The RMSNorm statistic (per-row sum of squares) that a GEMM epilogue applies is kept
// as ss_slots(B) partial sums [slot][B] (at most kSsCap values).  A producer running in
// many workgroups adds into slot (workgroup % slots), so that only a few atomics meet
// on one address (hundreds of same-address atomics from all XCDs serialize at the
// memory side and hold the kernel's completion for microseconds); consumers add the
// slots up in slot order.  The sums are fp64: each addend is a float (a tile's 16
// squares summed in fp32), so the adds into a slot are exact, and the result does not
// depend on the atomics' order, unless one row's addends span more than 2^29.
constexpr int kSsCap = 256;
__host__ __device__ inline int ss_slots(int B) { return B <= 16 ? 16 : B <= kSsCap ? kSsCap / B : 1; }
// values (doubles) of one RMSNorm partial-sum buffer
inline size_t ss_count(int B) { return (size_t)ss_slots(B) * B > (size_t)kSsCap ? (size_t)ss_slots(B) * B : kSsCap; }

struct GemmPlan {
  int nt, btn, waves, sb_per_wave, tiles, maxt;
  size_t lds;
};

// total_tiles: workgroups (tile groups of nt tiles, or gate/up pairs with nt = 2).
GemmPlan plan_gemm(int wtype, int total_tiles, int K, int B, int nt);

// Tiles per workgroup of a plain (non-SwiGLU) GEMM launch: consecutive 16-row tiles of
// one matrix share each activation fragment when there are enough tiles to fill the
// chip in pairs.
inline int gemm_group(int tiles) { return tiles >= 1024 ? 2 : 1; }

// LDS per GEMM workgroup (gfx950: 160 KB per workgroup).
constexpr int kGemmLds = 160 * 1024;

// The tile-loop GEMM (workgroups walk runs of tile groups, activations held in
// registers): used when the batch is one activation tile, K is at most 16 super-blocks
// (two per wave) and there are at least two tile groups per CU.
bool use_tile_loop(int wtype, int groups, int K, int B);
struct TlPlan {
  int waves, grid, groups_per_wg, ring;
  size_t lds;
  bool whole;  // whole-tile staging (gemm_tlw_kernel: the Q4_K gate/up pairs)
};
TlPlan plan_gemm_tl(int wtype, int nt, int groups, int K, int B);
bool use_tile_loop_whole(int wtype, int groups, int K, int B);  // gemm_tlw_kernel's sizes
bool use_kcw(int wtype, int K, int B, int nmat);  // gemm_kcw_kernel's sizes (one matrix)
int kcw_waves(int nsb);
hipError_t launch_gemm_kcw(int tiles, GemmArgs a, hipStream_t st);
inline int tl_btn(int B) { return B <= 8 ? 1 : 2; }  // activation tiles of the tile loop
// The row-block GEMM (gemm_rb_kernel): the Q4_K gate/up pairs at 17 to 32 rows, K in
// ranges of 4 to 8 super-blocks (rb_ranges of them, 0: not this kernel).  rb_fits:
// whether the partial-sum floats and counters given suffice for `groups` pairs.
bool use_rb(int wtype, int K, int B);
int rb_ranges(int nsb);
size_t rb_part_floats(int groups, int K, bool pair);
bool rb_fits(int groups, int K, bool pair, size_t part_cap, int cnt_n);
int rb_grid(int nsb);  // workgroups of a launch
hipError_t launch_gemm_rb(int groups, GemmArgs a, hipStream_t st);
hipError_t launch_gemm_tl(int wtype, int nt, const TlPlan& pl, GemmArgs a, hipStream_t st);
hipError_t launch_gemm(int wtype, const GemmPlan& pl, const GemmArgs& a, hipStream_t st);

// Rows above kSkinnyRows take the many-row kernel (Q4_K and Q6_K weights; kMaxRows at
// most): a 2-D output tile per workgroup, ngroups groups of mm_group_tiles weight tiles
// (per matrix segment; SwiGLU: gate/up tile pairs), a.seg_tile_off counted in groups.
constexpr int kSkinnyRows = 64;
constexpr int kMaxRows = 512;
constexpr int kMmMinRows = 32;  // above this many rows Q4_K / Q6_K take the many-row kernel (measured: 32 rows skinny, 64 rows many-row)
constexpr int kMmMaxSplit = 4;        // K ranges of a many-row launch with few workgroups
constexpr int kMmSplitMaxCols = 8192;  // only launches this narrow are split
bool mm_required(int B);              // rows only the many-row kernel takes
bool use_mm(int wtype, int B);       // the kernel a GEMM of this type and rows takes
bool use_mm_store(int wtype, int B, int cols);  // the same for a plain store of `cols` outputs
bool mm_supported(int wtype);
int mm_group_tiles(bool swiglu);
hipError_t launch_gemm_mm(int wtype, int groups, GemmArgs a, hipStream_t st);
// K ranges of a many-row launch of `groups` weight tile groups and `cols` output columns
// (1: no split), given part_cap floats of partial-sum space
int mm_split(int wtype, int B, int cols, int nsb, int groups, int epi, size_t part_cap);

// ---------------------------------------------------------------------- actpack

// (above 64 rows, a multiple of 4 tiles: the many-row GEMM's activation tile groups)
__host__ __device__ inline int actpack_tiles(int B) {
  return B <= 8 ? 1 : B <= 16 ? 2 : B <= 32 ? 4 : B <= 64 ? 8 : ((B + 31) / 32) * 4;
}

// Bytes of an actpack for B rows of K values (16 MFMA rows of bf16 per batch tile).
inline size_t actpack_bytes(int B, int K) { return (size_t)actpack_tiles(B) * K * 16 * 2; }

// Store activation v of (row b, column k) into an actpack as bf16 hi / lo.
GR_DEV void actpack_put(u16* pack, int kind, int nslices, int b, int k, float v) {
  u16 hi, lo;
  split_bf16(v, hi, lo);
  const int t = b >> 3, m = 2 * (b & 7);
  size_t ih;
  if (kind == kK32) {
    const int s = k >> 5, w = k & 31, g = w >> 3, i = perm8(w & 7);
    ih = (((size_t)t * nslices + s) * 64 + g * 16 + m) * 8 + i;
    pack[ih] = hi;
    pack[ih + 8] = lo;
  } else {
    const int s = k >> 4, w = k & 15, g = w >> 2, i = perm4(w & 3);
    ih = (((size_t)t * (nslices >> 1) + (s >> 1)) * 64 + g * 16 + m) * 8 + (s & 1) * 4 + i;
    pack[ih] = hi;
    pack[ih + 8] = lo;
  }
}

struct PackOut {
  u16* pack;
  int kind;  // kK32 / kK16; pack == nullptr: unused
};

// x [B][K] -> actpack(s) of x * gain (gain NULL: 1); with ss_out, also the per-row sum
// of squares of x (RMSNorm of the consumer).  Zeroes the padding rows of the packs.
// RoPE of the step's new tokens (position ctx[b]): for pair i < half_d the angle
// ctx[b] * theta^(-2i / (2 half_d)), its cosine and sine in fp64 at out[(b * half_d +
// i) * 2 + {0, 1}], computed once per step for every layer's attention.
struct RopeTable {
  const int32_t* ctx = nullptr;  // per sequence; row b sits at ctx[b / T] + b % T
  double theta = 0.0;
  int half_d = 0;
  int tokens_per_seq = 1;  // T
  const int32_t* row_pos = nullptr;  // when set, row b sits at row_pos[b]
  double* out = nullptr;  // NULL: none
};
// Optional row selection of a pack: packed row b is x row idx[b] (clamped to
// [0, src_rows)).
struct RowSel {
  const int32_t* idx = nullptr;
  int src_rows = 0;
};
// The decode attention's work list of a step (one token per row), built once per step
// by its first kernel (one block) and read by every layer's attention.  Pages per
// workgroup P: a multiple of group_pages, at most max_groups groups, chosen so that the
// step's workgroups (each row's ceil(pages / P) ranges times the KV heads) about fill
// `slots` resident workgroups.  Row b's ranges j < ceil(ceil((ctx[b] + self) / 16) / P)
// are listed by the number of page groups they hold, most first (rows, then j, in order
// within a count), so that when the list needs more than one round of resident
// workgroups the ones that start late are the short last ranges of rows.  The order is
// only a schedule: a range's result and the merge order depend on (b, j) alone.  The
// list: [0] its entries, [1] P, then the entries {(b << 16) | j, ctx[b]}; and the
// attention's arrival counters cleared.
constexpr int kSchedMaxGroups = 16;  // groups of pages per range at most
struct AttnSched {
  const int32_t* ctx = nullptr;
  int B = 0, self = 1;
  int n_kv_heads = 1, slots = 512, group_pages = 16, max_groups = kSchedMaxGroups;
  uint32_t* list = nullptr;  // entry i at list[2 + 2 i], list[3 + 2 i]
  uint32_t* cnt = nullptr;   // arrival counters to clear
  int n_cnt = 0;
};
// Words of a list for B rows of up to wg_max ranges each.
inline size_t attn_sched_words(int B, int wg_max) { return 2 + 2 * (size_t)B * wg_max; }
// LDS words the builder needs for workgroups of up to 1024 threads.
constexpr int kSchedScratchWords = (2 + 1024 / 64) * (kSchedMaxGroups + 1);
GR_DEV uint32_t block_sum_u32(uint32_t v, uint32_t* lds_scratch) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) lds_scratch[wave] = v;
  __syncthreads();
  uint32_t t = 0;
  for (int w = 0; w < (int)blockDim.x / 64; ++w) t += lds_scratch[w];
  __syncthreads();
  return t;
}
// The list and the counters by one workgroup of blockDim.x <= 1024 threads (a multiple
// of 64); lds_scratch: kSchedScratchWords words.
GR_DEV void build_attn_sched(const AttnSched& s, uint32_t* lds_scratch) {
  constexpr int NB = kSchedMaxGroups + 1;  // bucket k (1 .. G) holds the ranges of k groups
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wave = tid >> 6, nw = nthr / 64;
  // the thread's first row's context, loaded once (rows past the first nthr are read
  // again in each pass)
  const int ctx_own = tid < s.B ? s.ctx[tid] : 0;
  auto ctx_of = [&](int b) { return b == tid ? ctx_own : s.ctx[b]; };
  for (int i = tid; i < s.n_cnt; i += nthr) s.cnt[i] = 0u;
  // pages per workgroup from the step's total
  uint32_t mine = 0;
  for (int b = tid; b < s.B; b += nthr) mine += (uint32_t)((ctx_of(b) + s.self + 15) / 16);
  const uint64_t total = (uint64_t)block_sum_u32(mine, lds_scratch) * (uint64_t)s.n_kv_heads;
  const uint64_t gp = (uint64_t)s.group_pages;
  const int maxg = s.max_groups < 1 ? 1 : s.max_groups > kSchedMaxGroups ? kSchedMaxGroups : s.max_groups;
  uint64_t want = (total + (uint64_t)s.slots - 1) / (uint64_t)s.slots;
  want = (want + gp - 1) / gp * gp;
  const uint32_t wpp = (uint32_t)(want < gp ? gp : want > gp * (uint64_t)maxg ? gp * maxg : want);
  const uint32_t G = wpp / (uint32_t)gp;  // groups of a whole range
  // row b: n ranges, the last of kl groups (n = 0 for an empty row past B)
  auto row_ranges = [&](int b, uint32_t& n, uint32_t& kl) {
    const uint32_t pages = b < s.B ? (uint32_t)((ctx_of(b) + s.self + 15) / 16) : 0u;
    n = (pages + wpp - 1) / wpp;
    kl = n ? (pages - (n - 1) * wpp + (uint32_t)gp - 1) / (uint32_t)gp : 0u;
  };
  uint32_t* first = lds_scratch;     // [NB]: the next free entry of each bucket
  uint32_t* wcnt = lds_scratch + NB;  // [nw + 1][NB]: per wave, then the chunk's totals
  // bucket sizes, then their first entries (bucket G first)
  if (tid < NB) first[tid] = 0u;
  __syncthreads();
  for (int b = tid; b < s.B; b += nthr) {
    uint32_t n, kl;
    row_ranges(b, n, kl);
    if (n) {
      if (n > 1) atomicAdd(&first[G], n - 1);
      atomicAdd(&first[kl], 1u);
    }
  }
  __syncthreads();
  uint32_t n_entries = 0;
  if (tid == 0) {
    for (int k = (int)G; k >= 1; --k) {
      const uint32_t c = first[k];
      first[k] = n_entries;
      n_entries += c;
    }
  }
  __syncthreads();
  for (int b0 = 0; b0 < s.B; b0 += nthr) {
    const int b = b0 + tid;
    uint32_t n, kl;
    row_ranges(b, n, kl);
    const int c = b < s.B ? ctx_of(b) : 0;
    // bucket G: this row's whole ranges (and its last when that is whole), by an
    // inclusive scan over the workgroup; the other buckets: one entry, ranked by ballots
    const uint32_t nG = n ? n - 1 + (kl == G ? 1u : 0u) : 0u;
    uint32_t v = nG;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t u = __shfl_up(v, o, 64);
      if (lane >= o) v += u;
    }
    if (lane == 63) wcnt[wave * NB] = v;
    uint32_t rank = 0;
    for (int k = 1; k < (int)G; ++k) {
      const unsigned long long m = __ballot(n != 0 && kl == (uint32_t)k);
      if (lane == 0) wcnt[wave * NB + k] = (uint32_t)__popcll(m);
      if (n != 0 && kl == (uint32_t)k) rank = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    }
    __syncthreads();
    if (tid < NB) {  // exclusive prefix over the waves per bucket (slot 0: bucket G)
      uint32_t acc = 0;
      for (int w = 0; w < nw; ++w) {
        const uint32_t t = wcnt[w * NB + tid];
        wcnt[w * NB + tid] = acc;
        acc += t;
      }
      wcnt[nw * NB + tid] = acc;
    }
    __syncthreads();
    if (n) {
      const uint32_t fg = first[G] + wcnt[wave * NB] + v - nG;
      for (uint32_t r = 0; r + 1 < n; ++r) {
        s.list[2 + 2 * (fg + r)] = ((uint32_t)b << 16) | r;
        s.list[3 + 2 * (fg + r)] = (uint32_t)c;
      }
      const uint32_t at = kl == G ? fg + n - 1 : first[kl] + wcnt[wave * NB + kl] + rank;
      s.list[2 + 2 * at] = ((uint32_t)b << 16) | (n - 1);
      s.list[3 + 2 * at] = (uint32_t)c;
    }
    __syncthreads();
    if (tid == 0) {
      first[G] += wcnt[nw * NB];
      for (int k = 1; k < (int)G; ++k) first[k] += wcnt[nw * NB + k];
    }
    __syncthreads();
  }
  if (tid == 0) {
    s.list[0] = n_entries;
    s.list[1] = wpp;
  }
}
hipError_t launch_pack_rows(const float* x, int ldx, int B, int K, const float* gain, PackOut o1, PackOut o2,
                            double* ss_out, hipStream_t st,  // ss_out: [ss_slots(B)][B], slot 0 the sum
                            RopeTable rope = RopeTable{}, RowSel sel = RowSel{}, AttnSched sched = AttnSched{});

}  // namespace gr
