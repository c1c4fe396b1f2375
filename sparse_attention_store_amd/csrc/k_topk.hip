// k_topk.hip -- per-row top-k (k <= 2048) over the indexer logits.
//
// The k largest logits among positions s <= pos[r] ("vLLM 推理链路概览: 以 GLM-5.2 为例",
// section DSA Indexer: TopK over positions j).  When pos[r] + 1 <= k every visible
// position is selected and the row is [0 .. pos[r], -1 ...] without reading logits
// ("GLM-5.3 推理全链路(十一)", section on skipping the score for short contexts).
//
// Exact radix select on the order-preserving 32-bit image ("key") of each fp32 logit,
// with a first digit fitted to the row's own key range so that the bin holding the k-th
// largest value is narrow whatever the logits' scale:
//  1. k_range:  grid (chunk, row): min / max key of the row (atomicMin / atomicMax).
//               The fused indexer+top-k entry gets the range from the logits kernel instead.
//  2. k_hist:   grid (chunk, row): LDS histogram of d = (key - kmin) >> shift, 4096 bins,
//               shift chosen from the range; merged into a per-row global histogram.
//  3. k_select: grid (chunk, row): each work-group finds the threshold bin T (the bin
//               holding the k-th largest key) from the row's merged histogram, then keys with
//               d > T are selected and keys with d == T become candidates.  Appends are
//               gathered per work-group in LDS and reserved with one global atomic per list.
//  4. k_final:  one work-group per row resolves the low `shift` bits over the candidates in
//               LDS (by ranking them against each other when few, else 10-bit rounds), keeps
//               the lowest positions among exact ties at the threshold, and writes the k
//               positions in ascending order (a counting sort on their high bits).  If more
//               candidates than fit in LDS share the threshold bin (massive exact ties), the
//               rounds and the tie walk run over the row in global memory instead.
#include "dsa_device.hpp"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kBins = 4096;          // first digit: 12 bits over the row's key range
constexpr int kCap = 4096;           // candidates kept per row
constexpr int kChunk = 8192;         // logits per work-group in passes 1-3
constexpr int kFinalThreads = 1024;
// Two 1024-thread work-groups per CU need 8 waves per SIMD: at most 64 vector registers per
// wave (the second argument of __launch_bounds__ is a minimum of waves per SIMD, not of
// work-groups per CU), and, measured on the device, at most about 60 scalar registers (a
// kernel of 76 runs one work-group per CU, whatever its LDS and vector registers).
#define DSA_TWO_GROUPS_PER_CU __launch_bounds__(kFinalThreads, 8) __attribute__((amdgpu_num_sgpr(56)))
constexpr int kBufferWord3 = 0x00020000;   // buffer descriptor word 3: 32-bit raw reads
// sampled keys a threshold work-group holds in registers: 8 per thread in the kernel two
// work-groups of which share a CU, 32 per thread (a row of up to 512K positions) in the one for
// launches with longer rows
constexpr int kThrPer = 8, kThrPerLong = 32;
static_assert(kCap % kFinalThreads == 0, "whole loads per thread");
// fused path: the filter keeps about kMarginNum / kMarginDen times k candidates per row
constexpr int kMarginNum = 3, kMarginDen = 2;

struct Ws {
  uint32_t* range;  // [R][2]: min key, max key
  int* hist;        // [R][kBins]
  int* cnt;         // [R][4]: 0 = selected-above count, 1 = candidate count, 2 = threshold bin T,
                    //         3 = filtered candidate count (fused path)
  int* above;       // [R][k]
  uint32_t* ckey;   // [R][kCap]   radix candidates, or the fused path's filtered candidates
  int* cpos;        // [R][kCap]
  uint32_t* thr;    // [R]  fused path: key threshold of the filter
  int* fcnt;        // [R]  fused path: filtered candidates of the row (may exceed kCap)
  int* flag;        // [R]  fused path: the row needs the exact fallback
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline size_t ws_bytes(int32_t R, int32_t k) {
  return align256((size_t)R * 8) + align256((size_t)R * kBins * 4) + align256((size_t)R * 16) +
         align256((size_t)R * k * 4) + 2 * align256((size_t)R * kCap * 4) + 3 * align256((size_t)R * 4);
}

__host__ __device__ inline Ws carve(void* base, int32_t R, int32_t k) {
  uint8_t* p = (uint8_t*)base;
  Ws w;
  w.range = (uint32_t*)p;  p += align256((size_t)R * 8);
  w.hist = (int*)p;        p += align256((size_t)R * kBins * 4);
  w.cnt = (int*)p;         p += align256((size_t)R * 16);
  w.above = (int*)p;       p += align256((size_t)R * k * 4);
  w.ckey = (uint32_t*)p;   p += align256((size_t)R * kCap * 4);
  w.cpos = (int*)p;        p += align256((size_t)R * kCap * 4);
  w.thr = (uint32_t*)p;    p += align256((size_t)R * 4);
  w.fcnt = (int*)p;        p += align256((size_t)R * 4);
  w.flag = (int*)p;
  return w;
}

__device__ inline uint32_t ord_key(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// shift so that (kmax - kmin) >> shift < kBins
__device__ inline int range_shift(uint32_t kmin, uint32_t kmax) {
  const uint32_t span = kmax - kmin;
  const int bits = span ? 32 - __clz(span) : 0;
  return bits > 12 ? bits - 12 : 0;
}

__device__ inline int64_t row_len(const int32_t* pos, int r, int64_t stride) {
  return min((int64_t)pos[r] + 1, stride);
}

// Workspace initialisation: ranges to (max, 0), counters to 0, every row's exact-path flag to
// `flag` (1: the rows go straight to the radix passes), and, with zero_hist, the histograms to
// 0 (the fused call's filtered path leaves them: it clears the histogram of each row it flags).
__global__ void k_init(Ws w, int32_t R, int flag, int zero_hist) {
  const int64_t n = zero_hist ? (int64_t)R * kBins : (int64_t)R * 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    if (zero_hist) w.hist[i] = 0;
    if (i < (int64_t)R * 4) w.cnt[i] = 0;
    if (i < R) { w.range[2 * i] = 0xFFFFFFFFu; w.range[2 * i + 1] = 0u; w.flag[i] = flag; w.fcnt[i] = 0; }
  }
}

__device__ inline void block_minmax256(uint32_t& mn, uint32_t& mx, uint32_t* sh) {
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) { sh[2 * wave] = mn; sh[2 * wave + 1] = mx; }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int i = 1; i < 4; i++) { mn = min(mn, sh[2 * i]); mx = max(mx, sh[2 * i + 1]); }
}

// `gate` (nullable): only rows with gate[r] != 0 are processed (the fused path's fallback).
__global__ void __launch_bounds__(256) k_range(const float* __restrict__ logits, int64_t stride,
                                               const int32_t* __restrict__ pos, int32_t k, Ws ws,
                                               const int* __restrict__ gate) {
  __shared__ uint32_t sh[8];
  const int r = blockIdx.y;
  if (gate != nullptr && !gate[r]) return;
  const int64_t n = row_len(pos, r, stride);
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (n <= k || c0 >= n) return;
  const int64_t c1 = min(c0 + kChunk, n);
  const float* row = logits + (int64_t)r * stride;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int64_t i = c0 + 4 * threadIdx.x; i < c1; i += 4 * 256) {
    const float4 v = *reinterpret_cast<const float4*>(row + i);   // c0, stride multiples of 4
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; j++)
      if (i + j < c1) { const uint32_t key = ord_key(e[j]); mn = min(mn, key); mx = max(mx, key); }
  }
  block_minmax256(mn, mx, sh);
  if (threadIdx.x == 0) {
    atomicMin(&ws.range[2 * r], mn);
    atomicMax(&ws.range[2 * r + 1], mx);
  }
}

// Passes 2 and 3 run 1024 threads per work-group, two float4 of the chunk each: with 256
// threads (eight each) one wave per SIMD walked the chunk alone and its dependent VALU chain set
// the pass time (a 1M-score row: select 26.6K cycles per work-group, 9K of them in the loop).
constexpr int kPassThreads = 1024;
constexpr int kPerThread = kChunk / kPassThreads / 4;   // float4 loads per thread per chunk (2)

// Loads this thread's share of a chunk (all loads issued before any use).
__device__ inline void load_chunk(const float* row, int64_t c0, int64_t c1, float4 (&v)[kPerThread]) {
#pragma unroll
  for (int u = 0; u < kPerThread; u++) {
    const int64_t i = c0 + 4 * (threadIdx.x + kPassThreads * u);
    v[u] = i < c1 ? *reinterpret_cast<const float4*>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Passes 2 and 3 take chunks blockIdx.x, blockIdx.x + gridDim.x, ... of their row: one chunk
// per work-group for the plain top-k, a few work-groups per row for the fused call's fallback,
// whose grid is mostly rows that are not flagged and exit at once.
__global__ void __launch_bounds__(kPassThreads) k_hist(const float* __restrict__ logits, int64_t stride,
                                              const int32_t* __restrict__ pos, int32_t k, Ws ws,
                                              const int* __restrict__ gate) {
  __shared__ int h[kBins];
  const int r = blockIdx.y;
  if (gate != nullptr && !gate[r]) return;
  const int64_t n = row_len(pos, r, stride);
  if (n <= k) return;
  const uint32_t kmin = ws.range[2 * r], kmax = ws.range[2 * r + 1];
  const int shift = range_shift(kmin, kmax);
  int* gh = ws.hist + (int64_t)r * kBins;
  for (int64_t c0 = (int64_t)blockIdx.x * kChunk; c0 < n; c0 += (int64_t)gridDim.x * kChunk) {
    const int64_t c1 = min(c0 + kChunk, n);
    float4 v[kPerThread];
    load_chunk(logits + (int64_t)r * stride, c0, c1, v);
    for (int i = threadIdx.x; i < kBins; i += kPassThreads) h[i] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPerThread; u++) {
      const int64_t i = c0 + 4 * (threadIdx.x + kPassThreads * u);
      const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (i + j < c1) {
          // keys outside [kmin, kmax] cannot occur when the range covers the row; clamp anyway
          const uint32_t key = min(max(ord_key(e[j]), kmin), kmax);
          atomicAdd(&h[(key - kmin) >> shift], 1);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kBins; i += kPassThreads)
      if (h[i]) atomicAdd(&gh[i], h[i]);
    __syncthreads();                  // h is cleared again for the next chunk
  }
}

// Inclusive prefix sum of v over the NT threads of the work-group in thread order (a wave
// scan by lane shuffles, then the wave totals); *total receives the sum over all threads.
// wsum holds NT / 64 ints of LDS.  Every thread calls it; it synchronises the work-group.
template <int NT>
__device__ inline int block_prefix(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; i++) {
    const int x = wsum[i];
    before += i < w ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// Threshold bin of an LDS histogram: the bin b with count(bins > b) < k <= count(bins >= b).
// result[0] = b, result[1] = count(bins > b).  blockDim.x == NT, NB % NT == 0.  Thread t
// holds the t-th block of bins from the top, so a prefix over threads is a suffix over bins.
template <int NT, int NB>
__device__ inline int find_threshold(const int* h, int k, int* scan, int* result) {
  constexpr int per = NB / NT;
  const int b = NT - 1 - (int)threadIdx.x;
  int local = 0;
  for (int i = 0; i < per; i++) local += h[b * per + i];
  int all;
  int running = block_prefix<NT>(local, scan, &all) - local;   // keys in the bins above this block
  for (int i = per - 1; i >= 0; i--) {
    const int c = h[b * per + i];
    if (running < k && running + c >= k) { result[0] = b * per + i; result[1] = running; }
    running += c;
  }
  __syncthreads();
  return result[0];
}

// Rank finish of a radix select: the bin that holds the need-th largest has in_bin <= kRankMax
// keys left (those whose (key - base) >> low equals prefix).  They are gathered into h and each
// is counted against the others: the key x with count(> x) < need <= count(>= x) is the
// need-th largest, and need - count(> x) of its exact ties belong to the selection.  This
// replaces the remaining radix rounds (a histogram clear, fill and scan each).  Returns x - base
// and sets need_eq (and *n_eq, when given, to the number of in-bin keys equal to x); all NT
// threads call it; res and scan (at least 3 ints) are scratch (res[0] counts the gather).
constexpr int kRankMax = 256;
template <int NT, int kPer>
__device__ inline uint32_t rank_finish(const uint32_t (&v)[kPer], int nv, int low, uint32_t prefix, int in_bin,
                                       int need, int* h, int* scan, int* res, int& need_eq, int* n_eq = nullptr) {
  const int tid = threadIdx.x;
  if (tid == 0) res[0] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; j++)
    if (j < nv && (v[j] >> low) == prefix) h[atomicAdd(&res[0], 1)] = (int)v[j];
  __syncthreads();
  if (tid < in_bin) {
    const uint32_t x = (uint32_t)h[tid];
    int gt = 0, eq = 0;
    for (int i = 0; i < in_bin; i++) {
      const uint32_t y = (uint32_t)h[i];
      gt += y > x;
      eq += y == x;
    }
    if (gt < need && need <= gt + eq) { scan[0] = (int)x; scan[1] = need - gt; scan[2] = eq; }   // one value, maybe several writers
  }
  __syncthreads();
  const uint32_t x = (uint32_t)scan[0];
  need_eq = scan[1];
  if (n_eq != nullptr) *n_eq = scan[2];
  __syncthreads();                     // h, scan and res are free again
  return x;
}

// ----------------------------------------------------------------------------- fused path
// Per row: the filter threshold from the sampled scores (pages 0, S, 2S, ... of the row,
// positions <= pos).  With n_s sampled positions of the row's n, m = ceil(margin * k * n_s / n)
// samples should pass; the threshold is the m-th largest sample itself when the histogram bin
// holding it has few samples left to rank, else the lower edge of that bin after two rounds, so
// at least m samples, and about margin * k of the row's scores, lie at or above it.  Short rows (n <= k) get a threshold nothing reaches; rows with too
// few samples get 0 (every score passes).
template <int kPer>
__device__ inline void filt_thresh(const float* __restrict__ logits, int64_t stride, const int32_t* __restrict__ pos,
                                   int32_t k, Ws ws) {
  constexpr int step = kTopkSampleStep;
  constexpr int kThrSamples = kPer * kFinalThreads;
  __shared__ int h[kBins];
  __shared__ int scan[kFinalThreads / 64];
  __shared__ int res[2];
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* row = logits + (int64_t)r * stride;
  // The held samples are requested first, together with the row's position and range, so the
  // kernel waits one memory round trip for all of them (the pass is latency-bound).  Sample
  // i = tid + j * kFinalThreads sits at position (i / 64) * step * 64 + i % 64: one lane offset
  // plus a per-j constant, read through a buffer descriptor of the whole logits row (reads past
  // it return 0; samples past the row's own ns are not counted below).
  uint32_t v[kPer];
  {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, (int)min(stride * 4, (int64_t)INT32_MAX), kBufferWord3);
    const int o0 = ((tid >> 6) * (step * 64) + (tid & 63)) * 4;
    constexpr int kJump = (kFinalThreads / 64) * step * 64 * 4;
#pragma unroll
    for (int j = 0; j < kPer; j++) v[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, o0 + j * kJump, 0, 0);
  }
  const uint32_t kmin = ws.range[2 * r], kmax = ws.range[2 * r + 1];
  const int64_t n = row_len(pos, r, stride);
  if (n <= k) {
    if (tid == 0) ws.thr[r] = 0xFFFFFFFFu;
    return;
  }
  const int64_t nsp = ((n + 63) / 64 + step - 1) / step;            // sampled pages
  const int64_t last = (nsp - 1) * step * 64;                        // first position of the last one
  const int64_t ns = (nsp - 1) * 64 + min((int64_t)64, n - last);    // sampled positions
  const int64_t m = (kMarginNum * (int64_t)k * ns + kMarginDen * n - 1) / (kMarginDen * n);
  if (m > ns) {
    if (tid == 0) ws.thr[r] = 0u;
    return;
  }
  // rows with few enough samples keep theirs in registers for both rounds
  const bool held = ns <= kThrSamples;
  if (held) {
#pragma unroll
    for (int j = 0; j < kPer; j++) v[j] = min(max(ord_key(__uint_as_float(v[j])), kmin), kmax) - kmin;
  }
  // this thread's samples are v[0 .. jn): sample tid + j * kFinalThreads exists for j < jn
  const int jn = held ? (int)min((int64_t)kPer, (ns - tid + kFinalThreads - 1) / kFinalThreads) : 0;
  // up to two 12-bit rounds over (key - kmin) (keys are close to logarithmic in the score, so
  // one round's bin near the top of the range is far too wide a step for the threshold), or one
  // round and a rank finish
  const int shift = range_shift(kmin, kmax);
  uint32_t prefix = 0;                 // high bits of (threshold - kmin) found so far
  int low = shift + 12, need = (int)m;
  for (int round = 0; round < 2 && low > 0; round++) {
    const int take = low > 12 ? 12 : low;
    const int sh = low - take;
    for (int i = tid; i < kBins; i += kFinalThreads) h[i] = 0;
    __syncthreads();
    if (held) {
#pragma unroll
      for (int j = 0; j < kPer; j++)
        if (j < jn && (low >= 32 || (v[j] >> low) == prefix)) atomicAdd(&h[(v[j] >> sh) & (kBins - 1)], 1);
    } else {
      // more samples than the registers hold: batches of kBatch per thread, every load of a
      // batch issued before any is used (one dependent load per sample would be a memory round
      // trip per iteration)
      constexpr int kBatch = kPer < 16 ? kPer : 16;
      for (int64_t i0 = 0; i0 < ns; i0 += kBatch * kFinalThreads) {
        float x[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; j++) {
          const int64_t i = i0 + tid + (int64_t)j * kFinalThreads;
          const int64_t s = (min(i, ns - 1) >> 6) * step * 64 + (min(i, ns - 1) & 63);
          x[j] = row[s];
        }
#pragma unroll
        for (int j = 0; j < kBatch; j++) {
          const int64_t i = i0 + tid + (int64_t)j * kFinalThreads;
          const uint32_t u = min(max(ord_key(x[j]), kmin), kmax) - kmin;
          if (i < ns && (low >= 32 || (u >> low) == prefix)) atomicAdd(&h[(u >> sh) & (kBins - 1)], 1);
        }
      }
    }
    __syncthreads();
    const int d = find_threshold<kFinalThreads, kBins>(h, need, scan, res);
    need -= res[1];
    prefix = (prefix << take) | (uint32_t)d;
    low = sh;
    const int in_bin = h[d];
    __syncthreads();
    if (held && low > 0 && in_bin <= kRankMax) {
      // the m-th largest sample itself, by ranking the few samples left in its bin
      int unused;
      const uint32_t x = rank_finish<kFinalThreads, kPer>(v, jn, low, prefix, in_bin, need, h, scan, res, unused);
      if (tid == 0) ws.thr[r] = kmin + x;
      return;
    }
  }
  if (tid == 0) ws.thr[r] = kmin + (prefix << low);   // lower edge of the final bin
}

__global__ void DSA_TWO_GROUPS_PER_CU k_filt_thresh(const float* __restrict__ logits, int64_t stride,
                                                    const int32_t* __restrict__ pos, int32_t k, Ws ws) {
  filt_thresh<kThrPer>(logits, stride, pos, k, ws);
}
__global__ void __launch_bounds__(kFinalThreads) k_filt_thresh_long(const float* __restrict__ logits, int64_t stride,
                                                                     const int32_t* __restrict__ pos, int32_t k, Ws ws) {
  filt_thresh<kThrPerLong>(logits, stride, pos, k, ws);
}

constexpr int kSelCap = 1024;    // candidates gathered per work-group before spilling to global appends

__global__ void __launch_bounds__(kPassThreads) k_select(const float* __restrict__ logits, int64_t stride,
                                                const int32_t* __restrict__ pos, int32_t k, Ws ws,
                                                const int* __restrict__ gate) {
  __shared__ int l_above[kTopkMax];
  __shared__ uint32_t l_ckey[kSelCap];
  __shared__ int l_cpos[kSelCap];
  __shared__ int n_above, n_cand, base_above, base_cand;
  __shared__ int h[kBins];
  __shared__ int scan[kPassThreads / 64];
  __shared__ int res[2];
  const int r = blockIdx.y;
  if (gate != nullptr && !gate[r]) return;
  const int64_t n = row_len(pos, r, stride);
  int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (n <= k || c0 >= n) return;
  const uint32_t kmin = ws.range[2 * r], kmax = ws.range[2 * r + 1];
  const int shift = range_shift(kmin, kmax);
  float4 v[kPerThread];
  load_chunk(logits + (int64_t)r * stride, c0, min(c0 + kChunk, n), v);
  // the threshold bin from the row's merged histogram (every work-group of the row finds the
  // same one; the first chunk's logits load meanwhile)
  for (int i = threadIdx.x; i < kBins; i += kPassThreads) h[i] = ws.hist[(int64_t)r * kBins + i];
  __syncthreads();
  const uint32_t T = (uint32_t)find_threshold<kPassThreads, kBins>(h, k, scan, res);
  uint32_t* ckey = ws.ckey + (int64_t)r * kCap;
  int* cpos = ws.cpos + (int64_t)r * kCap;
  for (;;) {
    const int64_t c1 = min(c0 + kChunk, n);
    if (threadIdx.x == 0) { n_above = 0; n_cand = 0; }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPerThread; u++) {
      const int64_t i = c0 + 4 * (threadIdx.x + kPassThreads * u);
      const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (i + j >= c1) continue;
        const uint32_t key = min(max(ord_key(e[j]), kmin), kmax);
        const uint32_t d = (key - kmin) >> shift;
        if (d > T) {
          const int sl = atomicAdd(&n_above, 1);
          if (sl < kTopkMax) l_above[sl] = (int)(i + j);
        } else if (d == T) {
          const int sl = atomicAdd(&n_cand, 1);
          if (sl < kSelCap) {
            l_ckey[sl] = key; l_cpos[sl] = (int)(i + j);
          } else {                                  // rare: many ties in this chunk
            const int gsl = atomicAdd(&ws.cnt[(int64_t)r * 4 + 1], 1);
            if (gsl < kCap) { ckey[gsl] = key; cpos[gsl] = (int)(i + j); }
          }
        }
      }
    }
    __syncthreads();
    // fewer than k keys of the whole row lie above T, so n_above < k here
    const int nc_local = min(n_cand, kSelCap);
    if (threadIdx.x == 0) {
      base_above = n_above ? atomicAdd(&ws.cnt[(int64_t)r * 4], n_above) : 0;
      base_cand = nc_local ? atomicAdd(&ws.cnt[(int64_t)r * 4 + 1], nc_local) : 0;
    }
    __syncthreads();
    int* above = ws.above + (int64_t)r * k;
    for (int i = threadIdx.x; i < min(n_above, kTopkMax); i += kPassThreads)
      if (base_above + i < k) above[base_above + i] = l_above[i];
    for (int i = threadIdx.x; i < nc_local; i += kPassThreads)
      if (base_cand + i < kCap) { ckey[base_cand + i] = l_ckey[i]; cpos[base_cand + i] = l_cpos[i]; }
    c0 += (int64_t)gridDim.x * kChunk;
    if (c0 >= n) break;
    load_chunk(logits + (int64_t)r * stride, c0, min(c0 + kChunk, n), v);
    __syncthreads();                    // the stage and its counters are reused for the next chunk
  }
}

__device__ inline void push(int* sel, int* n, int v) {
  const int s = atomicAdd(n, 1);
  if (s < kTopkMax) sel[s] = v;
}

// Writes the ns <= k selected positions sel[] (distinct, any order) of a row of n positions to
// out[0..k) in ascending order, -1 after them, by a counting sort on the positions' high bits:
// 2048 buckets of 2^s positions each (the smallest s with (n - 1) >> s < 2048), a block prefix
// over the bucket counts, then each position's rank among the few others of its bucket.  The
// sorted positions go back to sel and leave as one coalesced copy.  Unlike a bitmap of the row,
// the cost does not grow with n (an LDS bitmap of a 1M-position row took 71K cycles: each thread
// owned 32 consecutive words, so a wave's reads of them hit one bank), and it takes 5 barriers
// where a bitonic network over 2048 elements took 20 plus 56 lane-shuffle steps.  A bucket
// holds about one position; a row whose selection falls in one bucket costs ns compares per
// position.  scratch holds 2 * kTopkMax ints.  All kFinalThreads threads call it.
constexpr int kSortBuckets = kTopkMax;
__device__ inline void write_ascending(int* sel, int ns, int64_t n, int k, int32_t* out, int* scratch, int* scan) {
  static_assert(kTopkMax <= 2 * kFinalThreads && kSortBuckets == 2 * kFinalThreads, "two per thread");
  const int tid = threadIdx.x;
  int* start = scratch;                     // bucket counts, then start offsets
  int* grouped = scratch + kSortBuckets;    // positions grouped by bucket
  int s = 0;
  while (((n - 1) >> s) >= kSortBuckets) s++;
  start[2 * tid] = 0;
  start[2 * tid + 1] = 0;
  __syncthreads();
  int p[2], b[2], slot[2];
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int i = tid + u * kFinalThreads;
    p[u] = i < ns ? sel[i] : 0;
    b[u] = p[u] >> s;
    slot[u] = i < ns ? atomicAdd(&start[b[u]], 1) : 0;
  }
  __syncthreads();
  const int c0 = start[2 * tid], c1 = start[2 * tid + 1];
  int all;
  const int before = block_prefix<kFinalThreads>(c0 + c1, scan, &all) - c0 - c1;
  start[2 * tid] = before;
  start[2 * tid + 1] = before + c0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; u++)
    if (tid + u * kFinalThreads < ns) grouped[start[b[u]] + slot[u]] = p[u];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; u++) {
    if (tid + u * kFinalThreads >= ns) continue;
    const int b0 = start[b[u]], b1 = b[u] + 1 < kSortBuckets ? start[b[u] + 1] : ns;
    int rank = 0;
    for (int j = b0; j < b1; j++) rank += grouped[j] < p[u];
    sel[b0 + rank] = p[u];
  }
  __syncthreads();
  for (int j = tid; j < k; j += kFinalThreads) out[j] = j < ns ? sel[j] : -1;
}

__global__ void __launch_bounds__(kFinalThreads) k_final(const float* __restrict__ logits, int64_t stride,
                                                         const int32_t* __restrict__ pos, int32_t k,
                                                         int32_t* __restrict__ idx, Ws ws,
                                                         const int* __restrict__ gate) {
  __shared__ uint32_t skey[kCap];    // candidate keys; the output sort's scratch once sel is complete
  __shared__ int spos[kCap];
  static_assert(kCap >= 2 * kTopkMax, "the sort scratch fits the candidate keys");
  __shared__ int sel[kTopkMax];
  __shared__ int h[1024];
  __shared__ int scan[kFinalThreads / 64];
  __shared__ int res[2];
  __shared__ int nsel;
  const int r = blockIdx.x, tid = threadIdx.x;
  if (gate != nullptr && !gate[r]) return;
  // every candidate slot and every selected-above slot of the row is read at once, before the
  // counts arrive (slots past them hold stale words that are never used): one memory round trip
  constexpr int kPer = kCap / kFinalThreads, kPerA = kTopkMax / kFinalThreads;
  uint32_t ck[kPer];
  int cp[kPer], ab[kPerA];
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    ck[j] = ws.ckey[(int64_t)r * kCap + tid + j * kFinalThreads];
    cp[j] = ws.cpos[(int64_t)r * kCap + tid + j * kFinalThreads];
  }
#pragma unroll
  for (int j = 0; j < kPerA; j++) {
    const int i = tid + j * kFinalThreads;
    ab[j] = i < k ? ws.above[(int64_t)r * k + i] : 0;
  }
  const int64_t n = row_len(pos, r, stride);
  int32_t* out = idx + (int64_t)r * k;
  if (n <= k) {                       // short context or padded row: every visible position
    for (int j = tid; j < k; j += kFinalThreads) out[j] = j < n ? j : -1;
    return;
  }
  const uint32_t kmin = ws.range[2 * r], kmax = ws.range[2 * r + 1];
  const int shift = range_shift(kmin, kmax);
  const int* cnt = ws.cnt + (int64_t)r * 4;
  const int na = min(cnt[0], k);
  const int nc = cnt[1];
  const int need = k - na;            // >= 1: the threshold bin holds the k-th key
  const float* row = logits + (int64_t)r * stride;
  const bool in_lds = nc <= kCap;
  if (in_lds) {
#pragma unroll
    for (int j = 0; j < kPer; j++) {
      const int i = tid + j * kFinalThreads;
      if (i < nc) { skey[i] = ck[j]; spos[i] = cp[j]; }
    }
  }
#pragma unroll
  for (int j = 0; j < kPerA; j++) {
    const int i = tid + j * kFinalThreads;
    if (i < na) sel[i] = ab[j];
  }
  if (tid == 0) nsel = na;
  __syncthreads();
  // threshold bin, recovered from any candidate (all share it)
  const uint32_t T = ((in_lds ? skey[0] : ws.ckey[(int64_t)r * kCap]) - kmin) >> shift;

  // resolve the low `shift` bits of (key - kmin): by ranking the candidates against each other
  // when there are few, else in rounds of at most 10 bits
  uint32_t prefix = T;                // known high part of (key - kmin)
  int low = shift;                    // bits still to resolve
  int need_r = need;
  int n_eq = -1;                      // exact ties at the threshold among the candidates, when known
  if (in_lds && low > 0 && nc <= kRankMax) {
    uint32_t v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; j++) {
      const int i = tid + j * kFinalThreads;
      v[j] = i < nc ? skey[i] - kmin : 0u;
    }
    const int nv = (int)min((int64_t)kPer, max((int64_t)0, ((int64_t)nc - tid + kFinalThreads - 1) / kFinalThreads));
    int need_eq = 0;
    prefix = rank_finish<kFinalThreads, kPer>(v, nv, low, prefix, nc, need_r, h, scan, res, need_eq, &n_eq);   // key - kmin
    need_r = need_eq;
    low = 0;
  }
  while (low > 0) {
    const int take = low > 10 ? 10 : low;
    const int sh = low - take;
    for (int i = tid; i < 1024; i += kFinalThreads) h[i] = 0;
    __syncthreads();
    if (in_lds) {
      for (int i = tid; i < nc; i += kFinalThreads) {
        const uint32_t v = skey[i] - kmin;
        if ((v >> low) == prefix) atomicAdd(&h[(v >> sh) & ((1u << take) - 1)], 1);
      }
    } else {
      for (int64_t i = tid; i < n; i += kFinalThreads) {
        const uint32_t v = min(max(ord_key(row[i]), kmin), kmax) - kmin;
        if ((v >> low) == prefix) atomicAdd(&h[(v >> sh) & ((1u << take) - 1)], 1);
      }
    }
    __syncthreads();
    const int d = find_threshold<kFinalThreads, 1024>(h, need_r, scan, res);
    need_r -= res[1];
    prefix = (prefix << take) | (uint32_t)d;
    low = sh;
    __syncthreads();
  }
  const uint32_t thr = prefix + kmin;   // exact key of the k-th largest
  const int need_ties = need_r;         // elements equal to thr to keep (lowest positions)
  if (in_lds) {
    for (int i = tid; i < nc; i += kFinalThreads) {
      if (skey[i] > thr) {
        push(sel, &nsel, spos[i]);
      } else if (skey[i] == thr) {
        // every tie is kept when there are no more than needed; else the position rank among them
        int rank = 0;
        if (n_eq != need_ties) {
#pragma unroll 8
          for (int j = 0; j < nc; j++) rank += (skey[j] == thr && spos[j] < spos[i]);
        }
        if (rank < need_ties) push(sel, &nsel, spos[i]);
      }
    }
  } else {
    // more candidates than LDS holds: walk the row in position order
    int nties_seen = 0;
    for (int64_t b = 0; b < n; b += kFinalThreads) {
      const int64_t i = b + tid;
      const uint32_t key = i < n ? min(max(ord_key(row[i]), kmin), kmax) : 0u;
      const bool inT = i < n && ((key - kmin) >> shift) == T;
      if (inT && key > thr) push(sel, &nsel, (int)i);
      const int tie = (inT && key == thr) ? 1 : 0;
      int all;
      const int incl = block_prefix<kFinalThreads>(tie, scan, &all);
      if (tie && nties_seen + incl - 1 < need_ties) push(sel, &nsel, (int)i);
      nties_seen += all;
    }
  }
  __syncthreads();
  write_ascending(sel, min(nsel, k), n, k, out, (int*)skey, scan);
}

// The need-th largest (1 <= need <= cnt) of keys[0..cnt) in LDS, all in [base, base + 2^width),
// in radix rounds of at most 12 bits over (key - base) from bit `width` down, and a rank finish
// once the threshold bin holds at most kRankMax keys.  need_eq receives how many keys equal to
// it belong to the need largest.  All kFinalThreads threads call it; cnt <= kCap; h holds
// kFinalBins ints.
constexpr int kFinalBits = 12;
constexpr int kFinalBins = 1 << kFinalBits;
__device__ inline uint32_t kth_largest(const uint32_t* keys, int cnt, int need, uint32_t base, int width, int* h,
                                       int* scan, int* res, int& need_eq) {
  constexpr int kPer = kCap / kFinalThreads;
  const int tid = threadIdx.x;
  // this thread's keys (tid + j * kFinalThreads), relative to base, for the rank finish
  uint32_t kv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int i = tid + j * kFinalThreads;
    kv[j] = i < cnt ? keys[i] - base : 0u;
  }
  const int nv = (int)min((int64_t)kPer, max((int64_t)0, ((int64_t)cnt - tid + kFinalThreads - 1) / kFinalThreads));
  uint32_t prefix = 0;
  int low = width;
  while (low > 0) {
    const int take = low > kFinalBits ? kFinalBits : low;
    const int sh = low - take;
    for (int i = tid; i < kFinalBins; i += kFinalThreads) h[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; j++)
      if (j < nv && (low >= 32 || (kv[j] >> low) == prefix)) atomicAdd(&h[(kv[j] >> sh) & ((1u << take) - 1)], 1);
    __syncthreads();
    const int d = find_threshold<kFinalThreads, kFinalBins>(h, need, scan, res);
    need -= res[1];
    prefix = (prefix << take) | (uint32_t)d;
    low = sh;
    const int in_bin = h[d];
    __syncthreads();
    if (low > 0 && in_bin <= kRankMax)
      return base + rank_finish<kFinalThreads, kPer>(kv, nv, low, prefix, in_bin, need, h, scan, res, need_eq);
  }
  need_eq = need;
  return base + prefix;
}

// Per row: the exact top-k among its filtered candidates (all scores >= the threshold), in
// LDS; rows with fewer than k candidates or an overflowed list are flagged for the exact
// fallback instead.  Among exactly equal scores at the k-th the lower positions are kept:
// the tied positions go to their own list, and when it holds more than are needed a second
// selection over the complemented positions picks the lowest.
__global__ void DSA_TWO_GROUPS_PER_CU k_filt_final(const int32_t* __restrict__ pos, int64_t stride,
                                                              int32_t k, int32_t* __restrict__ idx, Ws ws) {
  // Under 64 KiB of LDS, so two work-groups share a CU.  The candidates (keys, then positions)
  // and, once they are selected, the output sort's scratch share one buffer; the radix
  // histogram lives in whichever of the tie list and the candidate buffer is idle at the time.
  __shared__ uint32_t cand[2 * kCap];
  __shared__ uint32_t ties[kCap];
  __shared__ int sel[kTopkMax];
  __shared__ int scan[kFinalThreads / 64];
  static_assert(kCap >= kFinalBins, "the histogram fits the tie list");
  __shared__ int res[2];
  __shared__ int nsel, nties;
  __shared__ uint32_t cmax;
  static_assert(2 * kCap >= 2 * kTopkMax, "the output sort's scratch reuses the candidate buffer");
  uint32_t* skey = cand;
  int* spos = (int*)(cand + kCap);
  const int r = blockIdx.x, tid = threadIdx.x;
  // every candidate slot of the row is read at once, before the count arrives (slots past the
  // count hold stale words that are never used), so the candidates cost one memory round trip
  constexpr int kPer = kCap / kFinalThreads;
  uint32_t key[kPer];
  int p[kPer];
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    key[j] = ws.ckey[(int64_t)r * kCap + tid + j * kFinalThreads];
    p[j] = ws.cpos[(int64_t)r * kCap + tid + j * kFinalThreads];
  }
  const int c = ws.fcnt[r];
  const uint32_t base = ws.thr[r];
  const int64_t n = row_len(pos, r, stride);
  int32_t* out = idx + (int64_t)r * k;
  if (n <= k) {                       // short context or padded row: every visible position
    for (int j = tid; j < k; j += kFinalThreads) out[j] = j < n ? j : -1;
    return;
  }
  if (c < k || c > kCap) {            // the filter kept too few (or too many): exact fallback,
    for (int i = tid; i < kBins; i += kFinalThreads) ws.hist[(int64_t)r * kBins + i] = 0;   // from a clear histogram
    if (tid == 0) ws.flag[r] = 1;
    return;
  }
  if (tid == 0) { nsel = 0; nties = 0; cmax = 0u; }
  __syncthreads();
  uint32_t mx = 0u;
  {
#pragma unroll
    for (int j = 0; j < kPer; j++) {
      const int i = tid + j * kFinalThreads;
      if (i < c) { skey[i] = key[j]; spos[i] = p[j]; mx = max(mx, key[j]); }
    }
  }
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  if ((tid & 63) == 0) atomicMax(&cmax, mx);     // one LDS atomic per wave, not per thread
  __syncthreads();
  // every candidate lies in [filter threshold, cmax]: the rounds start at that span's width
  const uint32_t span = cmax - base;
  const int width = span == 0u ? 0 : 32 - __clz(span);
  int need = 0;
  const uint32_t thr = kth_largest(skey, c, k, base, width, (int*)ties, scan, res, need);   // exact key of the k-th largest
  for (int i = tid; i < c; i += kFinalThreads) {
    if (skey[i] > thr) push(sel, &nsel, spos[i]);
    else if (skey[i] == thr) ties[atomicAdd(&nties, 1)] = ~(uint32_t)spos[i];   // larger = lower position
  }
  __syncthreads();
  const int nt = nties;               // >= need >= 1
  uint32_t tcut = 0;                  // every tie at or above it is kept
  if (nt > need) {
    int one = 0;
    tcut = kth_largest(ties, nt, need, 0u, 32, (int*)cand, scan, res, one);   // positions are unique: exactly need
  }
  for (int i = tid; i < nt; i += kFinalThreads)
    if (ties[i] >= tcut) push(sel, &nsel, (int)~ties[i]);
  __syncthreads();
  write_ascending(sel, min(nsel, k), n, k, out, (int*)cand, scan);
}

// Rows of at most 32 x NT scores: one work-group of NT threads per row does the whole
// selection, with the row's keys in registers (thread t holds positions [32t, 32t + 32)):
//  * the row's key range by a block reduction;
//  * radix rounds of 12 bits over (key - kmin) from the range's width down, until the bin
//    holding the k-th largest holds at most NT keys; those are gathered in LDS and each is
//    ranked against the others, which gives the exact key of the k-th largest without the
//    remaining rounds;
//  * the keys above it and the lowest positions among the exact ties at it, written in
//    ascending order from one block prefix count of each thread's (above, tie) counts.
// No workspace and no other launch.
constexpr int kRowPer = 32;
constexpr int kRowMax = kRowPer * kFinalThreads;        // 32,768 scores
constexpr int kRowSmallThreads = 256;                   // rows of at most 8,192 scores
template <int NT>
__global__ void __launch_bounds__(NT) k_row_topk(const float* __restrict__ logits, int64_t stride,
                                                 const int32_t* __restrict__ pos, int32_t k,
                                                 int32_t* __restrict__ idx) {
  static_assert(kBins % NT == 0 && kRowPer * NT <= 65535, "bins per thread; packed 16-bit counts");
  __shared__ int h[kBins];
  __shared__ int scan[NT / 64];
  __shared__ int res[2];
  __shared__ uint32_t red[2 * (NT / 64)];
  __shared__ uint32_t cand[NT];
  __shared__ int ncand;
  __shared__ uint32_t thr_found;
  __shared__ int need_found;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = row_len(pos, r, stride);
  int32_t* out = idx + (int64_t)r * k;
  if (n <= k) {                        // short context or padded row: every visible position
    for (int j = tid; j < k; j += NT) out[j] = j < n ? j : -1;
    return;
  }
  const float* row = logits + (int64_t)r * stride;
  const int base = kRowPer * tid;
  const int n4 = (int)((n + 3) & ~int64_t{3});           // <= stride (a multiple of 256)
  uint32_t key[kRowPer];
#pragma unroll
  for (int u = 0; u < kRowPer / 4; u++) {
    const int i = base + 4 * u;
    const float4 v = i < n4 ? *reinterpret_cast<const float4*>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    key[4 * u] = ord_key(v.x);
    key[4 * u + 1] = ord_key(v.y);
    key[4 * u + 2] = ord_key(v.z);
    key[4 * u + 3] = ord_key(v.w);
  }
  const int nv = (int)min((int64_t)kRowPer, max((int64_t)0, n - base));   // this thread's valid positions
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < kRowPer; j++)
    if (j < nv) { mn = min(mn, key[j]); mx = max(mx, key[j]); }
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  }
  if (lane == 0) { red[2 * wave] = mn; red[2 * wave + 1] = mx; }
  if (tid == 0) ncand = 0;
  __syncthreads();
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int w2 = 0; w2 < NT / 64; w2++) { kmin = min(kmin, red[2 * w2]); kmax = max(kmax, red[2 * w2 + 1]); }
  // radix rounds over d = key - kmin: the bits above `low` are known (prefix); `need` of the
  // keys whose high bits are prefix still belong to the k largest
  const uint32_t span = kmax - kmin;
  int low = span == 0u ? 0 : 32 - __clz(span);
  uint32_t prefix = 0;
  int need = k;
  bool ranked = false;
  uint32_t thr = kmin;
  while (low > 0) {
    const int take = low > 12 ? 12 : low;
    const int sh = low - take;
    for (int i = tid; i < kBins; i += NT) h[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRowPer; j++) {
      const uint32_t d = key[j] - kmin;
      if (j < nv && (low >= 32 || (d >> low) == prefix)) atomicAdd(&h[(d >> sh) & ((1u << take) - 1)], 1);
    }
    __syncthreads();
    const int dg = find_threshold<NT, kBins>(h, need, scan, res);
    need -= res[1];
    prefix = (prefix << take) | (uint32_t)dg;
    low = sh;
    const int in_bin = h[dg];
    __syncthreads();
    if (low > 0 && in_bin <= NT) {
      // few keys left in the bin: rank each against the others
#pragma unroll
      for (int j = 0; j < kRowPer; j++)
        if (j < nv && ((key[j] - kmin) >> low) == prefix) cand[atomicAdd(&ncand, 1)] = key[j];
      __syncthreads();
      if (tid < in_bin) {
        const uint32_t x = cand[tid];
        int gt = 0, eq = 0;
        for (int i = 0; i < in_bin; i++) {
          const uint32_t y = cand[i];
          gt += y > x;
          eq += y == x;
        }
        if (gt < need && need <= gt + eq) { thr_found = x; need_found = need - gt; }   // one value, maybe several writers
      }
      __syncthreads();
      thr = thr_found;
      need = need_found;
      ranked = true;
      break;
    }
  }
  if (!ranked) thr = kmin + prefix;    // exact key of the k-th largest; `need` ties at it are kept
  int above = 0, ties = 0;
#pragma unroll
  for (int j = 0; j < kRowPer; j++)
    if (j < nv) { above += key[j] > thr; ties += key[j] == thr; }
  // (above, ties) packed in one int: both totals are at most 32 x NT < 2^16
  int all;
  const int incl = block_prefix<NT>((above << 16) | ties, scan, &all);
  const int above_before = (incl >> 16) - above, ties_before = (incl & 0xFFFF) - ties;
  const int keep_ties = max(0, min(ties, need - ties_before));        // the lowest positions among the ties
  int o = above_before + min(need, ties_before);
  int kept_ties = 0;
#pragma unroll
  for (int j = 0; j < kRowPer; j++) {
    if (j >= nv) continue;
    const bool tie = key[j] == thr;
    const bool keep = key[j] > thr || (tie && kept_ties < keep_ties);
    kept_ties += tie;
    if (keep) out[o++] = base + j;
  }
}

}  // namespace

size_t topk_workspace_bytes(int32_t R, int64_t /*stride*/, int32_t k) { return ws_bytes(R, k); }

bool topk_single_group_rows(int64_t max_pos) { return max_pos + 1 <= kRowMax; }

hipError_t launch_row_topk(const float* logits, int64_t stride, RowsView rows, int32_t k, int32_t* idx,
                           hipStream_t s) {
  if (rows.n <= 0) return hipSuccess;
  if ((int64_t)rows.max_pos + 1 <= (int64_t)kRowPer * kRowSmallThreads)
    hipLaunchKernelGGL(k_row_topk<kRowSmallThreads>, dim3(rows.n), dim3(kRowSmallThreads), 0, s, logits, stride,
                       rows.pos, k, idx);
  else
    hipLaunchKernelGGL(k_row_topk<kFinalThreads>, dim3(rows.n), dim3(kFinalThreads), 0, s, logits, stride, rows.pos,
                       k, idx);
  return hipGetLastError();
}

hipError_t launch_topk_init(int32_t R, int32_t k, void* ws, hipStream_t s, bool flag_all, bool zero_hist) {
  Ws w = carve(ws, R, k);
  const int64_t n = zero_hist ? (int64_t)R * kBins : (int64_t)R * 4;
  const int64_t grid = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(k_init, dim3((unsigned)grid), dim3(256), 0, s, w, R, flag_all ? 1 : 0, zero_hist ? 1 : 0);
  return hipGetLastError();
}

// Passes 2-4 (the row ranges are already in the workspace); gate: only flagged rows.  With
// few_flagged (the fused call's fallback, where most rows are not flagged and their
// work-groups exit at once), a row takes kGatedChunkGroups work-groups for passes 2 and 3.
constexpr unsigned kGatedChunkGroups = 4;
static hipError_t launch_radix_passes(const float* logits, int64_t stride, RowsView rows, int32_t k, int32_t* idx,
                                      Ws w, const int* gate, bool few_flagged, hipStream_t s) {
  const int R = rows.n;
  const int64_t visible = (int64_t)rows.max_pos + 1;
  if (visible > k) {
    unsigned nchunk = (unsigned)((visible + kChunk - 1) / kChunk);
    if (few_flagged && nchunk > kGatedChunkGroups) nchunk = kGatedChunkGroups;
    hipLaunchKernelGGL(k_hist, dim3(nchunk, R), dim3(kPassThreads), 0, s, logits, stride, rows.pos, k, w, gate);
    hipLaunchKernelGGL(k_select, dim3(nchunk, R), dim3(kPassThreads), 0, s, logits, stride, rows.pos, k, w, gate);
  }
  hipLaunchKernelGGL(k_final, dim3(R), dim3(kFinalThreads), 0, s, logits, stride, rows.pos, k, idx, w, gate);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t stride, RowsView rows, int32_t k, int32_t* idx, void* ws,
                       hipStream_t s) {
  const int R = rows.n;
  if (R <= 0) return hipSuccess;
  if (topk_single_group_rows(rows.max_pos)) return launch_row_topk(logits, stride, rows, k, idx, s);
  hipError_t e = launch_topk_init(R, k, ws, s, false, true);
  if (e != hipSuccess) return e;
  Ws w = carve(ws, R, k);
  const int64_t visible = (int64_t)rows.max_pos + 1;
  if (visible > k) {
    const unsigned nchunk = (unsigned)((visible + kChunk - 1) / kChunk);
    hipLaunchKernelGGL(k_range, dim3(nchunk, R), dim3(256), 0, s, logits, stride, rows.pos, k, w, nullptr);
  }
  return launch_radix_passes(logits, stride, rows, k, idx, w, nullptr, false, s);
}

LogitsMode topk_sample_mode(void* ws, int32_t R, int32_t k, int32_t skip_upto) {
  LogitsMode m;
  m.kind = kLogitsSample;
  m.range = carve(ws, R, k).range;
  m.skip_upto = skip_upto;
  m.page_step = kTopkSampleStep;
  return m;
}

hipError_t launch_topk_threshold(const float* logits, int64_t stride, RowsView rows, int32_t k, void* ws,
                                 hipStream_t s) {
  // samples of the longest row: one page in kTopkSampleStep, 64 positions each
  const int64_t max_samples = (((int64_t)rows.max_pos + 64) / 64 + kTopkSampleStep - 1) / kTopkSampleStep * 64;
  if (max_samples <= (int64_t)kThrPer * kFinalThreads)
    hipLaunchKernelGGL(k_filt_thresh, dim3(rows.n), dim3(kFinalThreads), 0, s, logits, stride, rows.pos, k,
                       carve(ws, rows.n, k));
  else
    hipLaunchKernelGGL(k_filt_thresh_long, dim3(rows.n), dim3(kFinalThreads), 0, s, logits, stride, rows.pos, k,
                       carve(ws, rows.n, k));
  return hipGetLastError();
}

LogitsMode topk_filter_mode(void* ws, int32_t R, int32_t k, int32_t skip_upto) {
  const Ws w = carve(ws, R, k);
  LogitsMode m;
  m.kind = kLogitsFilter;
  m.skip_upto = skip_upto;
  m.thr = w.thr;
  m.fcnt = w.fcnt;
  m.fkey = w.ckey;
  m.fpos = w.cpos;
  m.fcap = kCap;
  m.sampled_step = kTopkSampleStep;
  return m;
}

hipError_t launch_topk_filtered_final(RowsView rows, int64_t stride, int32_t k, int32_t* idx, void* ws,
                                      hipStream_t s) {
  hipLaunchKernelGGL(k_filt_final, dim3(rows.n), dim3(kFinalThreads), 0, s, rows.pos, stride, k, idx,
                     carve(ws, rows.n, k));
  return hipGetLastError();
}

LogitsMode topk_fallback_mode(void* ws, int32_t R, int32_t k, int32_t skip_upto) {
  const Ws w = carve(ws, R, k);
  LogitsMode m;
  m.kind = kLogitsFallback;
  m.skip_upto = skip_upto;
  m.flag = w.flag;
  m.range = w.range;      // the full scores widen the sample's range to the row's
  return m;
}

hipError_t launch_topk_fallback(const float* logits, int64_t stride, RowsView rows, int32_t k, int32_t* idx,
                                void* ws, bool all_flagged, hipStream_t s) {
  const Ws w = carve(ws, rows.n, k);
  return launch_radix_passes(logits, stride, rows, k, idx, w, all_flagged ? nullptr : w.flag, !all_flagged, s);
}

DSA_DEFINE_ERROR_ACCESSOR(take_device_errors_topk)

}  // namespace dsa
