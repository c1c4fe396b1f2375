// k_topk.hip -- per-row top-k (k <= 2048) over the indexer logits.
//
// The k largest logits among positions s <= pos[r] ("vLLM 推理链路概览: 以 GLM-5.2 为例",
// section DSA Indexer: TopK over positions j).  When pos[r] + 1 <= k every visible
// position is selected and the row is [0 .. pos[r], -1 ...] without reading logits
// ("GLM-5.3 推理全链路(十一)", section on skipping the score for short contexts).
//
// Radix select on the order-preserving 32-bit image of each fp32 logit:
//  1. k_hist:   grid (chunk, row) -> LDS histogram of the top 12 bits, merged into a
//               per-row global histogram (one atomic per non-empty bin).
//  2. k_select: grid (chunk, row) -> every work-group finds the same threshold bin T
//               (the bin holding the k-th largest) from the histogram; elements above T
//               are appended to the row's output list, elements in T to a candidate list
//               (wave-aggregated atomics).
//  3. k_final:  one work-group per row refines the low 20 bits over the candidates in
//               LDS (two 10-bit rounds), keeps the lowest positions among exact ties at
//               the threshold, sorts the k positions ascending and writes them.
//               If more candidates than fit in LDS fell into T (e.g. massive ties), the
//               same rounds run over the row in global memory instead.
#include "dsa_device.hpp"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kBins = 4096;      // 12-bit first digit
constexpr int kCap = 4096;       // candidates kept per row
constexpr int kChunk = 8192;     // logits per work-group in passes 1-2
constexpr int kFinalThreads = 1024;

struct Ws {
  int* hist;       // [R][kBins]
  int* cnt;        // [R][4]: 0 = above count, 1 = candidate count
  int* above;      // [R][k]
  uint32_t* ckey;  // [R][kCap]
  int* cpos;       // [R][kCap]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Ws carve(void* base, int32_t R, int32_t k) {
  uint8_t* p = (uint8_t*)base;
  Ws w;
  w.hist = (int*)p;        p += align256((size_t)R * kBins * 4);
  w.cnt = (int*)p;         p += align256((size_t)R * 4 * 4);
  w.above = (int*)p;       p += align256((size_t)R * k * 4);
  w.ckey = (uint32_t*)p;   p += align256((size_t)R * kCap * 4);
  w.cpos = (int*)p;
  return w;
}

__device__ inline uint32_t ord_key(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Appends for the lanes where pred holds; returns the slot (or -1).
__device__ inline int wave_append(bool pred, int* counter) {
  const int lane = threadIdx.x & 63;
  uint64_t m = __ballot(pred);
  if (m == 0) return -1;
  int leader = __ffsll((unsigned long long)m) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, __popcll(m));
  base = __shfl(base, leader, 64);
  return pred ? base + __popcll(m & ((1ull << lane) - 1ull)) : -1;
}

__global__ void k_zero(int* __restrict__ p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void __launch_bounds__(256) k_hist(const float* __restrict__ logits, int64_t stride,
                                              const int32_t* __restrict__ pos, int32_t k, Ws ws) {
  __shared__ int h[kBins];
  const int r = blockIdx.y;
  const int64_t n = min((int64_t)pos[r] + 1, stride);
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (n <= k || c0 >= n) return;
  for (int i = threadIdx.x; i < kBins; i += 256) h[i] = 0;
  __syncthreads();
  const int64_t c1 = min(c0 + kChunk, n);
  const float* row = logits + (int64_t)r * stride;
  for (int64_t i = c0 + 4 * threadIdx.x; i < c1; i += 4 * 256) {
    float4 v = *reinterpret_cast<const float4*>(row + i);   // stride and c0 are multiples of 4
    float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; j++)
      if (i + j < c1) atomicAdd(&h[ord_key(e[j]) >> 20], 1);
  }
  __syncthreads();
  int* gh = ws.hist + (int64_t)r * kBins;
  for (int i = threadIdx.x; i < kBins; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Threshold bin of a histogram held in LDS: the bin b with count(bins > b) < k <=
// count(bins >= b).  Returns b; *above_out = count(bins > b).  blockDim.x == NT.
template <int NT, int NB>
__device__ inline int find_threshold(const int* h, int k, int* scan, int* result) {
  constexpr int per = NB / NT;
  const int t = threadIdx.x;
  int local = 0;
  for (int i = 0; i < per; i++) local += h[t * per + i];
  scan[t] = local;
  __syncthreads();
  // inclusive suffix sums over threads (Hillis-Steele)
  for (int o = 1; o < NT; o <<= 1) {
    int v = scan[t] + (t + o < NT ? scan[t + o] : 0);
    __syncthreads();
    scan[t] = v;
    __syncthreads();
  }
  int running = scan[t] - local;    // count in bins of higher threads
  for (int i = per - 1; i >= 0; i--) {
    int c = h[t * per + i];
    if (running < k && running + c >= k) { result[0] = t * per + i; result[1] = running; }
    running += c;
  }
  __syncthreads();
  return result[0];
}

__global__ void __launch_bounds__(256) k_select(const float* __restrict__ logits, int64_t stride,
                                                const int32_t* __restrict__ pos, int32_t k, Ws ws) {
  __shared__ int h[kBins];
  __shared__ int scan[256];
  __shared__ int res[2];
  const int r = blockIdx.y;
  const int64_t n = min((int64_t)pos[r] + 1, stride);
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (n <= k || c0 >= n) return;
  for (int i = threadIdx.x; i < kBins; i += 256) h[i] = ws.hist[(int64_t)r * kBins + i];
  __syncthreads();
  const uint32_t T = (uint32_t)find_threshold<256, kBins>(h, k, scan, res);
  const int64_t c1 = min(c0 + kChunk, n);
  const float* row = logits + (int64_t)r * stride;
  int* cnt = ws.cnt + (int64_t)r * 4;
  int* above = ws.above + (int64_t)r * k;
  uint32_t* ckey = ws.ckey + (int64_t)r * kCap;
  int* cpos = ws.cpos + (int64_t)r * kCap;
  // uniform trip count across the block so that the wave-level ballots see every lane
  for (int64_t b = c0; b < c1; b += 4 * 256) {
    const int64_t i = b + 4 * threadIdx.x;
    float e[4] = {0.f, 0.f, 0.f, 0.f};
    if (i < c1) {
      float4 v = *reinterpret_cast<const float4*>(row + i);
      e[0] = v.x; e[1] = v.y; e[2] = v.z; e[3] = v.w;
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const bool valid = i + j < c1;
      const uint32_t key = ord_key(e[j]);
      const uint32_t bin = key >> 20;
      int slot = wave_append(valid && bin > T, &cnt[0]);
      if (slot >= 0 && slot < k) above[slot] = (int)(i + j);
      slot = wave_append(valid && bin == T, &cnt[1]);
      if (slot >= 0 && slot < kCap) { ckey[slot] = key; cpos[slot] = (int)(i + j); }
    }
  }
}

// Appends to the LDS selection list (never past its end).
__device__ inline void push(int* sel, int* n, int v) {
  const int s = atomicAdd(n, 1);
  if (s < kTopkMax) sel[s] = v;
}

// In-LDS bitonic sort of n (power of two) ints ascending; blockDim.x == kFinalThreads.
__device__ inline void bitonic_sort(int* a, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += kFinalThreads) {
        int lo = 2 * i - (i & (stride - 1));
        int hi = lo + stride;
        bool up = ((lo & size) == 0);
        int x = a[lo], y = a[hi];
        if ((x > y) == up) { a[lo] = y; a[hi] = x; }
      }
      __syncthreads();
    }
  }
}

__global__ void __launch_bounds__(kFinalThreads) k_final(const float* __restrict__ logits, int64_t stride,
                                                         const int32_t* __restrict__ pos, int32_t k,
                                                         int32_t* __restrict__ idx, Ws ws) {
  __shared__ uint32_t skey[kCap];
  __shared__ int spos[kCap];
  __shared__ int sel[kTopkMax];
  __shared__ int h[1024];
  __shared__ int scan[kFinalThreads];
  __shared__ int res[2];
  __shared__ int nsel, nties;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t n = min((int64_t)pos[r] + 1, stride);
  int32_t* out = idx + (int64_t)r * k;
  if (n <= k) {                       // short context (or padded row): all visible positions
    for (int j = tid; j < k; j += kFinalThreads) out[j] = j < n ? j : -1;
    return;
  }
  const int* cnt = ws.cnt + (int64_t)r * 4;
  const int na = min(cnt[0], k);
  const int nc = cnt[1];
  const int need = k - na;            // >= 1 by construction of the threshold bin
  const float* row = logits + (int64_t)r * stride;
  const bool in_lds = nc <= kCap;
  if (in_lds) {
    for (int i = tid; i < nc; i += kFinalThreads) { skey[i] = ws.ckey[(int64_t)r * kCap + i]; spos[i] = ws.cpos[(int64_t)r * kCap + i]; }
  }
  for (int i = tid; i < kTopkMax; i += kFinalThreads) sel[i] = 0x7FFFFFFF;
  if (tid == 0) { nsel = 0; nties = 0; }
  __syncthreads();
  // the first digit T is common to all candidates (nc >= 1 since need >= 1)
  const uint32_t T = (in_lds ? skey[0] : ws.ckey[(int64_t)r * kCap]) >> 20;

  // two 10-bit refinement rounds on bits 19..10 and 9..0
  uint32_t prefix = T;      // known high bits
  int need_r = need;
  for (int round = 0; round < 2; round++) {
    const int shift = round == 0 ? 10 : 0;
    for (int i = tid; i < 1024; i += kFinalThreads) h[i] = 0;
    __syncthreads();
    const int pshift = shift + 10;    // bits above the digit
    if (in_lds) {
      for (int i = tid; i < nc; i += kFinalThreads)
        if ((skey[i] >> pshift) == prefix) atomicAdd(&h[(skey[i] >> shift) & 1023], 1);
    } else {
      for (int64_t i = tid; i < n; i += kFinalThreads) {
        uint32_t key = ord_key(row[i]);
        if ((key >> pshift) == prefix) atomicAdd(&h[(key >> shift) & 1023], 1);
      }
    }
    __syncthreads();
    const int d = find_threshold<kFinalThreads, 1024>(h, need_r, scan, res);
    need_r -= res[1];
    prefix = (prefix << 10) | (uint32_t)d;
    __syncthreads();
  }
  const uint32_t thr = prefix;        // exact key of the k-th largest
  const int need_ties = need_r;       // how many elements equal to thr to keep
  // selected = above-bin list + candidates > thr + the lowest-position ties
  for (int i = tid; i < na; i += kFinalThreads) sel[i] = ws.above[(int64_t)r * k + i];
  if (tid == 0) nsel = na;
  __syncthreads();
  if (in_lds) {
    for (int i = tid; i < nc; i += kFinalThreads)
      if (skey[i] > thr) push(sel, &nsel, spos[i]);
    __syncthreads();
    // ties: rank each tie by position among ties, keep rank < need_ties
    for (int i = tid; i < nc; i += kFinalThreads) {
      if (skey[i] != thr) continue;
      int rank = 0;
      for (int j = 0; j < nc; j++) rank += (skey[j] == thr && spos[j] < spos[i]);
      if (rank < need_ties) push(sel, &nsel, spos[i]);
    }
  } else {
    // overflow: walk the row in position order; keys > thr inside bin T are taken,
    // ties are taken in ascending position until need_ties are kept
    for (int64_t b = 0; b < n; b += kFinalThreads) {
      const int64_t i = b + tid;
      uint32_t key = i < n ? ord_key(row[i]) : 0u;
      const bool inT = i < n && (key >> 20) == T;
      if (inT && key > thr) push(sel, &nsel, (int)i);
      const int tie = (inT && key == thr) ? 1 : 0;
      scan[tid] = tie;
      __syncthreads();
      for (int o = 1; o < kFinalThreads; o <<= 1) {        // inclusive prefix sum
        int v = scan[tid] + (tid >= o ? scan[tid - o] : 0);
        __syncthreads();
        scan[tid] = v;
        __syncthreads();
      }
      const int before = nties;
      if (tie && before + scan[tid] - 1 < need_ties) push(sel, &nsel, (int)i);
      __syncthreads();
      if (tid == 0) nties = before + scan[kFinalThreads - 1];
      __syncthreads();
    }
  }
  __syncthreads();
  int m = 1;
  while (m < k) m <<= 1;
  bitonic_sort(sel, m);
  for (int j = tid; j < k; j += kFinalThreads) out[j] = sel[j];
}

}  // namespace

size_t topk_workspace_bytes(int32_t R, int64_t /*stride*/, int32_t k) {
  return align256((size_t)R * kBins * 4) + align256((size_t)R * 16) + align256((size_t)R * k * 4) +
         align256((size_t)R * kCap * 4) + align256((size_t)R * kCap * 4);
}

hipError_t launch_topk(const float* logits, int64_t stride, RowsView rows, int32_t k, int32_t* idx, void* ws,
                       hipStream_t s) {
  const int R = rows.n;
  if (R <= 0) return hipSuccess;
  Ws w = carve(ws, R, k);
  const int64_t nz = (int64_t)(((uint8_t*)w.above) - ((uint8_t*)w.hist)) / 4;   // hist + counters
  const int64_t zgrid = (nz + 255) / 256 < 4096 ? (nz + 255) / 256 : 4096;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)zgrid), dim3(256), 0, s, w.hist, nz);
  const int64_t visible = (int64_t)rows.max_pos + 1;
  if (visible > k) {
    const unsigned nchunk = (unsigned)((visible + kChunk - 1) / kChunk);
    hipLaunchKernelGGL(k_hist, dim3(nchunk, R), dim3(256), 0, s, logits, stride, rows.pos, k, w);
    hipLaunchKernelGGL(k_select, dim3(nchunk, R), dim3(256), 0, s, logits, stride, rows.pos, k, w);
  }
  hipLaunchKernelGGL(k_final, dim3(R), dim3(kFinalThreads), 0, s, logits, stride, rows.pos, k, idx, w);
  return hipGetLastError();
}

DSA_DEFINE_ERROR_ACCESSOR(take_device_errors_topk)

}  // namespace dsa
