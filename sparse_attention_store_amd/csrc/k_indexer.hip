// k_indexer.hip -- lightning-indexer logits over the paged FP8 index-K cache.
//
//   logits[r][s] = sum_h w[r][h] * ReLU(q_scale[r][h] * k_scale[s] * <q8[r][h], k8[s]>)
//
// for s <= pos[r], -inf after it ("vLLM 推理链路概览: 以 GLM-5.2 为例", section DSA
// Indexer for the score; section Sparse MLA Attention for the causal j <= i rule).
// Since both scales are positive powers of two, ReLU(qs*ks*x) = qs*ks*ReLU(x): the
// kernel folds w*qs per head and applies ks once per key after the head reduction.
//
// Mapping (gfx950, wave64):
//  * One work-group = one group of RG rows of one request x a chunk of pages; its four
//    waves take pages round-robin.  Every page (64 keys, 8448 B) is read from HBM once
//    per group, whatever RG is ("GLM-5.3 推理全链路(十一)", section on page-blocked
//    scoring: a page is one contiguous 8448-B burst).
//  * Contraction on the FP8 MFMA v_mfma_f32_16x16x128_f8f6f4: A = 16 heads x 128 dims of
//    q, B = 128 dims x 16 keys.  A key's 128 bytes feed the B operand directly from
//    global memory (lane l holds bytes [16g,16g+16) and [64+16g,64+16g+16) of key l%16,
//    g = l/16), so keys never pass through LDS; q is staged once per work-group in LDS.
//  * Epilogue per (row, 16-key tile): lane holds 4 heads x 1 key per head tile ->
//    8 FMAs of w'*ReLU(c); a 3-shuffle butterfly reduce-scatter over the four lane
//    groups leaves lane l with key l of the page, so each row's 64 logits are one
//    coalesced 256-B store.
//  * The next page's keys are loaded before the current page is computed.
#include "dsa_device.hpp"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kWaves = 4;

__device__ inline i32x8 load_b_operand(const uint8_t* key_row, int g) {
  i32x4 lo = *reinterpret_cast<const i32x4*>(key_row + 16 * g);
  i32x4 hi = *reinterpret_cast<const i32x4*>(key_row + 64 + 16 * g);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ inline f32x4 mfma_fp8(const i32x8& a, const i32x8& b) {
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

struct PageRegs {
  i32x8 b[4];   // four 16-key tiles
  float ks;     // scale of key `lane` of the page
};

__device__ inline void load_page(PageRegs& P, const uint8_t* page, int lane) {
  const int g = lane >> 4, k16 = lane & 15;
#pragma unroll
  for (int t = 0; t < 4; t++) P.b[t] = load_b_operand(page + (16 * t + k16) * kIdxDim, g);
  P.ks = *reinterpret_cast<const float*>(page + kIdxScaleOff + 4 * lane);
}

template <int RG>
__global__ void __launch_bounds__(256)
k_logits_decode(const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
                const int32_t* __restrict__ req, const int32_t* __restrict__ pos, DevPages pg,
                const uint8_t* __restrict__ cache, float* __restrict__ logits, int64_t stride,
                int chunk_pages) {
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[RG * kIdxHeads * kIdxDim];
  __shared__ float w_lds[RG * kIdxHeads];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, k16 = lane & 15;
  const int64_t row0 = (int64_t)blockIdx.y * RG;
  const int64_t pg0 = (int64_t)blockIdx.x * chunk_pages;
  const int64_t col_end = min((pg0 + chunk_pages) * 64, stride);

  int prow[RG];
  int pmax = -1;
#pragma unroll
  for (int r = 0; r < RG; r++) { prow[r] = pos[row0 + r]; pmax = max(pmax, prow[r]); }
  const int32_t rq = req[row0];
  // pages with a visible key (never past the logits row)
  const int64_t pend = min(min(pg0 + chunk_pages, (int64_t)(pmax >> 6) + 1), stride / 64);

  if (pg0 < pend) {
    // stage q (RG x 4 KiB) and w*q_scale in LDS
    for (int i = tid; i < RG * kIdxHeads * kIdxDim / 16; i += 256)
      reinterpret_cast<i32x4*>(q_lds)[i] = reinterpret_cast<const i32x4*>(q8 + row0 * kIdxHeads * kIdxDim)[i];
    for (int i = tid; i < RG * kIdxHeads; i += 256) w_lds[i] = w[row0 * kIdxHeads + i] * qs[row0 * kIdxHeads + i];
    __syncthreads();

    i32x8 A[RG][2];
    float wr[RG][2][4];
#pragma unroll
    for (int r = 0; r < RG; r++)
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const uint8_t* qrow = q_lds + (r * kIdxHeads + 16 * t + k16) * kIdxDim;
        i32x4 lo = *reinterpret_cast<const i32x4*>(qrow + 16 * g);
        i32x4 hi = *reinterpret_cast<const i32x4*>(qrow + 64 + 16 * g);
        A[r][t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int i = 0; i < 4; i++) wr[r][t][i] = w_lds[r * kIdxHeads + 16 * t + 4 * g + i];
      }

    int64_t pi = pg0 + wave;
    PageRegs cur, nxt;
    int64_t cur_id = pi < pend ? page_of(pg, rq, pi * 64) : -1;
    if (pi < pend && cur_id >= 0) load_page(cur, cache + cur_id * kIdxPageBytes, lane);
    for (; pi < pend; pi += kWaves) {
      const int64_t pn = pi + kWaves;
      int64_t nxt_id = pn < pend ? page_of(pg, rq, pn * 64) : -1;
      if (pn < pend && nxt_id >= 0) load_page(nxt, cache + nxt_id * kIdxPageBytes, lane);
      const int64_t s = pi * 64 + lane;
#pragma unroll
      for (int r = 0; r < RG; r++) {
        float part[4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
          f32x4 c0 = mfma_fp8(A[r][0], cur.b[t]);
          f32x4 c1 = mfma_fp8(A[r][1], cur.b[t]);
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            acc = fmaf(wr[r][0][i], fmaxf(c0[i], 0.f), acc);
            acc = fmaf(wr[r][1][i], fmaxf(c1[i], 0.f), acc);
          }
          part[t] = acc;
        }
        // reduce-scatter over lane groups g: lane group g ends with tile g (key = lane)
        const int h = g >> 1, o = g & 1;
        float keep0 = h ? part[2] : part[0], keep1 = h ? part[3] : part[1];
        float send0 = h ? part[0] : part[2], send1 = h ? part[1] : part[3];
        keep0 += __shfl_xor(send0, 32, 64);
        keep1 += __shfl_xor(send1, 32, 64);
        float mine = o ? keep1 : keep0, other = o ? keep0 : keep1;
        mine += __shfl_xor(other, 16, 64);
        float v = (cur_id >= 0 && s <= prow[r]) ? mine * cur.ks : -INFINITY;
        logits[(row0 + r) * stride + s] = v;
      }
      cur = nxt;
      cur_id = nxt_id;
    }
  }
  // columns of this chunk past the group's last visible page
  const int64_t fill0 = max(pend, pg0) * 64;
  for (int64_t c = fill0 + tid; c < col_end; c += 256)
#pragma unroll
    for (int r = 0; r < RG; r++) logits[(row0 + r) * stride + c] = -INFINITY;
}

template <int RG>
hipError_t launch_rg(const uint8_t* q8, const float* qs, const float* w, RowsView rows, DevPages g,
                     const uint8_t* cache, float* logits, int64_t stride, hipStream_t s) {
  const int64_t n_groups = rows.n / RG;
  const int64_t total_pages = stride / 64;
  // enough work-groups to cover the chip (each page is one wave-iteration)
  int chunk = 32;
  while (chunk > 4 && n_groups * ((total_pages + chunk - 1) / chunk) < 2048) chunk >>= 1;
  const int64_t nchunks = (total_pages + chunk - 1) / chunk;
  hipLaunchKernelGGL(k_logits_decode<RG>, dim3((unsigned)nchunks, (unsigned)n_groups), dim3(256), 0, s, q8, qs, w,
                     rows.req, rows.pos, g, cache, logits, stride, chunk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_logits(const uint8_t* q8, const float* qs, const float* w, RowsView rows, PagesView pg,
                                 const uint8_t* cache, float* logits, int64_t stride, hipStream_t s) {
  if (rows.n <= 0) return hipSuccess;
  DevPages g{pg.pt, pg.pt_stride, pg.num_reqs, pg.num_pages};
  // rows of a group are processed in sub-groups of the largest divisor of `group` <= 6
  // (the q operands of six rows fill the register file without spilling)
  int rg = 1;
  for (int d = 6; d >= 1; d--)
    if (rows.group % d == 0) { rg = d; break; }
  switch (rg) {
    case 6: return launch_rg<6>(q8, qs, w, rows, g, cache, logits, stride, s);
    case 5: return launch_rg<5>(q8, qs, w, rows, g, cache, logits, stride, s);
    case 4: return launch_rg<4>(q8, qs, w, rows, g, cache, logits, stride, s);
    case 3: return launch_rg<3>(q8, qs, w, rows, g, cache, logits, stride, s);
    case 2: return launch_rg<2>(q8, qs, w, rows, g, cache, logits, stride, s);
    default: return launch_rg<1>(q8, qs, w, rows, g, cache, logits, stride, s);
  }
}

DSA_DEFINE_ERROR_ACCESSOR(take_device_errors_indexer)

}  // namespace dsa
