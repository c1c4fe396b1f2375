// k_store.hip -- cache writers and the query quantiser.
//
//  * quant_fp8:      bf16 [n][128] -> fp8 E4M3 codes + one ue8m0 scale per 128
//                    (the indexer query format; "GLM-5.3 推理全链路(十一)", section on the
//                    two non-cache byte streams of the read path).
//  * index_k_store:  LayerNorm -> interleaved RoPE on dims 0..63 -> ue8m0 + fp8, into
//                    the token's slot of its 8448-B page ("GLM-5.3 推理全链路(十一)",
//                    section on what the indexer cache stores; "GLM-5.3 推理全链路(一)",
//                    section 4.5 on the interleaved indexer RoPE).
//  * latent_store:   576 bf16 -> 656-B record: 4 scaled fp8 blocks + bf16 rope tail
//                    ("GLM-5.3 推理全链路(十一)", section on the main KV cache).
//
// These writers are off the per-step critical path (a decode step stores one token
// per request); they are written for exactness first.  16 lanes own one 128-element
// block (8 elements = one 16-B load per lane); four blocks per wave.
#include "dsa_device.hpp"
#include "dsa_internal.h"

namespace dsa {
namespace {

__device__ inline void load8_bf16(const uint16_t* p, float* v) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Quantises 8 fp32 values owned by this lane of a 16-lane block group; returns the
// 8 codes packed and writes the block scale through *scale_out (all lanes agree).
__device__ inline uint2 quant8_group16(const float* v, float* scale_out) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<16>(amax);
  int e = ue8m0_exponent(amax);
  float inv = __builtin_ldexpf(1.0f, -e);        // exact power of two
  *scale_out = __builtin_ldexpf(1.0f, e);
  uint2 out;
  out.x = pack4_fp8(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);   // exact products
  out.y = pack4_fp8(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  return out;
}

__global__ void __launch_bounds__(256) k_quant_fp8(const uint16_t* __restrict__ x, int64_t n_blocks,
                                                   uint8_t* __restrict__ y, float* __restrict__ scale) {
  int64_t blk = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  int l16 = threadIdx.x & 15;
  if (blk >= n_blocks) return;          // whole 16-lane groups exit together
  float v[8];
  load8_bf16(x + blk * 128 + l16 * 8, v);
  float s;
  uint2 c = quant8_group16(v, &s);
  *reinterpret_cast<uint2*>(y + blk * 128 + l16 * 8) = c;
  if (l16 == 0) scale[blk] = s;
}

struct InvFreq { double v[32]; };

// LayerNorm then interleaved RoPE of one 128-dim key in fp64, spread over a 16-lane group
// (dims 8*l16 .. 8*l16+7 per lane), so the stored codes do not depend on fp32 rounding.
__device__ inline void ln_rope_group16(const uint16_t* kt, int l16, int64_t p, double eps, const InvFreq& f,
                                       double* x) {
  float xf[8];
  load8_bf16(kt + l16 * 8, xf);
  double sum = 0.0;
#pragma unroll
  for (int i = 0; i < 8; i++) { x[i] = (double)xf[i]; sum += x[i]; }
  double mu = group_sum_d<16>(sum) / 128.0;
  double sq = 0.0;
#pragma unroll
  for (int i = 0; i < 8; i++) { x[i] -= mu; sq += x[i] * x[i]; }
  double var = group_sum_d<16>(sq) / 128.0;
  double inv = 1.0 / sqrt(var + eps);
#pragma unroll
  for (int i = 0; i < 8; i++) x[i] *= inv;
  if (l16 < 8) {                        // dims 0..63: four interleaved pairs per lane
#pragma unroll
    for (int j = 0; j < 4; j++) {
      double s, c;
      sincos((double)p * f.v[l16 * 4 + j], &s, &c);
      double a = x[2 * j], b = x[2 * j + 1];
      x[2 * j] = a * c - b * s;
      x[2 * j + 1] = a * s + b * c;
    }
  }
}

// The final fp64 -> fp8 step rounds once.
__global__ void __launch_bounds__(256) k_index_k_store(const uint16_t* __restrict__ k, const int32_t* __restrict__ req,
                                                       const int32_t* __restrict__ pos, int32_t n, DevPages pg,
                                                       uint8_t* __restrict__ cache, double eps, InvFreq f) {
  int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  int l16 = threadIdx.x & 15;
  if (t >= n) return;
  int64_t p = pos[t];
  if (p < 0) return;                    // padded row: nothing stored
  int64_t page = page_of(pg, req[t], p);
  if (page < 0) return;
  double x[8];
  ln_rope_group16(k + t * 128, l16, p, eps, f, x);
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = fmax(amax, fabs(x[i]));
  amax = group_max_d<16>(amax);
  // ue8m0 from the fp64 bits: smallest e with amax <= 448 * 2^e (448 = 1.75 * 2^8)
  int e = 0;
  if (amax > 0.0) {
    uint64_t b = (uint64_t)__double_as_longlong(amax);
    int E = (int)(b >> 52) - 1023;
    e = E - 8 + ((b & ((1ULL << 52) - 1)) > (3ULL << 50) ? 1 : 0);
  }
  double sinv = __builtin_ldexp(1.0, -e);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) lo |= fp8_from_f64_rne(x[i] * sinv) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; i++) hi |= fp8_from_f64_rne(x[4 + i] * sinv) << (8 * i);
  uint8_t* base = cache + page * kIdxPageBytes;
  *reinterpret_cast<uint2*>(base + (p & 63) * 128 + l16 * 8) = make_uint2(lo, hi);
  if (l16 == 0) *reinterpret_cast<float*>(base + kIdxScaleOff + (p & 63) * 4) = __builtin_ldexpf(1.0f, e);
}

// e2m1 code of v (|v| <= 6 by the scale choice): round to nearest, ties to the even code.
// Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6: below 1 the step is 1/2; from 1 on, one mantissa bit
// per binade, rounded on the fp64 mantissa.
__device__ inline uint32_t fp4_from_f64_rne(double v) {
  const uint64_t bits = (uint64_t)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(bits >> 63) << 3;
  const uint64_t a = bits & 0x7FFFFFFFFFFFFFFFULL;
  const double av = __longlong_as_double((long long)a);
  if (av >= 6.0) return sign | 7u;
  if (av < 1.0) return sign | (uint32_t)rint(av * 2.0);      // 0, 1, or 2 (= 1.0)
  int e = (int)(a >> 52) - 1023;                              // 0, 1 or 2
  uint64_t mant = a & ((1ULL << 52) - 1);
  uint32_t q = (uint32_t)(mant >> 51);
  const uint64_t rem = mant & ((1ULL << 51) - 1), half = 1ULL << 50;
  if (rem > half || (rem == half && (q & 1))) q++;
  if (q == 2) { q = 0; e++; }
  const uint32_t code = (uint32_t)((e + 1) << 1) | q;
  return sign | (code > 7u ? 7u : code);
}

// MXFP4 index-K store: the same LN + RoPE, then per 32 dims (four lanes) the smallest power
// of two 2^e with amax <= 6 * 2^e, stored as the E8M0 byte e + 127, and e2m1 codes of
// x / 2^e, two per byte with the lower dim in the low nibble ("GLM-5.3 推理全链路(十一)",
// the paragraph on vLLM's MXFP4 indexer-cache format: 68 B per token).
__global__ void __launch_bounds__(256) k_index_k_store_mxfp4(const uint16_t* __restrict__ k,
                                                             const int32_t* __restrict__ req,
                                                             const int32_t* __restrict__ pos, int32_t n, DevPages pg,
                                                             uint8_t* __restrict__ cache, double eps, InvFreq f) {
  int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  int l16 = threadIdx.x & 15;
  if (t >= n) return;
  int64_t p = pos[t];
  if (p < 0) return;
  int64_t page = page_of(pg, req[t], p);
  if (page < 0) return;
  double x[8];
  ln_rope_group16(k + t * 128, l16, p, eps, f, x);
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = fmax(amax, fabs(x[i]));
  amax = group_max_d<4>(amax);          // the four lanes of this 32-dim block
  int e = 0;
  if (amax > 0.0) {                     // 6 = 1.5 * 2^2
    const uint64_t b = (uint64_t)__double_as_longlong(amax);
    const int E = (int)(b >> 52) - 1023;
    e = E - 2 + ((b & ((1ULL << 52) - 1)) > (1ULL << 51) ? 1 : 0);
  }
  const double sinv = __builtin_ldexp(1.0, -e);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) word |= fp4_from_f64_rne(x[i] * sinv) << (4 * i);
  uint8_t* base = cache + page * kMx4PageBytes;
  *reinterpret_cast<uint32_t*>(base + (p & 63) * kMx4KeyBytes + l16 * 4) = word;
  if ((l16 & 3) == 0) base[kMx4ScaleOff + (p & 63) * 4 + (l16 >> 2)] = (uint8_t)(e + 127);
}

// One wave per token: lanes 0..63 quantise latent dims 8l..8l+7 (16 lanes per block);
// lanes 0..7 copy the 128 rope bytes.
__global__ void __launch_bounds__(256) k_latent_store(const uint16_t* __restrict__ kv, const int32_t* __restrict__ req,
                                                      const int32_t* __restrict__ pos, int32_t n, DevPages pg,
                                                      uint8_t* __restrict__ cache) {
  int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  int lane = threadIdx.x & 63;
  if (t >= n) return;
  int64_t p = pos[t];
  if (p < 0) return;
  int64_t page = page_of(pg, req[t], p);
  if (page < 0) return;
  uint8_t* rec = cache + page * kLatPageBytes + (p & 63) * kRecBytes;
  const uint16_t* src = kv + t * kLat;
  float v[8];
  load8_bf16(src + lane * 8, v);
  float s;
  uint2 c = quant8_group16(v, &s);
  *reinterpret_cast<uint2*>(rec + lane * 8) = c;
  if ((lane & 15) == 0) *reinterpret_cast<float*>(rec + kRecScaleOff + (lane >> 4) * 4) = s;
  if (lane < 8)
    *reinterpret_cast<uint4*>(rec + kRecRopeOff + lane * 16) =
        *reinterpret_cast<const uint4*>(src + kVal + lane * 8);
}

}  // namespace

hipError_t launch_quant_fp8(const uint16_t* x, int64_t n_blocks, uint8_t* y, float* scale, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  int64_t grid = (n_blocks + 15) / 16;
  hipLaunchKernelGGL(k_quant_fp8, dim3((unsigned)grid), dim3(256), 0, s, x, n_blocks, y, scale);
  return hipGetLastError();
}

hipError_t launch_index_k_store_mxfp4(const uint16_t* k, RowsView tok, PagesView pg, uint8_t* cache, double eps,
                                      const double* inv_freq32, hipStream_t s) {
  if (tok.n <= 0) return hipSuccess;
  InvFreq f;
  for (int i = 0; i < 32; i++) f.v[i] = inv_freq32[i];
  DevPages g{pg.pt, pg.pt_stride, pg.num_reqs, pg.num_pages};
  int64_t grid = ((int64_t)tok.n + 15) / 16;
  hipLaunchKernelGGL(k_index_k_store_mxfp4, dim3((unsigned)grid), dim3(256), 0, s, k, tok.req, tok.pos, tok.n, g,
                     cache, eps, f);
  return hipGetLastError();
}

hipError_t launch_index_k_store(const uint16_t* k, RowsView tok, PagesView pg, uint8_t* cache, double eps,
                                const double* inv_freq32, hipStream_t s) {
  if (tok.n <= 0) return hipSuccess;
  InvFreq f;
  for (int i = 0; i < 32; i++) f.v[i] = inv_freq32[i];
  DevPages g{pg.pt, pg.pt_stride, pg.num_reqs, pg.num_pages};
  int64_t grid = ((int64_t)tok.n + 15) / 16;
  hipLaunchKernelGGL(k_index_k_store, dim3((unsigned)grid), dim3(256), 0, s, k, tok.req, tok.pos, tok.n, g, cache,
                     eps, f);
  return hipGetLastError();
}

hipError_t launch_latent_store(const uint16_t* kv, RowsView tok, PagesView pg, uint8_t* cache, hipStream_t s) {
  if (tok.n <= 0) return hipSuccess;
  DevPages g{pg.pt, pg.pt_stride, pg.num_reqs, pg.num_pages};
  int64_t grid = ((int64_t)tok.n + 3) / 4;
  hipLaunchKernelGGL(k_latent_store, dim3((unsigned)grid), dim3(256), 0, s, kv, tok.req, tok.pos, tok.n, g, cache);
  return hipGetLastError();
}

DSA_DEFINE_ERROR_ACCESSOR(take_device_errors_store)

}  // namespace dsa
