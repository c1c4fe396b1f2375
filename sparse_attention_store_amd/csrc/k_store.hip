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
//  * fused_norm_rope_store: the step after the KV A projection in one pass per token:
//                    RMSNorm of the 512-dim latent (times gamma) and RoPE of k_pe into the
//                    656-B record, the index-K entry when the layer runs its own indexer, and
//                    the query's rope parts rotated in place ("vLLM 推理链路概览", section on
//                    the KV low-rank projection and cache; "GLM-5.3 推理全链路(一)", section
//                    4.3 on fused_norm_rope and has_indexer).
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

// fp64 -> bf16 bits with one rounding (RNE): round to odd into fp32 (16 more bits than bf16,
// so the second rounding cannot land on a false tie), then RNE on the fp32 bits.
__device__ inline uint32_t bf16_from_f64_rne(double v) {
  const float f = (float)v;
  uint32_t b = __float_as_uint(f);
  const double back = (double)f;
  if (back != v) {
    if (fabs(back) > fabs(v)) b -= 1;   // truncate toward zero (f != 0 here)
    b |= 1;                              // sticky
  }
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Rotates the interleaved pairs (x[2j], x[2j+1]) by the angles whose cosines and sines are
// c[j], s[j] (fused multiply-adds: within an ulp of double of the unfused expressions).
__device__ inline void rotate4(double* x, const double* c, const double* s) {
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const double a = x[2 * j], b = x[2 * j + 1];
    x[2 * j] = a * c[j] - b * s[j];
    x[2 * j + 1] = a * s[j] + b * c[j];
  }
}

// Eight doubles (|v| <= 448) -> eight e4m3 codes, each rounded once to nearest even.  As for
// bf16: the hardware rounds to fp32 and then to e4m3, which is one rounding unless an fp32
// value sits exactly on an e4m3 midpoint (low 20 bits 0x80000 in the normal range) or in the
// e4m3 subnormal range (below 2^-6); lanes with such a value round from the double's bits.
__device__ inline uint2 fp8x8_from_f64(const double* x) {
  float f[8];
  bool slow = false;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    f[i] = (float)x[i];
    slow |= (__float_as_uint(f[i]) & 0xFFFFFu) == 0x80000u || fabsf(f[i]) < 0x1p-6f;
  }
  uint2 out;
  if (__builtin_expect(slow, 0)) {
    out.x = out.y = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      out.x |= fp8_from_f64_rne(x[i]) << (8 * i);
      out.y |= fp8_from_f64_rne(x[4 + i]) << (8 * i);
    }
  } else {
    out.x = pack4_fp8(f[0], f[1], f[2], f[3]);
    out.y = pack4_fp8(f[4], f[5], f[6], f[7]);
  }
  return out;
}

// ue8m0 exponent from a positive fp64 amax: the smallest e with amax <= 448 * 2^e.
__device__ inline int ue8m0_exponent_d(double amax) {
  if (!(amax > 0.0)) return 0;
  const uint64_t b = (uint64_t)__double_as_longlong(amax);
  const int E = (int)(b >> 52) - 1023;
  return E - 8 + ((b & ((1ULL << 52) - 1)) > (3ULL << 50) ? 1 : 0);
}

struct FusedStoreArgs {
  const uint16_t* kv;        // [n][kv_stride]; latent at 0..511, k_pe at 512..575
  int64_t kv_stride;
  const uint16_t* gamma;     // [512] or null (1)
  const uint16_t* k_idx;     // [n][128]; used when idx is not null
  const int32_t* req;
  const int32_t* pos;
  int32_t n;
  uint8_t* lat;
  uint8_t* idx;              // null: no index-K entry (a layer without its own indexer)
  uint16_t* q_pe;            // null, or head h of token t at q_pe + t*q_row + h*q_head
  int64_t q_row, q_head;
  double rms_eps, ln_eps;
};

__device__ inline void unpack8_bf16(const uint4& u, double* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = (double)__uint_as_float(w[i] << 16);
    x[2 * i + 1] = (double)__uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Eight doubles -> eight bf16, each rounded once to nearest even.  The hardware rounds to fp32
// and then to bf16; the pair rounds as one step unless the fp32 value sits exactly on a bf16
// midpoint (low 16 bits 0x8000): only then can the first rounding have made the tie, and the
// lane redoes its eight values with the one-step rounding.
__device__ inline uint4 pack8_bf16_rne(const double* x) {
  float f[8];
  bool tie = false;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    f[i] = (float)x[i];
    tie |= (uint16_t)__float_as_uint(f[i]) == 0x8000u;
  }
  uint32_t o[4];
  if (__builtin_expect(tie, 0)) {
#pragma unroll
    for (int i = 0; i < 4; i++) o[i] = bf16_from_f64_rne(x[2 * i]) | (bf16_from_f64_rne(x[2 * i + 1]) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++)
      o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){f[2 * i], f[2 * i + 1]}, bf16x2));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// One wave per token (four per work-group).  Lane l owns latent dims 8l..8l+7 (a 16-lane group
// per fp8 block); lanes 0..7 own the 64 rope dims; lanes 0..15 own the index key; lane l rotates
// dims 8m..8m+7 (m = l mod 8) of query heads 8k + l/8.  Every load of the token is issued first
// (none depends on its position), so their latency overlaps the position lookup and the angles.
// The 32 main and 32 index RoPE angles are evaluated once, in double, by lanes 0..31 and 32..63;
// each lane fetches the four of each it needs by shuffle.
__global__ void __launch_bounds__(256, 4) k_fused_norm_rope_store(FusedStoreArgs a, DevPages pg, InvFreq fm,
                                                               InvFreq fi) {
  // the wave index is uniform: position and page-table reads become scalar loads, which do
  // not wait behind the vector loads below
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int m = lane & 7;
  if (t >= a.n) return;                 // whole waves exit together

  const double freq = lane < 32 ? fm.v[lane & 31] : fi.v[lane & 31];   // issued first: needed first
  const uint16_t* src = a.kv + t * a.kv_stride;
  const uint4 kv_u = *reinterpret_cast<const uint4*>(src + lane * 8);
  const uint4 kpe_u = *reinterpret_cast<const uint4*>(src + kVal + m * 8);
  // optional operands are loaded unconditionally (from the token's own kv row when absent) so
  // every path has the same loads in flight and the waits below stay partial
  const uint4 g_u = *reinterpret_cast<const uint4*>((a.gamma ? a.gamma : src) + lane * 8);
  const uint4 ki_u =
      *reinterpret_cast<const uint4*>((a.idx ? a.k_idx + t * kIdxDim : src) + (lane & 15) * 8);
  uint16_t* qt = a.q_pe ? a.q_pe + t * a.q_row + m * 8 : nullptr;
  const int64_t qh = a.q_pe ? a.q_head : 0;
  const uint16_t* qsrc = a.q_pe ? qt : src + m * 8;
  uint4 qv[8];
#pragma unroll
  for (int k = 0; k < 8; k++) qv[k] = *reinterpret_cast<const uint4*>(qsrc + (8 * k + (lane >> 3)) * qh);

  const int64_t p = a.pos[t];
  if (p < 0) return;                    // padded token: nothing stored, q left alone
  const int64_t page = page_of(pg, a.req[t], p);
  if (page < 0) return;

  double ang_s, ang_c;
  sincos((double)p * freq, &ang_s, &ang_c);

  // latent: RMSNorm over 512 dims in double, times gamma, then four ue8m0-scaled fp8 blocks
  double x[8], g[8], sq = 0.0;
  unpack8_bf16(kv_u, x);
  unpack8_bf16(g_u, g);
#pragma unroll
  for (int i = 0; i < 8; i++) sq += x[i] * x[i];
  const double rinv = 1.0 / sqrt(group_sum_d<64>(sq) / 512.0 + a.rms_eps);
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    x[i] = x[i] * rinv * (a.gamma ? g[i] : 1.0);
    amax = fmax(amax, fabs(x[i]));
  }
  const int e = ue8m0_exponent_d(group_max_d<16>(amax));
  const double sinv = __builtin_ldexp(1.0, -e);
#pragma unroll
  for (int i = 0; i < 8; i++) x[i] *= sinv;            // exact: a power of two
  uint8_t* rec = a.lat + page * kLatPageBytes + (p & 63) * kRecBytes;
  *reinterpret_cast<uint2*>(rec + lane * 8) = fp8x8_from_f64(x);
  if ((lane & 15) == 0) *reinterpret_cast<float*>(rec + kRecScaleOff + (lane >> 4) * 4) = __builtin_ldexpf(1.0f, e);

  // index-K entry: LayerNorm, RoPE on dims 0..63, ue8m0 + fp8.  All four 16-lane groups
  // compute the key (the group reductions need every lane); group 0 stores it.
  if (a.idx) {
    const int l16 = lane & 15;
    double y[8], sum = 0.0;
    unpack8_bf16(ki_u, y);
#pragma unroll
    for (int i = 0; i < 8; i++) sum += y[i];
    const double mu = group_sum_d<16>(sum) / 128.0;
    double s2 = 0.0;
#pragma unroll
    for (int i = 0; i < 8; i++) { y[i] -= mu; s2 += y[i] * y[i]; }
    const double inv = 1.0 / sqrt(group_sum_d<16>(s2) / 128.0 + a.ln_eps);
#pragma unroll
    for (int i = 0; i < 8; i++) y[i] *= inv;
    double ci[4], si[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      ci[j] = __shfl(ang_c, 32 + 4 * m + j, 64);
      si[j] = __shfl(ang_s, 32 + 4 * m + j, 64);
    }
    if (l16 < 8) rotate4(y, ci, si);
    double am = 0.0;
#pragma unroll
    for (int i = 0; i < 8; i++) am = fmax(am, fabs(y[i]));
    const int ek = ue8m0_exponent_d(group_max_d<16>(am));
    const double kinv = __builtin_ldexp(1.0, -ek);
#pragma unroll
    for (int i = 0; i < 8; i++) y[i] *= kinv;
    const uint2 kc = fp8x8_from_f64(y);
    if (lane < 16) {
      uint8_t* base = a.idx + page * kIdxPageBytes;
      *reinterpret_cast<uint2*>(base + (p & 63) * kIdxDim + l16 * 8) = kc;
      if (l16 == 0) *reinterpret_cast<float*>(base + kIdxScaleOff + (p & 63) * 4) = __builtin_ldexpf(1.0f, ek);
    }
  }

  // main RoPE angles for dims 8m..8m+7, shared by k_pe and the query heads
  double cm[4], sm[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    cm[j] = __shfl(ang_c, 4 * m + j, 64);
    sm[j] = __shfl(ang_s, 4 * m + j, 64);
  }

  // k_pe: RoPE in double, one rounding to bf16 (lanes 0..7 store)
  if (lane < 8) {
    double r[8];
    unpack8_bf16(kpe_u, r);
    rotate4(r, cm, sm);
    *reinterpret_cast<uint4*>(rec + kRecRopeOff + lane * 16) = pack8_bf16_rne(r);
  }

  // query rope parts, rotated in place
  if (qt) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      double r[8];
      unpack8_bf16(qv[k], r);
      rotate4(r, cm, sm);
      *reinterpret_cast<uint4*>(qt + (8 * k + (lane >> 3)) * a.q_head) = pack8_bf16_rne(r);
    }
  }
}

}  // namespace

hipError_t launch_fused_norm_rope_store(const FusedStoreParams& f, RowsView tok, PagesView pg, hipStream_t s) {
  if (tok.n <= 0) return hipSuccess;
  InvFreq fm, fi;
  for (int i = 0; i < 32; i++) {
    fm.v[i] = f.inv_freq[i];
    fi.v[i] = f.index_inv_freq[i];
  }
  FusedStoreArgs a{f.kv, f.kv_stride, f.gamma, f.k_idx, tok.req, tok.pos, tok.n, f.latent_cache, f.index_cache,
                   f.q_pe, f.q_row_stride, f.q_head_stride, f.rms_eps, f.ln_eps};
  DevPages g{pg.pt, pg.pt_stride, pg.num_reqs, pg.num_pages};
  const int64_t grid = ((int64_t)tok.n + 3) / 4;
  hipLaunchKernelGGL(k_fused_norm_rope_store, dim3((unsigned)grid), dim3(256), 0, s, a, g, fm, fi);
  return hipGetLastError();
}

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
