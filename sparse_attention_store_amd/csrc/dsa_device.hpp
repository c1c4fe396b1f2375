// dsa_device.hpp -- device-side building blocks shared by the libdsa kernels
// (gfx950 / CDNA4, wave64).  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kPage = 64;
constexpr int kIdxDim = 128;
constexpr int kIdxHeads = 32;
constexpr int kIdxPageBytes = 8448;     // 64 x 128 B keys + 64 x 4 B scales
constexpr int kIdxScaleOff = 8192;
// MXFP4 index-K page: 64 x 64 B of packed e2m1 codes (lower dim in the low nibble), then
// 64 x 4 E8M0 scale bytes, one per 32 dims: 68 B per token
constexpr int kMx4KeyBytes = 64;
constexpr int kMx4ScaleOff = kPage * kMx4KeyBytes;          // 4096
constexpr int kMx4PageBytes = kPage * (kMx4KeyBytes + 4);   // 4352
constexpr int kHeads = 64;
constexpr int kLat = 576;
constexpr int kVal = 512;
constexpr int kRope = 64;
constexpr int kRecBytes = 656;          // 512 fp8 + 16 scales + 128 rope bytes
constexpr int kRecScaleOff = 512;
constexpr int kRecRopeOff = 528;
constexpr int kLatPageBytes = kPage * kRecBytes;
constexpr int kTopkMax = 2048;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define DSA_LDS __attribute__((address_space(3)))
#define DSA_GLOBAL __attribute__((address_space(1)))

// Device error flag raised by in-kernel range checks (page ids, indices); one per
// translation unit, read and cleared by that unit's take_device_errors_*().
static __device__ int g_dsa_device_error;
__device__ inline void raise_device_error(int code) { atomicOr(&g_dsa_device_error, code); }
enum { kErrPageId = 1, kErrIndex = 2, kErrRequest = 4 };

// bf16 bit pattern -> fp32 (exact).
__device__ inline float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ inline uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// ue8m0 exponent: the smallest e with amax <= 448 * 2^e, from the fp32 bit pattern.
// amax = 1.f * 2^E with mantissa fraction f; 448 = 1.75 * 2^8, so e = E - 8 when the
// fraction is <= 0.75 (bits <= 0x600000), else E - 7.  amax == 0 gives e = 0.
__device__ inline int ue8m0_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  uint32_t b = __float_as_uint(amax);
  int bias = 0;
  if ((b >> 23) == 0) {  // subnormal: renormalise exactly
    b = __float_as_uint(amax * 0x1p64f);
    bias = 64;
  }
  int E = (int)(b >> 23) - 127 - bias;
  return E - 8 + ((b & 0x7FFFFF) > 0x600000 ? 1 : 0);
}

// Two fp32 -> two OCP e4m3 codes (hardware RNE; inputs are within +-448 here).
__device__ inline uint32_t pack2_fp8(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}
__device__ inline uint32_t pack4_fp8(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// fp64 -> e4m3 code with a single rounding (RNE), for |v| <= 448.  Integer logic on
// the double's bits: keep 3 mantissa bits, round on the 49 dropped ones.
__device__ inline uint32_t fp8_from_f64_rne(double v) {
  uint64_t bits = (uint64_t)__double_as_longlong(v);
  uint32_t sign = (uint32_t)(bits >> 63) << 7;
  uint64_t a = bits & 0x7FFFFFFFFFFFFFFFULL;
  if (a == 0) return sign;
  int e = (int)(a >> 52) - 1023;
  if (e < -6) {                         // e4m3 subnormal: quantum 2^-9
    double t = __longlong_as_double((long long)a) * 512.0;   // exact
    return sign | (uint32_t)rint(t);    // rint: round half to even; 8 -> smallest normal
  }
  uint64_t mant = a & ((1ULL << 52) - 1);
  uint32_t q = (uint32_t)(mant >> 49);
  uint64_t rem = mant & ((1ULL << 49) - 1), half = 1ULL << 48;
  if (rem > half || (rem == half && (q & 1))) q++;
  if (q == 8) { q = 0; e++; }
  uint32_t code = (uint32_t)((e + 7) << 3) | q;
  return sign | (code > 0x7E ? 0x7Eu : code);
}

// Reductions across aligned groups of lanes (width a power of two <= 64).
template <int W>
__device__ inline float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int W>
__device__ inline double group_sum_d(double v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <int W>
__device__ inline double group_max_d(double v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

// Page table as the kernels see it.
struct DevPages {
  const int32_t* pt;
  int64_t pt_stride;
  int32_t num_reqs;
  int64_t num_pages;
};

// Page id of logical position p (>= 0) of request b, range-checked: -1 (and the
// device error flag) for a request, table column or page id out of range.
__device__ inline int64_t page_of(const DevPages& g, int32_t req, int64_t p) {
  if (req < 0 || req >= g.num_reqs || (p >> 6) >= g.pt_stride) { raise_device_error(kErrRequest); return -1; }
  int64_t pg = g.pt[(int64_t)req * g.pt_stride + (p >> 6)];
  if (pg < 0 || pg >= g.num_pages) { raise_device_error(kErrPageId); return -1; }
  return pg;
}

}  // namespace dsa

#define DSA_DEFINE_ERROR_ACCESSOR(fn)                                           \
  int fn() {                                                                    \
    int v = 0, z = 0;                                                           \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(dsa::g_dsa_device_error), 4) != hipSuccess) return -1; \
    if (hipMemcpyToSymbol(HIP_SYMBOL(dsa::g_dsa_device_error), &z, 4) != hipSuccess) return -1;   \
    return v;                                                                   \
  }
