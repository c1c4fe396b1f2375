// k_probe.hip -- reference memory rates for the benchmark: a streaming read and a gather of
// whole 656-B latent records at the positions a sparse-MLA launch selects.  They are no step
// of the layer; the benchmark reports each hot kernel's rate beside the rate of the plain
// access pattern it performs, measured on the same device.
#include "../../include/dsa.h"
#include "dsa_device.hpp"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kInFlight = 8;           // independent 16-B loads per thread per step

__device__ inline uint32_t xor4(const i32x4& v) { return (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]); }

// XOR of the work-group's words to sink[blockIdx.x] (one plain store per work-group: atomics of
// every wave on one word serialise and took as long as the reads), so that no load is dropped.
__device__ inline void fold_into(uint32_t acc, uint32_t* sink) {
  __shared__ uint32_t part[kProbeThreads / 64];
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kProbeThreads / 64; w++) acc ^= part[w];
    sink[blockIdx.x] = acc;
  }
}

// Non-temporal 16-B loads: in these probes they read 7.1 TB/s against 6.3 for plain loads (stream)
// and 5.5 against 5.2-5.3 (gather), so the reference is the faster of the two.
__device__ inline i32x4 ld_nt(const i32x4* p) { return __builtin_nontemporal_load(p); }

// Read of n16 16-B chunks: each step of a work-group covers kInFlight consecutive blocks of
// kProbeThreads chunks (one 4-KiB block per wave-wide load set), all issued before any is used.
__global__ void __launch_bounds__(kProbeThreads) k_stream_read(const i32x4* __restrict__ p, int64_t n16,
                                                              uint32_t* __restrict__ sink) {
  const int64_t step = (int64_t)gridDim.x * kProbeThreads * kInFlight;
  uint32_t acc = 0;
  for (int64_t b = (int64_t)blockIdx.x * kProbeThreads * kInFlight + threadIdx.x; b < n16; b += step) {
    i32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; u++) v[u] = ld_nt(p + min(b + u * kProbeThreads, n16 - 1));
#pragma unroll
    for (int u = 0; u < kInFlight; u++)
      if (b + u * kProbeThreads < n16) acc ^= xor4(v[u]);
  }
  fold_into(acc, sink);
}

// The gather in batches of kProbeThreads records per work-group: the batch's record ids are
// staged in LDS once (ids outside the pool are clamped into it), then chunk c of the batch is
// 16-B chunk c % rc16 of the batch's record c / rc16, kInFlight chunks per thread in flight.
// RC16 > 0 fixes rc16 at compile time (the 41 chunks of a latent record), so the division
// costs a multiply instead of a long integer-division sequence per load.
template <int RC16>
__global__ void __launch_bounds__(kProbeThreads) k_gather_records(const uint8_t* __restrict__ pool,
                                                                 int64_t pool_records, int rc16_arg,
                                                                 const int32_t* __restrict__ ids, int64_t n,
                                                                 uint32_t* __restrict__ sink) {
  const int rc16 = RC16 > 0 ? RC16 : rc16_arg;
  __shared__ int64_t base[kProbeThreads];
  uint32_t acc = 0;
  for (int64_t b0 = (int64_t)blockIdx.x * kProbeThreads; b0 < n; b0 += (int64_t)gridDim.x * kProbeThreads) {
    const int nb = (int)min((int64_t)kProbeThreads, n - b0);
    __syncthreads();                    // the previous batch's ids are no longer read
    if ((int)threadIdx.x < nb) {
      const int64_t rec = min(max((int64_t)ids[b0 + threadIdx.x], (int64_t)0), pool_records - 1);
      base[threadIdx.x] = rec * (int64_t)(16 * rc16);
    }
    __syncthreads();
    const int total = nb * rc16;
    for (int c0 = threadIdx.x; c0 < total; c0 += kInFlight * kProbeThreads) {
      i32x4 v[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight; u++) {
        const int c = min(c0 + u * kProbeThreads, total - 1);
        v[u] = ld_nt(reinterpret_cast<const i32x4*>(pool + base[c / rc16] + 16 * (c % rc16)));
      }
#pragma unroll
      for (int u = 0; u < kInFlight; u++)
        if (c0 + u * kProbeThreads < total) acc ^= xor4(v[u]);
    }
  }
  fold_into(acc, sink);
}

constexpr int kProbeGroups = DSA_PROBE_SINK_WORDS;   // eight work-groups per CU
static_assert(kProbeGroups == 256 * 8, "one sink word per work-group");

}  // namespace

hipError_t launch_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read, dim3(kProbeGroups), dim3(kProbeThreads), 0, s, (const i32x4*)buf, bytes / 16,
                     sink);
  return hipGetLastError();
}

hipError_t launch_probe_gather_records(const uint8_t* pool, int64_t pool_records, int32_t rec_bytes,
                                       const int32_t* ids, int64_t n, uint32_t* sink, hipStream_t s) {
  if (rec_bytes == kRecBytes)
    hipLaunchKernelGGL(k_gather_records<kRecBytes / 16>, dim3(kProbeGroups), dim3(kProbeThreads), 0, s, pool,
                       pool_records, rec_bytes / 16, ids, n, sink);
  else
    hipLaunchKernelGGL(k_gather_records<0>, dim3(kProbeGroups), dim3(kProbeThreads), 0, s, pool, pool_records,
                       rec_bytes / 16, ids, n, sink);
  return hipGetLastError();
}

}  // namespace dsa
