// gen_device.hip -- device twin of gen_host.c: the same SplitMix64 counter
// generator, producing bit-identical synthetic tensors directly in HBM so that
// multi-GB inputs never cross PCIe.  Holds no arithmetic of the attention method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kG = 0x9E3779B97F4A7C15ULL;

__host__ __device__ inline uint64_t mix(uint64_t z) {
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27; z *= 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}
__host__ __device__ inline uint64_t sm(uint64_t x) { return mix(x + kG); }
__device__ inline uint64_t draw(uint64_t key, uint64_t i, uint64_t j) { return sm(key + kG * (4 * i + j)); }

__device__ inline uint16_t normal_bf16(uint64_t key, uint64_t i) {
  int64_t s = 0;
  for (int j = 0; j < 3; j++) {
    uint64_t x = draw(key, i, (uint64_t)j);
    s += (int64_t)(x & 0xFFFF) + (int64_t)((x >> 16) & 0xFFFF) +
         (int64_t)((x >> 32) & 0xFFFF) + (int64_t)(x >> 48);
  }
  float f = (float)(s - 393210) / 65536.0f;
  uint32_t u = __float_as_uint(f);
  u += 0x7FFF + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}

__global__ void k_normal(uint64_t key, uint64_t start, int64_t n, uint16_t* out) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += stride)
    out[t] = normal_bf16(key, start + (uint64_t)t);
}

__global__ void k_uniform(uint64_t key, uint64_t start, int64_t n, double mul, float* out) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += stride) {
    double u = (double)(draw(key, start + (uint64_t)t, 0) >> 40) / 16777216.0;
    out[t] = (float)(u * mul);
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (int)(g < 8192 ? (g < 1 ? 1 : g) : 8192);
}

}  // namespace

extern "C" {

int gen_dev_normal_bf16(uint64_t seed, uint64_t tensor_id, uint64_t start, int64_t n,
                        uint16_t* out, void* stream) {
  if (n <= 0) return 0;
  uint64_t key = sm(sm(seed) ^ tensor_id);
  hipLaunchKernelGGL(k_normal, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key, start, n, out);
  return (int)hipGetLastError();
}

int gen_dev_uniform_f32(uint64_t seed, uint64_t tensor_id, uint64_t start, int64_t n, double mul,
                        float* out, void* stream) {
  if (n <= 0) return 0;
  uint64_t key = sm(sm(seed) ^ tensor_id);
  hipLaunchKernelGGL(k_uniform, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key, start, n, mul, out);
  return (int)hipGetLastError();
}

}  // extern "C"
