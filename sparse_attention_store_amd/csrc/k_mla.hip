// k_mla.hip -- sparse MLA (absorbed / MQA form) over the selected latents.
//
// For each query row r and head h (64 heads), over the selected positions j
// (0 <= j <= pos[r]):  l_j = sm * <q[h], [c_j ; kr_j]>,  o[h] = sum_j softmax(l)_j c_j
// ("vLLM 推理链路概览: 以 GLM-5.2 为例", section Sparse MLA Attention; the latent is shared
// by all heads and also serves as the value: "GLM-5.3 推理全链路(一)", section on the
// decode MQA form and absorption).
//
// Work-group = (row, split of the row's selected keys); 4 waves; keys in tiles of 32.
//  * Record addresses of the split are resolved once into LDS (idx -> page table).
//  * Each tile's 32 records (656 B each: fp8 latent, 4 scales, bf16 rope) are loaded to
//    registers one tile ahead and written to LDS.
//  * Phase 1 (QK, wave w owns heads 16w..16w+15): S^T[32 keys x 16 heads] on
//    v_mfma_f32_16x16x32_bf16; the A operand is the key tile, converted fp8 -> bf16 with
//    its block scale in one v_cvt_scalef32_pk_bf16_fp8 per pair; q stays in registers.
//    Online softmax per head in registers (exp2 domain); P scaled by each key's block
//    scale is written to LDS for the four value blocks.
//  * Phase 2 (PV, wave w owns value dims 128w..128w+127 for all 64 heads): O += P_w V_w,
//    V read transposed straight from the fp8 key tile with ds_read_b64_tr_b8.
//  * A split's un-normalised O, running max and sum go to a workspace and a combine
//    kernel merges the splits; with one split the kernel normalises and writes bf16.
#include "dsa_device.hpp"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTile = 32;
constexpr int kLatStride = 512 + 16;       // fp8 latent row in LDS (padded)
constexpr int kRopeStride = 128 + 16;      // bf16 rope row in LDS, bytes (padded)
constexpr int kChunks = kRecBytes / 16;    // 41 x 16 B per record
constexpr int kMaxSplitKeys = 2048;
constexpr float kLog2e = 1.4426950408889634f;

struct TileLds {
  uint8_t lat[kTile * kLatStride];
  uint8_t rope[kTile * kRopeStride];
  float sc[kTile * 4];
};

__device__ inline f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 fp8 codes (two dwords) -> 8 bf16, multiplied by `scale` (exact for power-of-two scales).
__device__ inline bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi, float scale) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, scale, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, scale, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, scale, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, scale, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

struct Gather {     // one thread's share of a tile: up to 6 chunks of 16 B
  uint4 v[6];
};

__device__ inline void gather_issue(Gather& G, const uint8_t* cache, const int* phys, int tile_base, int nkeys) {
#pragma unroll
  for (int u = 0; u < 6; u++) {
    const int it = threadIdx.x + 256 * u;
    G.v[u] = make_uint4(0, 0, 0, 0);
    if (it < kTile * kChunks) {
      const int key = it / kChunks, ch = it - key * kChunks;
      const int j = tile_base + key;
      const int ph = j < nkeys ? phys[j] : -1;
      if (ph >= 0) G.v[u] = *reinterpret_cast<const uint4*>(cache + (int64_t)ph * kRecBytes + 16 * ch);
    }
  }
}

__device__ inline void gather_commit(const Gather& G, TileLds& T) {
#pragma unroll
  for (int u = 0; u < 6; u++) {
    const int it = threadIdx.x + 256 * u;
    if (it < kTile * kChunks) {
      const int key = it / kChunks, ch = it - key * kChunks;
      if (ch < 32) *reinterpret_cast<uint4*>(T.lat + key * kLatStride + 16 * ch) = G.v[u];
      else if (ch == 32) *reinterpret_cast<uint4*>(T.sc + 4 * key) = G.v[u];
      else *reinterpret_cast<uint4*>(T.rope + key * kRopeStride + 16 * (ch - 33)) = G.v[u];
    }
  }
}

template <bool kSplit>
__global__ void __launch_bounds__(256)
k_sparse_mla(const uint16_t* __restrict__ q, const int32_t* __restrict__ req, const int32_t* __restrict__ pos,
             DevPages pg, const uint8_t* __restrict__ cache, const int32_t* __restrict__ idx, int32_t k,
             int keys_per_split, float sm_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
             float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  __shared__ TileLds tiles[2];
  __shared__ __attribute__((aligned(16))) uint16_t pl[4][kHeads][kTile + 8];   // P scaled per value block
  __shared__ float alpha_s[kHeads];
  __shared__ float m_s[kHeads], l_s[kHeads];
  __shared__ int phys[kMaxSplitKeys];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int r = blockIdx.y, split = blockIdx.x;
  const int j0 = split * keys_per_split;
  const int nkeys = max(0, min(keys_per_split, k - j0));
  const int p = pos[r];
  const int rq = req[r];

  // resolve record addresses (physical token index) of this split's keys
  for (int j = tid; j < nkeys; j += 256) {
    const int s = idx[(int64_t)r * k + j0 + j];
    int ph = -1;
    if (p >= 0 && s >= 0 && s <= p) {
      const int64_t page = page_of(pg, rq, s);
      if (page >= 0) ph = (int)(page * kPage + (s & 63));
    }
    phys[j] = ph;
  }

  // q of this wave's 16 heads as the B operand: lane holds head 16w+c16, dims 32ks+8g..+7
  bf16x8 qb[18];
  {
    const uint16_t* qh = q + ((int64_t)r * kHeads + 16 * wave + c16) * kLat;
#pragma unroll
    for (int ks = 0; ks < 18; ks++) qb[ks] = *reinterpret_cast<const bf16x8*>(qh + 32 * ks + 8 * g);
  }

  f32x4 O[4][8];
#pragma unroll
  for (int a = 0; a < 4; a++)
#pragma unroll
    for (int b = 0; b < 8; b++) O[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;        // for head 16w + c16 (phase-1 role)

  __syncthreads();                              // phys ready
  const int ntiles = (nkeys + kTile - 1) / kTile;
  Gather G;
  if (ntiles > 0) {
    gather_issue(G, cache, phys, 0, nkeys);
    gather_commit(G, tiles[0]);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; t++) {
    TileLds& T = tiles[t & 1];
    const bool more = t + 1 < ntiles;
    if (more) gather_issue(G, cache, phys, (t + 1) * kTile, nkeys);

    // ---------------- phase 1: S^T (keys x heads) for this wave's heads
    f32x4 s_acc[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const int key = 16 * mt + c16;
      const float4 ksc = *reinterpret_cast<const float4*>(T.sc + 4 * key);
      const float kscale[4] = {ksc.x, ksc.y, ksc.z, ksc.w};
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 16; ks++) {
        const uint2 w8 = *reinterpret_cast<const uint2*>(T.lat + key * kLatStride + 32 * ks + 8 * g);
        acc = mfma_bf16(fp8x8_to_bf16(w8.x, w8.y, kscale[ks >> 2]), qb[ks], acc);
      }
#pragma unroll
      for (int ks = 16; ks < 18; ks++) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(T.rope + key * kRopeStride + 2 * (32 * (ks - 16) + 8 * g));
        acc = mfma_bf16(a, qb[ks], acc);
      }
      s_acc[mt] = acc;
    }
    // scores in log2 units; invalid keys -> -inf.  lane: keys 4g+i (+16 mt), head c16
    float sv[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int j = t * kTile + 16 * mt + 4 * g + i;
        const bool ok = j < nkeys && phys[j] >= 0;
        sv[mt][i] = ok ? s_acc[mt][i] * sm_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[mt][i]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
    float pv[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        pv[mt][i] = (m_new == -INFINITY) ? 0.f : exp2f(sv[mt][i] - m_new);
        psum += pv[mt][i];
      }
    l_part = l_part * alpha + psum;
    m_run = m_new;
    const int hh = 16 * wave + c16;
    if (g == 0) alpha_s[hh] = alpha;
    // P scaled by the value block scale of each key, bf16, for the four value blocks
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      float4 kb[4];
#pragma unroll
      for (int i = 0; i < 4; i++) kb[i] = *reinterpret_cast<const float4*>(T.sc + 4 * (16 * mt + 4 * g + i));
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const float s0 = b == 0 ? kb[0].x : b == 1 ? kb[0].y : b == 2 ? kb[0].z : kb[0].w;
        const float s1 = b == 0 ? kb[1].x : b == 1 ? kb[1].y : b == 2 ? kb[1].z : kb[1].w;
        const float s2 = b == 0 ? kb[2].x : b == 1 ? kb[2].y : b == 2 ? kb[2].z : kb[2].w;
        const float s3 = b == 0 ? kb[3].x : b == 1 ? kb[3].y : b == 2 ? kb[3].z : kb[3].w;
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_bits(pv[mt][0] * s0) | ((uint32_t)f32_to_bf16_bits(pv[mt][1] * s1) << 16);
        packed.y = (uint32_t)f32_to_bf16_bits(pv[mt][2] * s2) | ((uint32_t)f32_to_bf16_bits(pv[mt][3] * s3) << 16);
        *reinterpret_cast<uint2*>(&pl[b][hh][16 * mt + 4 * g]) = packed;
      }
    }
    __syncthreads();

    // ---------------- phase 2: O[64 heads x 128 dims of block w] += P_w V_w
    float al[4][4];
#pragma unroll
    for (int ht = 0; ht < 4; ht++)
#pragma unroll
      for (int i = 0; i < 4; i++) al[ht][i] = alpha_s[16 * ht + 4 * g + i];
#pragma unroll
    for (int ht = 0; ht < 4; ht++)
#pragma unroll
      for (int dt = 0; dt < 8; dt++)
#pragma unroll
        for (int i = 0; i < 4; i++) O[ht][dt][i] *= al[ht][i];
    bf16x8 pa[4];
#pragma unroll
    for (int ht = 0; ht < 4; ht++) pa[ht] = *reinterpret_cast<const bf16x8*>(&pl[wave][16 * ht + c16][8 * g]);
    // tr8: lane i of a 16-lane group points at key 8g + i/2, dims +8*(i%2); gets 8 keys of dim c16
    DSA_LDS uint8_t* lat_lds = (DSA_LDS uint8_t*)T.lat;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      const int dim0 = 128 * wave + 16 * dt;
      DSA_LDS i32x2* src =
          (DSA_LDS i32x2*)(lat_lds + (8 * g + (c16 >> 1)) * kLatStride + dim0 + 8 * (c16 & 1));
      const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(src);
      const bf16x8 vb = fp8x8_to_bf16((uint32_t)v[0], (uint32_t)v[1], 1.0f);
#pragma unroll
      for (int ht = 0; ht < 4; ht++) O[ht][dt] = mfma_bf16(pa[ht], vb, O[ht][dt]);
    }
    if (more) gather_commit(G, tiles[(t + 1) & 1]);
    __syncthreads();
  }

  // ---------------- finish: per-head max and sum
  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (g == 0) { m_s[16 * wave + c16] = m_run; l_s[16 * wave + c16] = l_tot; }
  __syncthreads();
  if (!kSplit) {
#pragma unroll
    for (int ht = 0; ht < 4; ht++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int h = 16 * ht + 4 * g + i;
        const float l = l_s[h];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t* orow = out + ((int64_t)r * kHeads + h) * kVal + 128 * wave + c16;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) orow[16 * dt] = f32_to_bf16_bits(O[ht][dt][i] * inv);
      }
    if (lse != nullptr && tid < kHeads) {
      const float l = l_s[tid];
      lse[(int64_t)r * kHeads + tid] = l > 0.f ? (m_s[tid] + log2f(l)) * 0.69314718055994531f : -INFINITY;
    }
  } else {
    const int nsplit = gridDim.x;
    float* wo = ws_o + (((int64_t)r * nsplit + split) * kHeads) * kVal;
#pragma unroll
    for (int ht = 0; ht < 4; ht++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int h = 16 * ht + 4 * g + i;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) wo[(int64_t)h * kVal + 128 * wave + 16 * dt + c16] = O[ht][dt][i];
      }
    if (tid < kHeads) {
      float* ml = ws_ml + (((int64_t)r * nsplit + split) * kHeads + tid) * 2;
      ml[0] = m_s[tid];
      ml[1] = l_s[tid];
    }
  }
}

// Merges the splits of one row: block = (row, head), 128 threads x 4 dims.
__global__ void __launch_bounds__(128) k_mla_combine(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                                                     int nsplit, uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int r = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; s++) M = fmaxf(M, ws_ml[(((int64_t)r * nsplit + s) * kHeads + h) * 2]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nsplit; s++) {
    const float* ml = ws_ml + (((int64_t)r * nsplit + s) * kHeads + h) * 2;
    const float f = (ml[0] == -INFINITY) ? 0.f : exp2f(ml[0] - M);
    L += ml[1] * f;
    const float4 o = *reinterpret_cast<const float4*>(ws_o + (((int64_t)r * nsplit + s) * kHeads + h) * kVal + 4 * tid);
    acc.x += o.x * f; acc.y += o.y * f; acc.z += o.z * f; acc.w += o.w * f;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = out + ((int64_t)r * kHeads + h) * kVal + 4 * tid;
  uint2 pk;
  pk.x = (uint32_t)f32_to_bf16_bits(acc.x * inv) | ((uint32_t)f32_to_bf16_bits(acc.y * inv) << 16);
  pk.y = (uint32_t)f32_to_bf16_bits(acc.z * inv) | ((uint32_t)f32_to_bf16_bits(acc.w * inv) << 16);
  *reinterpret_cast<uint2*>(orow) = pk;
  if (lse != nullptr && tid == 0)
    lse[(int64_t)r * kHeads + h] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

int choose_splits(int32_t R, int32_t k) {
  // enough work-groups to cover 256 CUs a few times over; at least 64 keys per split
  int s = 1;
  while (s < 32 && (int64_t)R * s < 512 && k / (2 * s) >= 64) s <<= 1;
  return s;
}

}  // namespace

size_t mla_workspace_bytes(int32_t R, int32_t k) {
  const int s = choose_splits(R, k);
  if (s == 1) return 0;
  return (size_t)R * s * kHeads * (kVal + 2) * sizeof(float);
}

hipError_t launch_sparse_mla(const uint16_t* q, RowsView rows, PagesView pg, const uint8_t* cache,
                             const int32_t* idx, int32_t k, float sm_scale, uint16_t* out, float* lse, void* ws,
                             size_t ws_bytes, bool /*prefill*/, hipStream_t s) {
  const int R = rows.n;
  if (R <= 0) return hipSuccess;
  DevPages g{pg.pt, pg.pt_stride, pg.num_reqs, pg.num_pages};
  const int nsplit = choose_splits(R, k);
  const int kps = (k + nsplit - 1) / nsplit;
  const float sm_log2 = sm_scale * kLog2e;
  if (nsplit == 1) {
    hipLaunchKernelGGL(k_sparse_mla<false>, dim3(1, R), dim3(256), 0, s, q, rows.req, rows.pos, g, cache, idx, k,
                       kps, sm_log2, out, lse, nullptr, nullptr);
    return hipGetLastError();
  }
  if (ws == nullptr || ws_bytes < mla_workspace_bytes(R, k)) return hipErrorInvalidValue;
  float* wo = (float*)ws;
  float* wml = wo + (size_t)R * nsplit * kHeads * kVal;
  hipLaunchKernelGGL(k_sparse_mla<true>, dim3(nsplit, R), dim3(256), 0, s, q, rows.req, rows.pos, g, cache, idx, k,
                     kps, sm_log2, out, lse, wo, wml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_mla_combine, dim3(kHeads, R), dim3(128), 0, s, wo, wml, nsplit, out, lse);
  return hipGetLastError();
}

DSA_DEFINE_ERROR_ACCESSOR(take_device_errors_mla)

}  // namespace dsa
