// k_mla.hip -- sparse MLA (absorbed / MQA form) over the selected latents.
//
// For each query row r and head h (64 heads), over the selected positions j
// (0 <= j <= pos[r]):  l_j = sm * <q[h], [c_j ; kr_j]>,  o[h] = sum_j softmax(l)_j c_j
// ("vLLM 推理链路概览: 以 GLM-5.2 为例", section Sparse MLA Attention; the latent is shared
// by all heads and also serves as the value: "GLM-5.3 推理全链路(一)", section on the
// decode MQA form and absorption).
//
// Work-group = (row, split of the row's selected keys); 8 waves; keys in tiles of kTile (64).
//  * Record addresses of the split are resolved once into LDS (idx -> page table).
//  * Each tile's records (656 B each: fp8 latent, 4 scales, bf16 rope) are copied from HBM
//    straight into LDS with gfx950's global_load_lds_dwordx4, kDepth tiles ahead of the compute
//    (one for 64-key tiles; explicit vmcnt waits + raw s_barrier: a full __syncthreads() would
//    drain the in-flight copies every tile).  The copies scatter the records' 16-B chunks so that every
//    wave-wide LDS access of the tile reads one contiguous block (see the tile layout below).
//  * Wave specialisation, one barrier per tile: waves 0-3 score tile t (S^T[64 keys x 16
//    heads]; the 512 latent dims on the block-scaled FP8 MFMA v_mfma_scale_f32_16x16x128_
//    f8f6f4 fed with the cached codes and their ue8m0 scales as E8M0 operands, against a
//    two-term FP8 expansion of q that keeps bf16's precision; the 64 rope dims on the bf16
//    MFMA), run the online softmax (exp2
//    domain, lazy rescaling of the running max) and write P (bf16, unscaled) to LDS; at the same time
//    waves 4-7 accumulate O += P V for tile t-1 (each owns 128 value dims = one value block
//    of all 64 heads): they scale P by each key's scale of their block, pack it to bf16 and
//    read V transposed straight from the fp8 key tile with ds_read_b64_tr_b8.  Each SIMD so
//    hosts one VALU-heavy and one MFMA-heavy wave.
//  * Few rows (R < 256): a split's un-normalised O, running max and sum go to a workspace
//    and a combine kernel merges the splits; with one split the kernel normalises and writes
//    bf16.  Many rows: a stream-K schedule, one persistent work-group per CU over equal
//    ranges of all rows' tiles; a row cut between two work-groups is merged by the second.
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <mutex>

#include "dsa_device.hpp"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 512;             // 4 QK waves + 4 PV waves
static_assert(kThreads == kVal, "the two-part merge maps one thread to each value dim");
#ifndef DSA_MLA_TILE
#define DSA_MLA_TILE 64
#endif
constexpr int kTile = DSA_MLA_TILE;        // keys per tile
static_assert(kTile == 32 || kTile == 64, "tiles of 32 or 64 keys");
constexpr int kMT = kTile / 16;            // 16-key blocks of the QK MFMAs
constexpr int kKS = kTile / 32;            // 32-key K steps of the PV MFMAs
constexpr int kChunks = kRecBytes / 16;    // 41 x 16 B per record
constexpr int kTileChunks = kTile * kChunks;            // 1312 / 2624 chunks of 16 B
constexpr int kDmaWaves = 4;                             // the QK waves issue every copy
constexpr int kTileSlots = (kTileChunks + 63) / 64;     // 21 / 41 wave-wide 1-KiB copies hold a tile
constexpr int kDmaPerWave = (kTileSlots + kDmaWaves - 1) / kDmaWaves;   // 6 / 11 per QK wave
constexpr int kTileBytes = (kTileSlots + 1) * 1024;      // + one sink for the surplus copies
#ifndef DSA_MLA_DEPTH
#define DSA_MLA_DEPTH (kTile == 32 ? 2 : 1)
#endif
constexpr int kDepth = DSA_MLA_DEPTH;                     // tiles in flight ahead of the QK tile
constexpr int kBufs = kDepth + 2;                        // + the QK tile + the PV tile
static_assert(kDepth >= 1 && kDepth <= 4, "the tile wait handles up to three tiles ahead");
static_assert(3 * kDmaPerWave < 64, "vmcnt counts the copies in flight");
static_assert(kDmaWaves * kDmaPerWave >= kTileSlots, "copy slots must cover a tile");
constexpr int kMaxSplitKeys = 2048;
static_assert(kDepth * kTile <= kMaxSplitKeys, "the first tiles' lookups stay inside phys");
static_assert(kMaxSplitKeys % kThreads == 0, "whole index loads per thread");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;      // log2 units the running max may lag behind

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

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Work-group barrier that waits for this wave's LDS traffic only (not for outstanding
// global->LDS copies, which the tile pipeline tracks with explicit vmcnt waits).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Tile layout in LDS, in 16-B chunks (41 per key).  Every wave-wide access of the scoring and
// accumulation steps reads one contiguous block: measured with the LDS bank-conflict counter,
// 16-B reads of records stored back to back (a 656-B stride between the lanes' keys) took
// twice the cycles of a contiguous 1-KiB read, and contiguous reads took none extra.
//  * chunks [0, kScaleChunk0): latent.  Block (mt * 4 + b) * 2 + half of 64 chunks holds, at
//    chunk 16 gg + kk, bytes 128 b + 64 half + 16 gg .. +16 of key 16 mt + kk;
//  * [kScaleChunk0, kRopeChunk0): the 16 scale bytes of key c - kScaleChunk0;
//  * [kRopeChunk0, kTileChunks): rope.  Block mt * 2 + ks holds, at chunk 16 gg + kk, rope
//    bytes 64 ks + 16 gg .. +16 of key 16 mt + kk.
constexpr int kScaleChunk0 = kMT * 8 * 64, kRopeChunk0 = kScaleChunk0 + kTile;
static_assert(kRopeChunk0 + kMT * 2 * 64 == kTileChunks, "the layout covers the tile");
// tile chunk of latent byte `byte` (a multiple of 8) of key `key`
__device__ __forceinline__ int lat_chunk(int key, int byte) {
  return (((key >> 4) * 4 + (byte >> 7)) * 2 + ((byte >> 6) & 1)) * 64 + 16 * ((byte >> 4) & 3) + (key & 15);
}
// tile chunk of record chunk rc of key `key`
__device__ __forceinline__ int rec_chunk(int key, int rc) {
  if (rc < kRecScaleOff / 16) return lat_chunk(key, 16 * rc);
  if (rc == kRecScaleOff / 16) return kScaleChunk0 + key;
  const int r = rc - kRecRopeOff / 16;          // rope chunk 0..7
  return kRopeChunk0 + ((key >> 4) * 2 + (r >> 2)) * 64 + 16 * (r & 3) + (key & 15);
}
// key and 16-B record chunk held at tile chunk c (0 <= c < kTileChunks)
__device__ __forceinline__ void chunk_src(int c, int& key, int& rc) {
  if (c < kScaleChunk0) {
    const int q = c >> 6, r = c & 63;
    key = 16 * (q >> 3) + (r & 15);
    rc = 8 * ((q >> 1) & 3) + 4 * (q & 1) + (r >> 4);
  } else if (c < kRopeChunk0) {
    key = c - kScaleChunk0;
    rc = kRecScaleOff / 16;
  } else {
    const int q = (c - kRopeChunk0) >> 6, r = (c - kRopeChunk0) & 63;
    key = 16 * (q >> 1) + (r & 15);
    rc = kRecRopeOff / 16 + 4 * (q & 1) + (r >> 4);
  }
}

// Global->LDS copies of one tile: lane l of copy u of a QK wave fills tile chunk
// (wave * kDmaPerWave + u) * 64 + l with its record chunk.  Each QK wave issues exactly
// kDmaPerWave copies so that per-tile vmcnt accounting is uniform; lanes past the tile or of
// invalid keys copy from the first record of the pool into the buffer (the records of
// invalid keys are zeroed before use).  The record lookups (read_tile_phys) are done a tile
// ahead of the copies (issue_copies), so the copies never wait for LDS.
__device__ __forceinline__ void read_tile_phys(const DSA_LDS int* __restrict__ phys, int tile_base, int wave, int lane,
                                               int (&ph)[kDmaPerWave]) {
#pragma unroll
  for (int u = 0; u < kDmaPerWave; u++) {
    const int c = (wave * kDmaPerWave + u) * 64 + lane;
    int key, rc;
    chunk_src(min(c, kTileChunks - 1), key, rc);
    ph[u] = phys[tile_base + key];   // < ntiles * kTile <= kMaxSplitKeys
  }
}
// Copies U0 .. U1-1 of this wave's share of a tile.
template <int U0, int U1>
__device__ __forceinline__ void issue_copies(const uint8_t* cache, const int (&ph)[kDmaPerWave], DSA_LDS uint8_t* buf,
                                             int wave, int lane) {
  static_assert(0 <= U0 && U0 <= U1 && U1 <= kDmaPerWave, "copy range");
#pragma unroll
  for (int u = U0; u < U1; u++) {
    const int c = (wave * kDmaPerWave + u) * 64 + lane;
    int key, rc;
    chunk_src(min(c, kTileChunks - 1), key, rc);
    const bool ok = c < kTileChunks && ph[u] >= 0;
    const uint8_t* src = ok ? cache + (int64_t)ph[u] * kRecBytes + 16 * rc : cache;
    const int slot = min(wave * kDmaPerWave + u, kTileSlots);   // surplus copies share the sink
    __builtin_amdgcn_global_load_lds((const void*)src, (DSA_LDS void*)(buf + slot * 1024), 16, 0, 0);
  }
}
// Zeroes the records of the invalid keys of a tile (all threads of the work-group).
__device__ __forceinline__ void zero_bad_records(DSA_LDS uint8_t* __restrict__ T, const DSA_LDS int* phys, int tile_base,
                                                 int tid) {
  for (int i = tid; i < kTileChunks; i += kThreads) {
    int key, rc;
    chunk_src(i, key, rc);
    if (phys[tile_base + key] < 0) *reinterpret_cast<DSA_LDS i32x4*>(T + 16 * i) = i32x4{0, 0, 0, 0};
  }
}

// two fp32 -> packed bf16 pair (low = a), round to nearest even, one v_cvt_pk_bf16_f32
__device__ __forceinline__ int pack2_bf16(float a, float b) {
  return __builtin_bit_cast(int, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// max over the four 16-lane rows (lanes l, l^16, l^32, l^48) with lane swaps, no LDS
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// q of one QK wave (heads 16qw..16qw+15) as MFMA B operands
struct QkOps {
  i32x8 qhi[4], qlo[4];
  int sbhi[4], sblo[4];
  bf16x8 qr[2];
};

// One pipeline step of a QK wave.  The tile pointers are restrict-qualified: the copy
// destination (tile it + kDepth) and the tile read here (tile it) are different buffers,
// which lets the compiler keep the copies in flight across the LDS reads; the arrival of
// tile `it` itself is ordered by the caller's vmcnt wait and barrier.
__device__ __forceinline__ void qk_step(const uint8_t* cache, const DSA_LDS int* __restrict__ phys, int it, int ntiles,
                                        bool bad,
                                        DSA_LDS uint8_t* __restrict__ dst, DSA_LDS uint8_t* __restrict__ T,
                                        DSA_LDS uint16_t* __restrict__ plp, DSA_LDS float* __restrict__ alpha_p,
                                        DSA_LDS int* __restrict__ resc_p, const QkOps& Q, float sm_log2, float& m_run, float& l_part, int qw, int wave,
                                        int lane, int tid, int (&phn)[kDmaPerWave]) {
  const int g = lane >> 4, c16 = lane & 15;
  // The copies of tile it + kDepth (record ids read a tile ago) go out in three groups: before
  // the first pair of 16-key blocks and after each pair's MFMAs.  A copy instruction waits for
  // room among the CU's outstanding misses; issued all at once, that wait held the wave for
  // about as long as its MFMA and softmax work that followed.  Spread out, the waits overlap
  // the MFMAs already in flight and the memory pipe is fed through the tile (c2: 198 -> 183 us
  // per launch).  The scheduling barriers keep the compiler from regrouping them.
  const bool more = it + kDepth < ntiles;
  constexpr int kCopyA = (kDmaPerWave + 2) / 3, kCopyB = kMT == 2 ? kDmaPerWave : 2 * kCopyA;
  if (more) issue_copies<0, kCopyA>(cache, phn, dst, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  if (bad) {
    zero_bad_records(T, phys, it * kTile, tid);
    lds_barrier();
  }
  // S^T (kTile keys x 16 heads): lane holds keys 16 mt + 4g + i, head c16.  The operands of
  // two 16-key blocks are read, then their MFMAs issued (two interleaved accumulator chains).
  f32x4 acc[kMT];
#pragma unroll
  for (int m0 = 0; m0 < kMT; m0 += 2) {
    i32x8 a[2][4];
    bf16x8 ar[2][2];
    int sa[2][4];
    // lane (g, c16) reads chunk `lane` of a 64-chunk block: bytes 16g.. of key 16mt + c16
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int mt = m0 + u;
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const i32x4 lo4 = *reinterpret_cast<const DSA_LDS i32x4*>(T + 16 * rec_chunk(16 * mt + c16, 8 * b + g));
        const i32x4 hi4 = *reinterpret_cast<const DSA_LDS i32x4*>(T + 16 * rec_chunk(16 * mt + c16, 8 * b + 4 + g));
        a[u][b] = i32x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
      const i32x4 ksc = *reinterpret_cast<const DSA_LDS i32x4*>(T + 16 * rec_chunk(16 * mt + c16, kRecScaleOff / 16));
#pragma unroll
      for (int b = 0; b < 4; b++) sa[u][b] = (ksc[b] >> 23) & 0xFF;   // E8M0 = the fp32 exponent of 2^e
#pragma unroll
      for (int ks = 0; ks < 2; ks++)
        ar[u][ks] = *reinterpret_cast<const DSA_LDS bf16x8*>(T + 16 * rec_chunk(16 * mt + c16, kRecRopeOff / 16 + 4 * ks + g));
    }
    f32x4 c2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int b = 0; b < 4; b++) {
#pragma unroll
      for (int u = 0; u < 2; u++)
        c2[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[u][b], Q.qhi[b], c2[u], 0, 0, 0, sa[u][b], 0,
                                                                 Q.sbhi[b]);
#pragma unroll
      for (int u = 0; u < 2; u++)
        c2[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[u][b], Q.qlo[b], c2[u], 0, 0, 0, sa[u][b], 0,
                                                                 Q.sblo[b]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int u = 0; u < 2; u++) c2[u] = mfma_bf16(ar[u][ks], Q.qr[ks], c2[u]);
    acc[m0] = c2[0];
    acc[m0 + 1] = c2[1];
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
      if (m0 == 0) issue_copies<kCopyA, kCopyB>(cache, phn, dst, wave, lane);
      else issue_copies<kCopyB, kDmaPerWave>(cache, phn, dst, wave, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  static_assert(kMT == 2 || kMT == 4, "one or two pairs of 16-key blocks per tile");

  float sv[kMT][4];
#pragma unroll
  for (int mt = 0; mt < kMT; mt++)
#pragma unroll
    for (int i = 0; i < 4; i++) sv[mt][i] = acc[mt][i] * sm_log2;
  if (bad) {     // invalid keys of the tile (runs of four consecutive entries of phys) score -inf
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) {
      const i32x4 vk = *reinterpret_cast<const DSA_LDS i32x4*>(phys + it * kTile + 16 * mt + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; i++) sv[mt][i] = vk[i] >= 0 ? sv[mt][i] : -INFINITY;
    }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < kMT; mt++)
#pragma unroll
    for (int i = 0; i < 4; i++) tmax = fmaxf(tmax, sv[mt][i]);
  tmax = rows_max(tmax);
  // lazy rescaling: the reference max only moves when the new max exceeds it by more
  // than kRescaleSlack (exp2 of the lag stays below 2^8, harmless in fp32 / bf16)
  float alpha = 1.f;
  if (tmax > m_run + kRescaleSlack) {
    alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - tmax);
    m_run = tmax;
  }
  const bool live = m_run != -INFINITY;
  float psum = 0.f;
  float p[kMT][4];
#pragma unroll
  for (int mt = 0; mt < kMT; mt++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      p[mt][i] = live ? __builtin_amdgcn_exp2f(sv[mt][i] - m_run) : 0.f;
      psum += p[mt][i];
    }
  l_part = l_part * alpha + psum;
  if (more && it + kDepth + 1 < ntiles) read_tile_phys(phys, (it + kDepth + 1) * kTile, wave, lane, phn);
  const int hh = 16 * qw + c16;
  if (g == 0) alpha_p[hh] = alpha;
  const bool any_resc = __any(alpha != 1.f);     // wave-uniform: tells the PV waves to rescale
  if (lane == 0) resc_p[qw] = any_resc;
  // P as bf16, unscaled: the PV waves multiply in each key's value-block scale (a power of
  // two, so the product is the bf16 rounding of P times the scale).  Per 32-key block ks (its
  // 64 heads x 32 keys at plp + ks * 2048), a lane's 16 B, its head's keys 32ks + 4g..4g+3 and
  // 32ks + 16+4g..16+4g+3, land at chunk 64 qw + lane: the PV waves read them as their MFMA
  // operand's K = 8g..8g+7 in that key order.
#pragma unroll
  for (int ks = 0; ks < kKS; ks++)
    *reinterpret_cast<DSA_LDS i32x4*>(plp + ks * kHeads * 32 + 8 * (64 * qw + lane)) =
        i32x4{pack2_bf16(p[2 * ks][0], p[2 * ks][1]), pack2_bf16(p[2 * ks][2], p[2 * ks][3]),
              pack2_bf16(p[2 * ks + 1][0], p[2 * ks + 1][1]), pack2_bf16(p[2 * ks + 1][2], p[2 * ks + 1][3])};
}

// Partial results cross work-groups (and XCDs, each with its own L2): they are written and
// read as relaxed agent-scope atomics, which the hardware keeps coherent across the L2s
// without a device-wide cache write-back.
__device__ __forceinline__ void store_coherent(DSA_GLOBAL float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const DSA_GLOBAL float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A row of the stream-K schedule cut between two work-groups: each part knows where both
// parts' partials go and the slot's tag word (tag null: a split of the split kernel, whose
// partial always goes to the workspace for k_mla_combine).
struct CutRow {
  float* part_o;                 // this part's un-normalised O [64][512] ...
  float* part_ml;                // ... and per head (m, l); null: a whole row
  const float* other_o;          // the other part's
  const float* other_ml;
  unsigned long long* tag;
  unsigned long long launch;
};

// Attention of query row r over keys [j0, j0 + nkeys) of its selection (one segment), as a
// warp-specialised pipeline: in iteration `it`, waves 0-3 (QK) score tile `it`, run the
// online softmax and write P for it; waves 4-7 (PV) accumulate tile it-1 with the P written
// one iteration earlier.  One barrier per iteration.
//  * QK wave q owns heads 16q..16q+15 over the full 576 contraction dims (q in registers).
//  * PV wave v owns value dims 128v..128v+127 (value block v) for all 64 heads.
// The result goes to the bf16 output (and lse) when cut.part_o is null.  Otherwise the
// segment is part of a row: its partial is un-normalised O [64][512] and, per head, the running
// max m (log2 units) and the sum l.  Without a tag it is written to part_o / part_ml.  With a
// tag (a row cut by the stream-K schedule) the part that finishes second merges: if the
// slot's tag already holds the launch, the other part is stored and this one combines it with
// its own O, still in registers, writing no partial of its own; otherwise this part stores its
// partial, waits for the stores to complete and swaps the launch into the tag, and if the
// swap returns the launch the other part got in meanwhile and this one merges after all.  The
// merger clears the tag.  No work-group waits for another.  All threads of the work-group
// call it together.
__device__ __forceinline__ void mla_segment(const uint16_t* __restrict__ q_in, const int32_t* __restrict__ req_in,
                                            const int32_t* __restrict__ pos_in, const DevPages& pg,
                                            const uint8_t* __restrict__ cache, const int32_t* __restrict__ idx_in,
                                            int32_t k, float sm_log2, int r, int j0, int nkeys,
                                            uint16_t* __restrict__ out_in, float* __restrict__ lse_in,
                                            const CutRow& cut) {
  // The stream kernel runs this body out of line, where pointer arguments arrive as generic
  // (flat) pointers; flat accesses count against the LDS counter as well, so every wait for
  // them would also wait for LDS.  Global data is therefore reached through global-space
  // pointers, and the page table's fields are read once.
  const DSA_GLOBAL uint16_t* __restrict__ q = (const DSA_GLOBAL uint16_t*)q_in;
  const DSA_GLOBAL int32_t* __restrict__ req = (const DSA_GLOBAL int32_t*)req_in;
  const DSA_GLOBAL int32_t* __restrict__ pos = (const DSA_GLOBAL int32_t*)pos_in;
  const DSA_GLOBAL int32_t* __restrict__ idx = (const DSA_GLOBAL int32_t*)idx_in;
  DSA_GLOBAL uint16_t* __restrict__ out = (DSA_GLOBAL uint16_t*)out_in;
  DSA_GLOBAL float* __restrict__ lse = (DSA_GLOBAL float*)lse_in;
  DSA_GLOBAL float* __restrict__ part_o = (DSA_GLOBAL float*)cut.part_o;
  DSA_GLOBAL float* __restrict__ part_ml = (DSA_GLOBAL float*)cut.part_ml;
  const DSA_GLOBAL float* __restrict__ other_o = (const DSA_GLOBAL float*)cut.other_o;
  const DSA_GLOBAL float* __restrict__ other_ml = (const DSA_GLOBAL float*)cut.other_ml;
  unsigned long long* const tag = cut.tag;
  const unsigned long long launch = cut.launch;
  const DSA_GLOBAL int32_t* __restrict__ pt = (const DSA_GLOBAL int32_t*)pg.pt;
  const int64_t pt_stride = pg.pt_stride, num_pages = pg.num_pages;
  const int32_t num_reqs = pg.num_reqs;
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[kBufs][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint16_t pl[2][kHeads * kTile];     // P of a tile, bf16
  __shared__ __attribute__((aligned(16))) float alpha_s[2][kHeads];
  __shared__ __attribute__((aligned(16))) int resc_s[2][4];     // per QK wave: some alpha != 1
  __shared__ float m_s[kHeads], l_s[kHeads];
  __shared__ __attribute__((aligned(16))) int phys[kMaxSplitKeys];
  __shared__ int tile_bad[kMaxSplitKeys / kTile];
  __shared__ int cut_s[2];                      // cut row: the other part was in / came in
  __shared__ float wgt_s[kHeads][3];            // merge: weight of this part, of the other, 1 / sum

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const bool is_qk = wave < 4;
  const int qw = wave & 3;                       // QK: head group; PV: value block
  const int ntiles = (nkeys + kTile - 1) / kTile;
  const int p = pos[r];
  const int rq = req[r];
  DSA_LDS uint8_t* tl = (DSA_LDS uint8_t*)&tiles[0][0];
  const DSA_LDS int* phl = (const DSA_LDS int*)phys;

  // QK waves fetch their q rows first: the loads then precede every tile copy, so the
  // per-tile vmcnt waits cover them and nothing in the loop waits for all copies
  i32x4 qraw[4][4];
  bf16x8 qr_raw[2];
  if (is_qk) {
    const DSA_GLOBAL uint16_t* qh = q + ((int64_t)r * kHeads + 16 * qw + c16) * kLat;
#pragma unroll
    for (int b = 0; b < 4; b++)
#pragma unroll
      for (int u = 0; u < 4; u++)
        qraw[b][u] = *reinterpret_cast<const DSA_GLOBAL i32x4*>(qh + 128 * b + 64 * (u >> 1) + 16 * g + 8 * (u & 1));
#pragma unroll
    for (int ks = 0; ks < 2; ks++) qr_raw[ks] = *reinterpret_cast<const DSA_GLOBAL bf16x8*>(qh + kVal + 32 * ks + 8 * g);
  }

  // resolve record addresses (physical token index) of this split's keys: every index load,
  // then every page-table load, so the lookups wait two memory round trips.  The PV waves do
  // them while the QK waves turn their q rows into MFMA operands: the conversion (about 8K
  // cycles of dependent VALU work per wave) then overlaps the lookups instead of following them
  // (one 128-key split: 9.8K cycles from entry to the barrier below, 6.1K + 8.1K before).
  for (int t = tid; t < ntiles; t += kThreads) tile_bad[t] = 0;
  __syncthreads();
  QkOps Q;
  if (!is_qk) {
    constexpr int kResolvers = kThreads / 2;
    constexpr int kPer = kMaxSplitKeys / kResolvers;
    const int rt = tid - kResolvers;
    int sv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; u++) {
      const int j = rt + u * kResolvers;
      sv[u] = j < nkeys ? idx[(int64_t)r * k + j0 + j] : -1;
    }
    // unconditional page-table reads (slot 0 stands in for keys that need none), range
    // checks after all of them, so the reads stay batched
    const bool req_ok = rq >= 0 && rq < num_reqs;
    const bool table = num_reqs > 0 && pt_stride > 0;            // uniform
    int64_t pv[kPer];
    bool want[kPer], col_ok[kPer];
#pragma unroll
    for (int u = 0; u < kPer; u++) {
      want[u] = p >= 0 && sv[u] >= 0 && sv[u] <= p;
      col_ok[u] = req_ok && (sv[u] >> 6) < pt_stride;
      pv[u] = -1;
    }
    if (table) {
      int64_t raw[kPer];
#pragma unroll
      for (int u = 0; u < kPer; u++)
        raw[u] = pt[want[u] && col_ok[u] ? (int64_t)rq * pt_stride + (sv[u] >> 6) : 0];
#pragma unroll
      for (int u = 0; u < kPer; u++) pv[u] = want[u] && col_ok[u] ? raw[u] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPer; u++) {
      if (want[u] && !col_ok[u]) raise_device_error(kErrRequest);
      if (want[u] && col_ok[u] && (pv[u] < 0 || pv[u] >= num_pages)) { raise_device_error(kErrPageId); pv[u] = -1; }
      const int j = rt + u * kResolvers;
      if (j < ntiles * kTile) {
        const int ph = want[u] && pv[u] >= 0 ? (int)(pv[u] * kPage + (sv[u] & 63)) : -1;
        phys[j] = ph;
        if (ph < 0) tile_bad[j / kTile] = 1;
      }
    }
  } else {
    // q of heads 16qw..16qw+15 as MFMA B operands.  The 512 latent dims are split into two
    // FP8 terms per 128-dim block, q = hi * 2^e_hi + lo * 2^e_lo (lo quantises the residual
    // of hi), which carries bf16's 8 significant bits; the 64 rope dims stay bf16.  Lane
    // holds head 16qw + c16, dims 128b + [16g, 16g+16) and 128b + 64 + [16g, 16g+16).
    {
#pragma unroll
      for (int b = 0; b < 4; b++) {
        float x[32];
#pragma unroll
        for (int u = 0; u < 4; u++)          // u = 2 * half + c: dims 64 * half + 16g + 8c + [0, 8)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const uint32_t wd = (uint32_t)qraw[b][u][i];
            x[8 * u + 2 * i] = __uint_as_float(wd << 16);
            x[8 * u + 2 * i + 1] = __uint_as_float(wd & 0xFFFF0000u);
          }
        // block amax over the 4 lanes holding this head's 128 dims (lanes c16, c16^16, ^32, ^48)
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 32; i++) am = fmaxf(am, fabsf(x[i]));
        am = rows_max(am);
        const int eh = ue8m0_exponent(am);
        const float ih = __builtin_ldexpf(1.0f, -eh), sh = __builtin_ldexpf(1.0f, eh);
        uint32_t hw[8];
#pragma unroll
        for (int i = 0; i < 8; i++) hw[i] = pack4_fp8(x[4 * i] * ih, x[4 * i + 1] * ih, x[4 * i + 2] * ih, x[4 * i + 3] * ih);
        // residual (exact in fp32: both terms carry few significant bits)
        float am2 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const f32x2 d0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hw[i], false);
          const f32x2 d1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hw[i], true);
          x[4 * i] -= d0[0] * sh; x[4 * i + 1] -= d0[1] * sh; x[4 * i + 2] -= d1[0] * sh; x[4 * i + 3] -= d1[1] * sh;
#pragma unroll
          for (int j = 0; j < 4; j++) am2 = fmaxf(am2, fabsf(x[4 * i + j]));
        }
        am2 = rows_max(am2);
        const int el = ue8m0_exponent(am2);
        const float il = __builtin_ldexpf(1.0f, -el);
        uint32_t lw[8];
#pragma unroll
        for (int i = 0; i < 8; i++) lw[i] = pack4_fp8(x[4 * i] * il, x[4 * i + 1] * il, x[4 * i + 2] * il, x[4 * i + 3] * il);
        Q.qhi[b] = i32x8{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
        Q.qlo[b] = i32x8{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
        Q.sbhi[b] = eh + 127;      // E8M0 scale operands
        Q.sblo[b] = el + 127;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ks++) Q.qr[ks] = qr_raw[ks];
    }
  }

  __syncthreads();                              // phys ready
  int phn[kDmaPerWave];                          // QK waves: record ids of the next tile to copy
  if (is_qk) {
    // every lookup before the first copy, so no LDS read waits for the copies in flight
    // The first kDepth tiles are always copied (tiles past the segment copy the pool's first
    // record into their unused buffer), so the number of copies after the q loads is fixed
    // and the q operands wait for the q loads only.
    int ph0[kDepth][kDmaPerWave];
#pragma unroll
    for (int t = 0; t < kDepth; t++) {
      read_tile_phys(phl, t * kTile, wave, lane, ph0[t]);      // t * kTile + 31 < kMaxSplitKeys
#pragma unroll
      for (int u = 0; u < kDmaPerWave; u++) ph0[t][u] = t < ntiles ? ph0[t][u] : -1;
    }
    if (kDepth < ntiles) read_tile_phys(phl, kDepth * kTile, wave, lane, phn);
#pragma unroll
    for (int t = 0; t < kDepth; t++) issue_copies<0, kDmaPerWave>(cache, ph0[t], tl + t * kTileBytes, wave, lane);
  }

  // Start of every iteration (both roles, same barriers in the same order): wait for this
  // wave's copies of tile `it`, then a barrier so that all of tile `it` is in LDS and every
  // wave is done with QK(it-1) and PV(it-2) (whose buffers are refilled next).
  auto wait_tile = [&](int it) {
    if (is_qk && it < ntiles) {
      // tiles it+1 .. it+kDepth-1 (those that exist) may stay in flight
      const int ahead = min(kDepth - 1, ntiles - 1 - it);
      if (ahead >= 3) wait_vmcnt<3 * kDmaPerWave>();
      else if (ahead >= 2) wait_vmcnt<2 * kDmaPerWave>();
      else if (ahead == 1) wait_vmcnt<kDmaPerWave>();
      else wait_vmcnt<0>();
    }
    lds_barrier();
  };

  if (is_qk) {
    // ======================= QK waves: heads 16qw..16qw+15, full 576 contraction dims
    // (their q operands Q were formed above, while the PV waves resolved the records)
    float m_run = -INFINITY, l_part = 0.f;      // for head 16qw + c16
    for (int it = 0; it < ntiles; it++) {
      wait_tile(it);
      const int par = it & 1;
      qk_step(cache, phl, it, ntiles, tile_bad[it] != 0, tl + ((it + kDepth) % kBufs) * kTileBytes,
              tl + (it % kBufs) * kTileBytes, (DSA_LDS uint16_t*)pl[par], (DSA_LDS float*)alpha_s[par],
              (DSA_LDS int*)resc_s[par], Q, sm_log2,
              m_run, l_part, qw, wave, lane, tid, phn);
    }
    wait_tile(ntiles);                          // the PV waves' last step
    const float l_tot = rows_sum(l_part);
    if (g == 0) { m_s[16 * qw + c16] = m_run; l_s[16 * qw + c16] = l_tot; }
    __syncthreads();
    if (part_o == nullptr) {
      if (tid < kHeads && lse != nullptr) {
        const float l = l_s[tid];
        lse[(int64_t)r * kHeads + tid] = l > 0.f ? (m_s[tid] + log2f(l)) * 0.69314718055994531f : -INFINITY;
      }
    } else if (tag == nullptr) {
      if (tid < kHeads) {
        store_coherent(&part_ml[2 * tid], m_s[tid]);
        store_coherent(&part_ml[2 * tid + 1], l_s[tid]);
      }
    } else {
      // the barriers below pair one for one with the PV waves' in the same branches
      if (tid == 0) cut_s[0] = __hip_atomic_load(tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == launch;
      __syncthreads();
      bool merge = cut_s[0] != 0;
      if (!merge) {
        if (tid < kHeads) {
          store_coherent(&part_ml[2 * tid], m_s[tid]);
          store_coherent(&part_ml[2 * tid + 1], l_s[tid]);
        }
        wait_vmcnt<0>();                        // this thread's stores are complete ...
        __syncthreads();
        if (tid == 0)                           // ... before the part is tagged
          cut_s[1] = __hip_atomic_exchange(tag, launch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == launch;
        __syncthreads();
        merge = cut_s[1] != 0;
      }
      if (merge) {
        if (tid < kHeads) {
          const float m0 = m_s[tid], l0 = l_s[tid];
          const float m1 = load_coherent(&other_ml[2 * tid]), l1 = load_coherent(&other_ml[2 * tid + 1]);
          const float M = fmaxf(m0, m1);
          const float f0 = m0 == -INFINITY ? 0.f : exp2f(m0 - M), f1 = m1 == -INFINITY ? 0.f : exp2f(m1 - M);
          const float L = l0 * f0 + l1 * f1;
          wgt_s[tid][0] = f0;
          wgt_s[tid][1] = f1;
          wgt_s[tid][2] = L > 0.f ? 1.f / L : 0.f;
          if (lse != nullptr)
            lse[(int64_t)r * kHeads + tid] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
        }
        if (tid == 0) __hip_atomic_store(tag, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();                        // weights ready
      }
    }
  } else {
    // ======================= PV waves: value dims 128qw..128qw+127 of all 64 heads
    f32x4 O[4][8];
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
      for (int b = 0; b < 8; b++) O[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it <= ntiles; it++) {
      wait_tile(it);
      if (it < ntiles && tile_bad[it]) {
        zero_bad_records(tl + (it % kBufs) * kTileBytes, phl, it * kTile, tid);
        lds_barrier();
      }
      if (it == 0) continue;
      // O += P V for tile it - 1.  PV waves issue no copies (the QK waves wait for them
      // before the barrier that starts the iteration), so these LDS reads need no vmcnt wait.
      const int par = (it - 1) & 1;
      DSA_LDS uint8_t* T = tl + ((it - 1) % kBufs) * kTileBytes;
      const i32x4 rf = *reinterpret_cast<const i32x4*>(resc_s[par]);
      if (rf[0] | rf[1] | rf[2] | rf[3]) {      // rare after the first tile (lazy rescaling)
        float al[4][4];
#pragma unroll
        for (int ht = 0; ht < 4; ht++)
#pragma unroll
          for (int i = 0; i < 4; i++) al[ht][i] = alpha_s[par][16 * ht + 4 * g + i];
#pragma unroll
        for (int ht = 0; ht < 4; ht++)
#pragma unroll
          for (int dt = 0; dt < 8; dt++)
#pragma unroll
            for (int i = 0; i < 4; i++) O[ht][dt][i] *= al[ht][i];
      }
      // per 32-key step ks of the tile:
#pragma unroll
      for (int kst = 0; kst < kKS; kst++) {
        // B operands: V of value block qw, read transposed (tr8: lane i of a 16-lane group
        // points at the key of K = 8g + i/2, i.e. key 32kst + 16(i/8) + 4g + (i/2)%4, dims
        // +8*(i%2), and gets those 8 keys of dim c16), all eight dim tiles converted up front
        const int vkey = 32 * kst + 16 * (c16 >> 3) + 4 * g + ((c16 >> 1) & 3);
        i32x2 vraw[8];
#pragma unroll
        for (int dt = 0; dt < 8; dt++)
          vraw[dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (DSA_LDS i32x2*)(T + 16 * lat_chunk(vkey, 128 * qw + 16 * dt) + 8 * (c16 & 1)));
        // A operands: P of heads 16ht + c16 for K = 8g..8g+7, i.e. keys 32kst + 4g..4g+3 and
        // 32kst + 16+4g..16+4g+3 (the order the QK waves wrote), times those keys' scale of value
        // block qw (a power of two: exact), rounded to bf16
        i32x4 praw[4];
#pragma unroll
        for (int ht = 0; ht < 4; ht++)
          praw[ht] = *reinterpret_cast<const DSA_LDS i32x4*>((const DSA_LDS uint16_t*)pl[par] + kst * kHeads * 32 +
                                                             8 * (64 * ht + lane));
        f32x4 ks[2];
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            ks[h][i] = *reinterpret_cast<const DSA_LDS float*>(
                T + 16 * rec_chunk(32 * kst + 16 * h + 4 * g + i, kRecScaleOff / 16) + 4 * qw);
        bf16x8 vv[8];
#pragma unroll
        for (int dt = 0; dt < 8; dt++) vv[dt] = fp8x8_to_bf16((uint32_t)vraw[dt][0], (uint32_t)vraw[dt][1], 1.0f);
        // head tile by head tile: the scaling of the next tile's P is independent of this tile's
        // eight MFMAs, so it issues while they run
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
          int w[4];
#pragma unroll
          for (int j = 0; j < 4; j++) {            // keys 8g + 2j, 8g + 2j + 1
            const uint32_t x = (uint32_t)praw[ht][j];
            w[j] = pack2_bf16(__uint_as_float(x << 16) * ks[j >> 1][2 * (j & 1)],
                              __uint_as_float(x & 0xFFFF0000u) * ks[j >> 1][2 * (j & 1) + 1]);
          }
          const bf16x8 pa = __builtin_bit_cast(bf16x8, i32x4{w[0], w[1], w[2], w[3]});
#pragma unroll
          for (int dt = 0; dt < 8; dt++) O[ht][dt] = mfma_bf16(pa, vv[dt], O[ht][dt]);
        }
      }
    }
    __syncthreads();                            // m_s / l_s written by the QK waves
    if (part_o == nullptr) {
      // the row's output goes through LDS (the tile buffers are idle once every PV step is
      // done): this wave's 64 heads x 128 dims as bf16 at a 272-B row pitch (the four head
      // groups of a store land in different banks), then 16-B pieces, 16 lanes to a head row,
      // instead of one 2-B global store per value.  The wave reads back only what it wrote, and
      // its LDS accesses complete in order, so no barrier is needed.  (The merging part of a cut
      // row keeps its direct stores: staged, it measured slower.)
      constexpr int kPitch = 272;
      static_assert(4 * kHeads * kPitch <= kBufs * kTileBytes, "the staging fits the tile buffers");
      DSA_LDS uint8_t* st = tl + qw * (kHeads * kPitch);
#pragma unroll
      for (int ht = 0; ht < 4; ht++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int h = 16 * ht + 4 * g + i;
          const float l = l_s[h];
          const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
          for (int dt = 0; dt < 8; dt++)
            *reinterpret_cast<DSA_LDS uint16_t*>(st + h * kPitch + 2 * (16 * dt + c16)) =
                f32_to_bf16_bits(O[ht][dt][i] * inv);
        }
#pragma unroll
      for (int kk = 0; kk < kHeads / 4; kk++) {
        const int h = 4 * kk + (lane >> 4);
        const i32x4 v = *reinterpret_cast<const DSA_LDS i32x4*>(st + h * kPitch + 16 * (lane & 15));
        *reinterpret_cast<DSA_GLOBAL i32x4*>(out + ((int64_t)r * kHeads + h) * kVal + 128 * qw + 8 * (lane & 15)) = v;
      }
    } else {
      auto store_part = [&]() {
#pragma unroll
        for (int ht = 0; ht < 4; ht++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int h = 16 * ht + 4 * g + i;
#pragma unroll
            for (int dt = 0; dt < 8; dt++)
              store_coherent(&part_o[(int64_t)h * kVal + 128 * qw + 16 * dt + c16], O[ht][dt][i]);
          }
      };
      if (tag == nullptr && gridDim.x * gridDim.y > 32) {
        store_part();
      } else if (tag == nullptr) {
        // A split's partial, read by the combine kernel after this launch (so plain stores).
        // In a grid of at most 32 work-groups (the split kernel's grid is splits x rows: one or
        // two rows in 16 splits) it is staged in the idle tile buffers like a finished row,
        // fp32, 32 heads at a time at a 528-B row pitch, and written in 16-B pieces, 32 lanes to
        // a head row: one 2048-key row 19.3 -> 17.6 us.  In grids of 256 (32 rows x 8 splits,
        // 64 x 4) the direct stores measured faster (the staged ones +1.2 us at 32 rows).
        constexpr int kPitchF = 528;
        static_assert(4 * 32 * kPitchF <= kBufs * kTileBytes, "the staging fits the tile buffers");
        DSA_LDS uint8_t* st = tl + qw * (32 * kPitchF);
#pragma unroll
        for (int half = 0; half < 2; half++) {
#pragma unroll
          for (int ht = 2 * half; ht < 2 * half + 2; ht++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int hl = 16 * (ht - 2 * half) + 4 * g + i;
#pragma unroll
              for (int dt = 0; dt < 8; dt++)
                *reinterpret_cast<DSA_LDS float*>(st + hl * kPitchF + 4 * (16 * dt + c16)) = O[ht][dt][i];
            }
#pragma unroll
          for (int kk = 0; kk < 16; kk++) {
            const int hl = 2 * kk + (lane >> 5);
            const i32x4 v = *reinterpret_cast<const DSA_LDS i32x4*>(st + hl * kPitchF + 16 * (lane & 31));
            *reinterpret_cast<DSA_GLOBAL i32x4*>(part_o + (int64_t)(32 * half + hl) * kVal + 128 * qw + 4 * (lane & 31)) = v;
          }
        }
      } else {
        __syncthreads();
        bool merge = cut_s[0] != 0;
        if (!merge) {
          store_part();
          wait_vmcnt<0>();
          __syncthreads();
          __syncthreads();
          merge = cut_s[1] != 0;
        }
        if (merge) {
          // the other part's partial, head tile by head tile (32 coherent loads each) with two
          // tiles in flight; the first is requested before the weights are ready (this side of
          // that barrier waits for LDS only, so the loads stay in flight across it)
          float ov[2][4][8];
          auto load_other = [&](int ht, float (&dst)[4][8]) {
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
              for (int dt = 0; dt < 8; dt++)
                dst[i][dt] = load_coherent(&other_o[(int64_t)(16 * ht + 4 * g + i) * kVal + 128 * qw + 16 * dt + c16]);
          };
          load_other(0, ov[0]);
          lds_barrier();                        // weights ready
          __asm__ volatile("" ::: "memory");    // (for the compiler: the weight reads stay below)
#pragma unroll
          for (int ht = 0; ht < 4; ht++) {
            if (ht + 1 < 4) load_other(ht + 1, ov[(ht + 1) & 1]);
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int h = 16 * ht + 4 * g + i;
              const float f0 = wgt_s[h][0], f1 = wgt_s[h][1], inv = wgt_s[h][2];
              DSA_GLOBAL uint16_t* orow = out + ((int64_t)r * kHeads + h) * kVal + 128 * qw + c16;
#pragma unroll
              for (int dt = 0; dt < 8; dt++)
                orow[16 * dt] = f32_to_bf16_bits((O[ht][dt][i] * f0 + ov[ht & 1][i][dt] * f1) * inv);
            }
          }
        }
      }
    }
  }
}

// One (row, split of its selection) per work-group; with one split the row is finished here,
// otherwise its partial goes to the workspace for k_mla_combine.
__global__ void __launch_bounds__(kThreads)
k_sparse_mla(const uint16_t* __restrict__ q, const int32_t* __restrict__ req, const int32_t* __restrict__ pos,
             DevPages pg, const uint8_t* __restrict__ cache, const int32_t* __restrict__ idx, int32_t k,
             int keys_per_split, float sm_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
             float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  const int r = blockIdx.y, split = blockIdx.x, nsplit = gridDim.x;
  const int j0 = split * keys_per_split;
  const int nkeys = max(0, min(keys_per_split, k - j0));
  CutRow part{};
  if (nsplit > 1) {
    part.part_o = ws_o + ((int64_t)r * nsplit + split) * kHeads * kVal;
    part.part_ml = ws_ml + ((int64_t)r * nsplit + split) * kHeads * 2;
  }
  mla_segment(q, req, pos, pg, cache, idx, k, sm_log2, r, j0, nkeys, out, lse, part);
}

// mla_segment as a call: the stream-K kernel runs several segments in a loop, and an
// inlined body there would spill registers.
__device__ __attribute__((noinline)) void mla_segment_call(const uint16_t* q, const int32_t* req, const int32_t* pos,
                                                          const DevPages& pg, const uint8_t* cache, const int32_t* idx,
                                                          int32_t k, float sm_log2, int r, int j0, int nkeys,
                                                          uint16_t* out, float* lse, float* part_o, float* part_ml,
                                                          const float* other_o, const float* other_ml,
                                                          unsigned long long* tag, unsigned long long launch) {
  mla_segment(q, req, pos, pg, cache, idx, k, sm_log2, r, j0, nkeys, out, lse,
              CutRow{part_o, part_ml, other_o, other_ml, tag, launch});
}

// Stream-K schedule for R >= gridDim.x: the R x T tiles (T = tiles per row) are cut into
// gridDim.x equal consecutive ranges, one per work-group, each covering at least one full
// row; a work-group runs its range as row segments.  A row cut between work-groups g-1 and
// g (never more than two parts) meets in slot g: the part that finishes second merges the
// other's stored partial into its own registers (mla_segment) and clears the slot's tag
// word.  Every launch so leaves its slots cleared, which keeps a captured graph correct on
// every replay (its tag is fixed at capture), and the tag is a random 64-bit value, never 0,
// so a word left in recycled memory matches it only with probability 2^-64: the workspace
// needs no initialisation.
__global__ void __launch_bounds__(kThreads)
k_sparse_mla_stream(const uint16_t* __restrict__ q, const int32_t* __restrict__ req, const int32_t* __restrict__ pos,
                    DevPages pg, const uint8_t* __restrict__ cache, const int32_t* __restrict__ idx, int32_t k,
                    int32_t R, float sm_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
                    float* __restrict__ ws_o, float* __restrict__ ws_ml, unsigned long long* __restrict__ tag,
                    unsigned long long launch) {
  const int G = gridDim.x, gi = blockIdx.x;
  const int T = (k + kTile - 1) / kTile;
  const int64_t U = (int64_t)R * T;
  const int64_t u0 = U * gi / G, u1 = U * (gi + 1) / G;
  for (int64_t u = u0; u < u1;) {
    const int r = (int)(u / T), t0 = (int)(u % T);
    const int t1 = (int)(t0 + (u1 - u) < T ? t0 + (u1 - u) : T);
    const int j0 = t0 * kTile, nkeys = min(t1 * kTile, k) - j0;
    CutRow cut{};
    if (t0 != 0 || t1 != T) {
      const int slot = t0 == 0 ? gi + 1 : gi, part = t0 == 0 ? 0 : 1;
      float* po = ws_o + (int64_t)slot * 2 * kHeads * kVal;
      float* pml = ws_ml + (int64_t)slot * 2 * kHeads * 2;
      cut = CutRow{po + (int64_t)part * kHeads * kVal, pml + part * kHeads * 2,
                   po + (int64_t)(1 - part) * kHeads * kVal, pml + (1 - part) * kHeads * 2, &tag[slot], launch};
    }
    mla_segment_call(q, req, pos, pg, cache, idx, k, sm_log2, r, j0, nkeys, out, lse, cut.part_o, cut.part_ml,
                     cut.other_o, cut.other_ml, cut.tag, cut.launch);
    u += t1 - t0;
  }
}

// Merges the splits of one row: block = (row, head), 128 threads x 4 dims.  Every split's (m, l)
// and partial O are loaded before any is used (a split count of at most kMaxSplits, predicated),
// so the loads are in flight together instead of one memory round trip per split.  At most 16
// splits: one row of 2048 keys took 20.3 us in 16 splits of 128 keys and 23.4 in 8 of 256 (split
// kernel + combine), and 29.5 in 4 of 512; rows of 32 or more never reach 8 splits.
constexpr int kMaxSplits = 16;
__global__ void __launch_bounds__(128) k_mla_combine(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                                                     int nsplit, uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int r = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  f32x2 ml[kMaxSplits];
  float4 o[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; s++) {
    if (s < nsplit) {
      ml[s] = *reinterpret_cast<const f32x2*>(ws_ml + (((int64_t)r * nsplit + s) * kHeads + h) * 2);
      o[s] = *reinterpret_cast<const float4*>(ws_o + (((int64_t)r * nsplit + s) * kHeads + h) * kVal + 4 * tid);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplits; s++)
    if (s < nsplit) M = fmaxf(M, ml[s][0]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < kMaxSplits; s++) {
    if (s < nsplit) {
      const float f = (ml[s][0] == -INFINITY) ? 0.f : exp2f(ml[s][0] - M);
      L += ml[s][1] * f;
      acc.x += o[s].x * f; acc.y += o[s].y * f; acc.z += o[s].z * f; acc.w += o[s].w * f;
    }
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

constexpr size_t kSplitPartBytes = (size_t)kHeads * (kVal + 2) * sizeof(float);   // O, m, l of one split

constexpr int kSplitGroups = 256;           // one round of work-groups: one fits a CU (LDS)
int choose_splits(int32_t R, int32_t k, size_t ws_cap = SIZE_MAX) {
  // up to one round of work-groups over the chip (a second round took c1's 32 rows from 37 to
  // 57 us, and every split adds a 128-KiB partial); at least one tile of keys per split; no
  // more splits than a workspace of ws_cap bytes holds
  int s = 1;
  while (s < kMaxSplits && (int64_t)R * 2 * s <= kSplitGroups && k / (2 * s) >= kTile &&
         (size_t)R * (2 * s) * kSplitPartBytes <= ws_cap)
    s <<= 1;
  return s;
}

constexpr int kStreamGroups = 256;              // one persistent work-group per CU (LDS-bound)

// SplitMix64 finaliser (Steele, Lea and Flood 2014): spreads a counter over 64 bits.
uint64_t mix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

// Merge tag of one stream-K launch: a per-process random salt (clock, process id, address
// layout) mixed with a launch counter; never 0, the cleared state of a slot.
unsigned long long stream_merge_tag() {
  static const uint64_t salt =
      mix64((uint64_t)std::chrono::high_resolution_clock::now().time_since_epoch().count() ^
            ((uint64_t)getpid() << 32) ^ (uint64_t)(uintptr_t)&kStreamGroups);
  static std::atomic<uint64_t> launches{0};
  const uint64_t t = mix64(salt + launches.fetch_add(1));
  return t ? t : 1;
}

}  // namespace

size_t mla_workspace_bytes(int32_t R, int32_t k) {
  if (R >= kStreamGroups)      // stream-K: two partials and a 64-bit tag per slot
    return (size_t)(kStreamGroups + 1) * (2 * kHeads * (kVal + 2) * sizeof(float) + sizeof(unsigned long long));
  const int s = choose_splits(R, k);
  if (s == 1) return 0;
  return (size_t)R * s * kSplitPartBytes;
}

hipError_t launch_sparse_mla(const uint16_t* q, RowsView rows, PagesView pg, const uint8_t* cache,
                             const int32_t* idx, int32_t k, float sm_scale, uint16_t* out, float* lse, void* ws,
                             size_t ws_bytes, bool /*prefill*/, hipStream_t s) {
  const int R = rows.n;
  if (R <= 0) return hipSuccess;
  DevPages g{pg.pt, pg.pt_stride, pg.num_reqs, pg.num_pages};
  const float sm_log2 = sm_scale * kLog2e;
  if (R >= kStreamGroups) {
    if (ws == nullptr || ws_bytes < mla_workspace_bytes(R, k)) return hipErrorInvalidValue;
    const int slots = kStreamGroups + 1;
    float* wo = (float*)ws;
    float* wml = wo + (size_t)slots * 2 * kHeads * kVal;
    unsigned long long* tag = (unsigned long long*)(wml + (size_t)slots * 2 * kHeads * 2);   // 8-B aligned
    const unsigned long long launch = stream_merge_tag();
    hipLaunchKernelGGL(k_sparse_mla_stream, dim3(kStreamGroups), dim3(kThreads), 0, s, q, rows.req, rows.pos, g,
                       cache, idx, k, R, sm_log2, out, lse, wo, wml, tag, launch);
    return hipGetLastError();
  }
  // a workspace of at least mla_workspace_bytes(R, k) gives the full split count; a smaller one
  // (the allocation-free entry point's fixed array) caps it
  const int nsplit = choose_splits(R, k, ws == nullptr ? 0 : ws_bytes);
  const int kps = (k + nsplit - 1) / nsplit;
  if (nsplit == 1) {
    hipLaunchKernelGGL(k_sparse_mla, dim3(1, R), dim3(kThreads), 0, s, q, rows.req, rows.pos, g, cache, idx, k,
                       kps, sm_log2, out, lse, nullptr, nullptr);
    return hipGetLastError();
  }
  if (ws == nullptr || ws_bytes < (size_t)R * nsplit * kSplitPartBytes) return hipErrorInvalidValue;
  float* wo = (float*)ws;
  float* wml = wo + (size_t)R * nsplit * kHeads * kVal;
  hipLaunchKernelGGL(k_sparse_mla, dim3(nsplit, R), dim3(kThreads), 0, s, q, rows.req, rows.pos, g, cache, idx, k,
                     kps, sm_log2, out, lse, wo, wml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_mla_combine, dim3(kHeads, R), dim3(128), 0, s, wo, wml, nsplit, out, lse);
  return hipGetLastError();
}

// ---------------------------------------------------------------- allocation-free variant
// Scratch of dsa_sparse_mla_decode_noalloc: a fixed array in device memory, one per GPU the
// library runs on, held until the process ends.  Its size is the stream-K schedule's need
// (two partials and a tag word for each of the 257 slots), which serves every row count of 256
// or more; fewer rows take at most as many splits as it holds.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol): kernels get the
// device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes =
    (size_t)(kStreamGroups + 1) * (2 * kSplitPartBytes + sizeof(unsigned long long));
static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];          // device address of `scratch` per device, once looked up
}  // namespace

size_t mla_static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t mla_static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));     // with device `dev` current
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

DSA_DEFINE_ERROR_ACCESSOR(take_device_errors_mla)

}  // namespace dsa
