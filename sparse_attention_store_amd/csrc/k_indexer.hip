// k_indexer.hip -- lightning-indexer logits over the paged index-K cache (FP8, or the
// MXFP4 variant of the same page scheme).
//
//   logits[r][s] = sum_h w[r][h] * ReLU(q_scale[r][h] * k_scale[s] * <q8[r][h], k8[s]>)
//
// MXFP4 keys ("GLM-5.3 推理全链路(十一)", the paragraph on vLLM's two indexer-cache
// formats): 64 B of e2m1 codes and four E8M0 scales per token, one per 32 dims; the
// block scales enter the product inside the MFMA (per-lane scale bytes), so the score is
// sum_h w * ReLU(q_scale * sum_b s_b <q8, k4>_b).
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
//    g = l/16), so keys never pass through LDS.
//  * Epilogue per (row, 16-key tile): lane holds 4 heads x 1 key per head tile ->
//    8 FMAs of w'*ReLU(c) (ReLU as one v_med3); a reduce-scatter over the four 16-lane rows
//    with gfx950's v_permlane32_swap / v_permlane16_swap (3 swaps + 3 adds, no LDS) leaves
//    lane l with key l of the page, so each row's 64 logits are one coalesced 256-B store.
//  * The q operands and head weights are staged in LDS and re-read per page, so a wave
//    needs few registers and four waves share each SIMD to hide latency.
//  * The next page's keys are loaded before the current page is computed.
//  * Optionally (fused indexer + top-k) each work-group also folds the min / max of its rows'
//    visible logits, as order-preserving 32-bit keys, into a per-row range for the top-k, and
//    skips row groups whose rows all see no more keys than the top-k keeps ("GLM-5.3
//    推理全链路(十一)", section 优化二: short contexts skip the score).
#include "dsa_device.hpp"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kWaves = 4;
constexpr int kLongGroupRG = 8;         // rows per sub-group of a prefill chunk's long group
// filter mode: candidates held per row and work-group (sized so that four work-groups of
// eight rows fit a CU's LDS: 32 KiB of q + 1 KiB of weights + 8 x 104 x 8 B of candidates)
template <int RG> constexpr int kStage = RG <= 6 ? 768 / RG : 104;
// q rows are 128 B in LDS; the 16-B chunk c of row r sits at chunk c ^ (r & 7), so the 16
// lanes reading chunk g of 16 consecutive rows hit distinct banks without padding
__device__ __forceinline__ int qswz(int row, int c) { return row * kIdxDim + 16 * (c ^ (row & 7)); }

// Plain loads: the nontemporal hint was slower here, also where a row group reads each page
// once (and prefill chunks re-read pages from the last-level cache).
__device__ __forceinline__ i32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const i32x4*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

__device__ inline i32x8 load_b_operand(const uint8_t* key_row, int g) {
  i32x4 lo = ld16(key_row + 16 * g);
  i32x4 hi = ld16(key_row + 64 + 16 * g);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// max(x, 0) as one v_med3_f32 (fmaxf would add a NaN-quieting max per input in IEEE mode;
// MFMA outputs here are finite).
__device__ inline float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.402823466e38f); }

__device__ inline f32x4 mfma_fp8(const i32x8& a, const i32x8& b) {
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// One page of keys in registers, as MFMA B operands of its four 16-key tiles.
template <int FMT> struct PageRegs;
template <> struct PageRegs<kIdxFp8> {
  i32x8 b[4];   // FP8: bytes [16g,16g+16) and [64+16g,64+16g+16) of key 16t + l%16
  float ks;     // scale of key `lane` of the page, applied after the head reduction
};
template <> struct PageRegs<kIdxMxfp4> {
  i32x4 b[4];   // MXFP4: dims [32g, 32g+32) of key 16t + l%16 (16 packed bytes)
  int sb;       // byte t: the E8M0 scale of that 32-dim block (the MFMA's per-lane scale)
};
template <int FMT> constexpr int kPageBytes = FMT == kIdxFp8 ? kIdxPageBytes : kMx4PageBytes;

__device__ inline void load_page(PageRegs<kIdxFp8>& P, const uint8_t* page, int lane) {
  const int g = lane >> 4, k16 = lane & 15;
#pragma unroll
  for (int t = 0; t < 4; t++) P.b[t] = load_b_operand(page + (16 * t + k16) * kIdxDim, g);
  P.ks = __uint_as_float(ld4(page + kIdxScaleOff + 4 * lane));
}
__device__ inline void load_page(PageRegs<kIdxMxfp4>& P, const uint8_t* page, int lane) {
  const int g = lane >> 4, k16 = lane & 15;
  uint32_t sw[4];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    P.b[t] = ld16(page + (16 * t + k16) * kMx4KeyBytes + 16 * g);
    sw[t] = ld4(page + kMx4ScaleOff + 4 * (16 * t + k16));
  }
  uint32_t sb = 0;
#pragma unroll
  for (int t = 0; t < 4; t++) sb |= ((sw[t] >> (8 * g)) & 0xFFu) << (8 * t);
  P.sb = (int)sb;
}
__device__ inline float key_scale(const PageRegs<kIdxFp8>& P) { return P.ks; }
__device__ inline float key_scale(const PageRegs<kIdxMxfp4>&) { return 1.0f; }   // inside the MFMA

// A (16 heads x 128 dims of q, FP8, unit scale: q's own scale is folded into w) times the
// keys of tile T.  The MXFP4 product is the block-scaled MFMA with an e2m1 B operand: each
// lane's 32 codes take that lane's scale byte (byte T of P.sb, chosen by the op_sel).  On
// this MFMA the FP8 operand's K order is bytes [16g,16g+16) -> K 16g.., [16..32) -> 64+16g..
// and the FP4 operand's is dims 32g.. in nibble order, so both see key dim k at K = k.
template <int T>
__device__ inline f32x4 mfma_tile(const i32x8& a, const PageRegs<kIdxFp8>& P) { return mfma_fp8(a, P.b[T]); }
template <int T>
__device__ inline f32x4 mfma_tile(const i32x8& a, const PageRegs<kIdxMxfp4>& P) {
  const i32x8 b = {P.b[T][0], P.b[T][1], P.b[T][2], P.b[T][3], 0, 0, 0, 0};
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 127, T, P.sb);
}

// The VALU reads the two results of a tile right after their MFMAs.  For the block-scaled
// FP8 x FP4 product a probe on this device read a scaled result too early after the 10-11 wait
// states the compiler puts in for an 8-pass MFMA, so there the wait is explicit: 20 wait states
// after the second MFMA (what a 16-pass MFMA needs), tied to both results' registers so that
// every read of them comes after it.  The unscaled FP8 product needs no more than the
// compiler's wait.
template <int FMT>
__device__ inline void mfma_results_ready(f32x4& c0, f32x4& c1) {
  if (FMT == kIdxMxfp4) __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(c0), "+v"(c1));
}

// tile index as a run-time value; the unrolled callers make it a constant
template <int FMT>
__device__ inline f32x4 mfma_tile_at(int t, const i32x8& a, const PageRegs<FMT>& P) {
  switch (t) {
    case 0: return mfma_tile<0>(a, P);
    case 1: return mfma_tile<1>(a, P);
    case 2: return mfma_tile<2>(a, P);
    default: return mfma_tile<3>(a, P);
  }
}

template <int RG, int KIND, int FMT>
__global__ void __launch_bounds__(256, 4)
k_logits_decode(const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
                const int32_t* __restrict__ req, const int32_t* __restrict__ pos, DevPages pg,
                const uint8_t* __restrict__ cache, float* __restrict__ logits, int64_t stride,
                int chunk_pages, LogitsMode md) {
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[RG * kIdxHeads * kIdxDim];
  __shared__ __attribute__((aligned(16))) float w_lds[RG * kIdxHeads];
  // filter mode: candidates of this work-group, per row, before one append per row
  constexpr int kStage = dsa::kStage<RG>;     // per row
  __shared__ uint32_t st_key[KIND == kLogitsFilter ? RG : 1][KIND == kLogitsFilter ? kStage : 1];
  __shared__ int st_pos[KIND == kLogitsFilter ? RG : 1][KIND == kLogitsFilter ? kStage : 1];
  __shared__ int st_n[RG];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, k16 = lane & 15;
  const int64_t row0 = (int64_t)blockIdx.y * RG;
  // only the sample and fallback passes of the fused top-k ask for row ranges
  constexpr bool kRange = KIND == kLogitsSample || KIND == kLogitsFallback;
  // pages are numbered in steps of page_step (the sample mode scores every page_step-th page)
  const int step = KIND == kLogitsSample ? md.page_step : 1;
  const int64_t pg0 = (int64_t)blockIdx.x * chunk_pages;          // in units of `step` pages
  const int64_t col_end = min((pg0 + chunk_pages) * 64, stride);

  int prow[RG];
  int pmax = -1;
  bool flagged = false;
#pragma unroll
  for (int r = 0; r < RG; r++) {
    prow[r] = pos[row0 + r];
    pmax = max(pmax, prow[r]);
    if (KIND == kLogitsFallback) flagged |= md.flag[row0 + r] != 0;
  }
  // every row of the group sees at most skip_upto keys: its top-k is all of them and needs
  // no score (the fused indexer + top-k passes k here; nothing of the group is written).  In
  // the plain pass (skip_upto 0) a group of padded rows (pos < 0) goes on to the -inf fill.
  if (md.skip_upto > 0 && pmax + 1 <= md.skip_upto) return;
  if (KIND == kLogitsFallback && !flagged) return;     // no row of the group needs the full scores
  // the rows' thresholds as floats: for a finite score v, key(v) >= thr exactly when
  // v >= thr_f, except that -0.0 also passes a threshold of +0.0 (a superset of the candidates;
  // the exact selection over them is unchanged).  Thresholds at or below key(-inf) pass every
  // score; those above key(+inf) decode to NaN, which no score reaches.
  float thr_f[RG];
  if (KIND == kLogitsFilter) {
#pragma unroll
    for (int r = 0; r < RG; r++) {
      const uint32_t t = md.thr[row0 + r];
      const uint32_t f = t <= 0x007FFFFFu ? 0xFF800000u : ((t & 0x80000000u) ? (t & 0x7FFFFFFFu) : ~t);
      thr_f[r] = __int_as_float(__builtin_amdgcn_readfirstlane((int)f));     // wave-uniform: scalar
    }
    if (tid < RG) st_n[tid] = 0;
  }
  const int32_t rq = req[row0];
  // pages with a visible key (never past the logits row), in units of `step`
  const int64_t vis_pages = min((int64_t)(pmax >> 6) + 1, stride / 64);
  const int64_t pend = min(pg0 + chunk_pages, (vis_pages + step - 1) / step);

  if (pg0 < pend) {
    // ids of this wave's pages pg0 + wave + kWaves * i, lane i holding the i-th (a chunk has
    // at most 128 pages, so at most 32 per wave); loaded once, ahead of the q staging, so the
    // page loop has no dependent page-table load
    // The filter pass skips the pages the sample pass scored (one in S, their scores are in
    // `logits`, bit-identical to a rescoring) when S divides the chunk: page j of the scored
    // sequence is then the j-th page of [pg0, pend) that is not a multiple of S.
    constexpr int S = kTopkSampleStep;
    const bool skip = KIND == kLogitsFilter && md.sampled_step == S && chunk_pages % S == 0;
    const int nchunk = (int)(pend - pg0);                                  // <= chunk_pages <= 128
    const int nsamp = skip ? (nchunk + S - 1) / S : 0;
    auto scored_page = [&](int j) -> int64_t { return pg0 + (skip ? (j / (S - 1)) * S + 1 + j % (S - 1) : j); };
    const int nscored = nchunk - nsamp;
    const int nw = nscored > wave ? (nscored - wave + kWaves - 1) / kWaves : 0;
    // stage q (RG x 32 heads x 128 B, 16-B chunks swizzled by row) and w*q_scale in LDS; the
    // MFMA A operands and head weights are re-read from LDS for every page, which keeps the
    // register file small enough for four waves per SIMD.  Every load of the staging (RG
    // chunks of q per thread, one weight and one scale) and the page-table loads are issued
    // before any of them is used, so the prologue waits one memory round trip, not one per
    // chunk.
    constexpr int kQPer = RG * kIdxHeads * kIdxDim / 16 / 256;
    static_assert(kQPer * 256 * 16 == RG * kIdxHeads * kIdxDim && RG * kIdxHeads <= 256, "staging shares");
    i32x4 qv[kQPer];
#pragma unroll
    for (int u = 0; u < kQPer; u++) qv[u] = reinterpret_cast<const i32x4*>(q8 + row0 * kIdxHeads * kIdxDim)[tid + 256 * u];
    float wq = 0.f, sq = 0.f;
    if (tid < RG * kIdxHeads) {
      wq = w[row0 * kIdxHeads + tid];
      sq = qs[row0 * kIdxHeads + tid];
    }
    int my_id = -1;
    if (lane < nw) my_id = (int)page_of(pg, rq, scored_page(wave + kWaves * lane) * step * 64);
#pragma unroll
    for (int u = 0; u < kQPer; u++) {
      const int i = tid + 256 * u, row = i >> 3, c = i & 7;
      *reinterpret_cast<i32x4*>(q_lds + qswz(row, c)) = qv[u];
    }
    if (tid < RG * kIdxHeads) w_lds[tid] = wq * sq;
    __syncthreads();

    // running min / max of the order-preserving key of this lane's visible logits over the
    // group's rows (only kept when the fused top-k asked for row ranges; a range covering a
    // row's keys is all the radix select needs, so the group's union serves each of its rows)
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
    auto key_of = [](float x) {
      const uint32_t u = __float_as_uint(x);
      return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    };
    // filter mode: one kept (key, position) of row r into the work-group's stage
    auto stage = [&](int r, int s, uint32_t key) {
      const int sl = atomicAdd(&st_n[r], 1);
      if (sl < kStage) {
        st_key[r][sl] = key;
        st_pos[r][sl] = s;
      } else {
        // stage full: straight to the row's list (a count past fcap still flags the row)
        const int gi = atomicAdd(&md.fcnt[row0 + r], 1);
        if (gi < md.fcap) {
          md.fkey[(row0 + r) * md.fcap + gi] = key;
          md.fpos[(row0 + r) * md.fcap + gi] = s;
        }
      }
    };
    // score one page (held in registers) for all RG rows
    auto process = [&](const PageRegs<FMT>& P, int64_t vi, int64_t pid) {
      // keep the per-page LDS reads of q / w inside the loop (hoisting them would pin all
      // rows' operands in registers again)
      __asm__ volatile("" ::: "memory");
      const int s = (int)(vi * step * 64) + lane;          // positions fit in int32
#pragma unroll
      for (int r = 0; r < RG; r++) {
        i32x8 A[2];
        float4 wr[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
          const int qr = r * kIdxHeads + 16 * t + k16;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(q_lds + qswz(qr, g));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(q_lds + qswz(qr, 4 + g));
          A[t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          wr[t] = *reinterpret_cast<const float4*>(w_lds + r * kIdxHeads + 16 * t + 4 * g);
        }
        float part[4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
          f32x4 c0 = mfma_tile_at(t, A[0], P);
          f32x4 c1 = mfma_tile_at(t, A[1], P);
          mfma_results_ready<FMT>(c0, c1);
          float acc = wr[0].x * relu(c0[0]);
          acc = fmaf(wr[0].y, relu(c0[1]), acc);
          acc = fmaf(wr[0].z, relu(c0[2]), acc);
          acc = fmaf(wr[0].w, relu(c0[3]), acc);
          acc = fmaf(wr[1].x, relu(c1[0]), acc);
          acc = fmaf(wr[1].y, relu(c1[1]), acc);
          acc = fmaf(wr[1].z, relu(c1[2]), acc);
          acc = fmaf(wr[1].w, relu(c1[3]), acc);
          part[t] = acc;
        }
        // reduce-scatter over the four 16-lane rows g with VALU lane swaps: lane row g ends
        // with the head sum of tile g, i.e. key `lane` of the page
        const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
        const float keep0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);   // rows 0,1: tile 0; rows 2,3: tile 2
        const float keep1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);   // rows 0,1: tile 1; rows 2,3: tile 3
        const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(keep0), __float_as_uint(keep1), false, false);
        const float mine = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
        const bool vis = pid >= 0 && s <= prow[r];        // pid < 0: a bad page id (flagged)
        const float v = vis ? mine * key_scale(P) : -INFINITY;
        if (KIND == kLogitsFilter) {
          // keep the scores at or above the row's threshold (rare: a few per cent)
          if (vis && v >= thr_f[r]) stage(r, s, key_of(v));
        } else {
          // nontemporal: 5% off the c2 logits pass, and the top-k that reads them back is no slower
          __builtin_nontemporal_store(v, &logits[(row0 + r) * stride + s]);
          if (kRange && md.range != nullptr && s <= prow[r]) {
            const uint32_t key = key_of(v);
            kmn = min(kmn, key);
            kmx = max(kmx, key);
          }
        }
      }
    };
    // two register buffers in ping-pong: the next page loads while this one is scored.  The
    // loop takes pages in pairs and leaves only at its end, with the same loads in flight on
    // every path (past the last page the last one is loaded again; a bad id loads page 0 and
    // scores as invisible), so the waits for a page's operands keep the next page in flight.
    // this wave's first sampled page (filter mode): its stored scores are requested before the
    // page loop, so they arrive with the first page instead of costing a round trip per row after
    // the loop (the other sampled pages, when a wave has more than one, follow the loop; groups of
    // eight rows load after the loop as well, their registers being full)
    const bool samp0 = RG <= 6 && wave < nsamp;
    const int s_samp0 = (int)((pg0 + (int64_t)wave * S) * 64) + lane;
    float vs0[RG];
    if (samp0) {
#pragma unroll
      for (int r = 0; r < RG; r++) vs0[r] = logits[(row0 + r) * stride + s_samp0];
    }
    PageRegs<FMT> pa, pb;
    auto page_addr = [&](int id) { return cache + (int64_t)(id < 0 ? 0 : id) * kPageBytes<FMT>; };
    auto page_id = [&](int i) { return __builtin_amdgcn_readlane(my_id, min(i, nw - 1)); };
    auto page_vi = [&](int i) { return scored_page(wave + kWaves * i); };
    if (nw > 0) {
      int ida = page_id(0);
      load_page(pa, page_addr(ida), lane);
      int i = 0;
      // The filter pass runs its work-groups in at most two rounds (four resident per CU).
      // Issue arbitration favours the oldest waves, so the four groups on a CU used to finish
      // staggered (page loops of 57-113 us for the same 60 pages in the first round) and the
      // last second-round groups ran alone at the end: a 39-us tail on a 214-us pass.  A wave's
      // priority now falls in four steps as it gets through its pages, so the groups started
      // together finish together (span 205 us; the fused call at c2 -1.6%).  Passes of more
      // rounds balance by dispatch and keep the default priority.
      const bool fair = KIND == kLogitsFilter && gridDim.x * gridDim.y <= 2 * 4 * 256;
      int level = 3;
      if (fair) __builtin_amdgcn_s_setprio(3);
      for (; i + 1 < nw; i += 2) {
        if (fair) {
          const int want = 3 - (4 * i) / nw;
          if (want != level) {
            level = want;
            if (want == 2) __builtin_amdgcn_s_setprio(2);
            else if (want == 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
          }
        }
        const int idb = page_id(i + 1);
        load_page(pb, page_addr(idb), lane);
        process(pa, page_vi(i), ida);
        ida = page_id(i + 2);
        load_page(pa, page_addr(ida), lane);
        process(pb, page_vi(i + 1), idb);
      }
      if (i < nw) process(pa, page_vi(i), ida);     // an odd page count: the last page
      if (fair) __builtin_amdgcn_s_setprio(0);
    }
    // the sampled pages of the chunk: their stored scores against the threshold (a page of a
    // bad id holds -inf: a visible key's score is finite, and the scored path never stages those,
    // whatever the threshold)
    if (samp0) {
#pragma unroll
      for (int r = 0; r < RG; r++)
        if (s_samp0 <= prow[r] && vs0[r] > -INFINITY && vs0[r] >= thr_f[r]) stage(r, s_samp0, key_of(vs0[r]));
    }
    for (int m = RG <= 6 ? wave + kWaves : wave; m < nsamp; m += kWaves) {
      const int s = (int)((pg0 + (int64_t)m * S) * 64) + lane;
      float vs[RG];
#pragma unroll
      for (int r = 0; r < RG; r++) vs[r] = logits[(row0 + r) * stride + s];
#pragma unroll
      for (int r = 0; r < RG; r++)
        if (s <= prow[r] && vs[r] > -INFINITY && vs[r] >= thr_f[r]) stage(r, s, key_of(vs[r]));
    }
    if (kRange && md.range != nullptr) {
      __shared__ uint32_t red[kWaves][2];
      uint32_t mn = kmn, mx = kmx;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
      }
      if (lane == 0) { red[wave][0] = mn; red[wave][1] = mx; }
      __syncthreads();
      if (tid < RG) {
        for (int w2 = 0; w2 < kWaves; w2++) { mn = min(mn, red[w2][0]); mx = max(mx, red[w2][1]); }
        if (mn <= mx) {
          atomicMin(&md.range[2 * (row0 + tid)], mn);
          atomicMax(&md.range[2 * (row0 + tid) + 1], mx);
        }
      }
    }
    if (KIND == kLogitsFilter) {
      // one append per row: reserve room in the row's candidate list, then copy
      __shared__ int st_base[RG];
      __syncthreads();
      if (tid < RG) {
        const int n = st_n[tid];
        // only the staged entries: the overflow went to the list directly
        const int ns = min(n, kStage);
        st_base[tid] = ns == 0 ? 0 : atomicAdd(&md.fcnt[row0 + tid], ns);
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < RG; r++) {
        const int n = min(st_n[r], kStage), base = st_base[r];
        for (int i = tid; i < n; i += 256)
          if (base + i < md.fcap) {
            md.fkey[(row0 + r) * md.fcap + base + i] = st_key[r][i];
            md.fpos[(row0 + r) * md.fcap + base + i] = st_pos[r][i];
          }
      }
    }
  }
  if (KIND == kLogitsPlain || KIND == kLogitsFallback) {
    // columns of this chunk past the group's last visible page
    const int64_t fill0 = max(pend, pg0) * 64;
    for (int64_t c = fill0 + tid; c < col_end; c += 256)
#pragma unroll
      for (int r = 0; r < RG; r++) logits[(row0 + r) * stride + c] = -INFINITY;
  }
}

template <int RG, int KIND, int FMT>
hipError_t launch_rg(const uint8_t* q8, const float* qs, const float* w, RowsView rows, DevPages g,
                     const uint8_t* cache, float* logits, int64_t stride, const LogitsMode& md, hipStream_t s) {
  const int64_t n_groups = rows.n / RG;
  const int step = KIND == kLogitsSample ? md.page_step : 1;
  const int64_t total_pages = (stride / 64 + step - 1) / step;      // in units of `step` pages
  // enough work-groups to cover the chip (each page is one wave-iteration); the sampling pass
  // reads few pages, so it stops at one round of resident work-groups to amortise the q staging,
  // and so does the fused call's fallback, whose work-groups mostly find no flagged row and exit.
  // A few long requests take fewer, longer work-groups, 512 per request (with >= 2 GB of cache
  // copies rotated so that HBM serves every page: one 1M-context row 34.0 -> 29.4 us, two
  // 512K-context rows 34.2 -> 30.6 us).  Four or more requests keep more chunks, which also
  // spreads requests of uneven length (a 32-request batch of 8K-32K is slower with fewer).
  int64_t want = KIND == kLogitsSample || KIND == kLogitsFallback ? 1024 : 2048;
  if (n_groups < 4) want = min(want, 512 * n_groups);
  // 32 pages per work-group; the filter pass, which writes no logits, takes up to 128 as its
  // stage allows (fewer work-groups amortise the q staging: 64 took 3% off the c2 filter pass
  // and 128 1.6% off the 1M prefill indexer, while the logits-writing pass was 1% slower with 64)
  int chunk = KIND == kLogitsFallback ? 128 : 32;
  if (KIND == kLogitsFilter) {
    // a row keeps up to fcap of its visible keys: a work-group's share, chunk * 64 * fcap /
    // visible, should fit its per-row stage
    const int64_t lim = (int64_t)kStage<RG> * ((int64_t)rows.max_pos + 1) / ((int64_t)md.fcap * 64);
    chunk = lim >= 128 ? 128 : lim >= 64 ? 64 : lim >= 32 ? 32 : lim >= 16 ? 16 : lim >= 8 ? 8 : 4;
  }
  while (chunk > 4 && n_groups * ((total_pages + chunk - 1) / chunk) < want) chunk >>= 1;
  const int64_t nchunks = (total_pages + chunk - 1) / chunk;
  hipLaunchKernelGGL((k_logits_decode<RG, KIND, FMT>), dim3((unsigned)nchunks, (unsigned)n_groups), dim3(256), 0, s, q8, qs,
                     w, rows.req, rows.pos, g, cache, logits, stride, chunk, md);
  return hipGetLastError();
}

template <int RG, int FMT>
hipError_t launch_kind(const uint8_t* q8, const float* qs, const float* w, RowsView rows, DevPages g,
                       const uint8_t* cache, float* logits, int64_t stride, const LogitsMode& md, hipStream_t s) {
  switch (md.kind) {
    case kLogitsSample: return launch_rg<RG, kLogitsSample, FMT>(q8, qs, w, rows, g, cache, logits, stride, md, s);
    case kLogitsFilter: return launch_rg<RG, kLogitsFilter, FMT>(q8, qs, w, rows, g, cache, logits, stride, md, s);
    case kLogitsFallback: return launch_rg<RG, kLogitsFallback, FMT>(q8, qs, w, rows, g, cache, logits, stride, md, s);
    default: return launch_rg<RG, kLogitsPlain, FMT>(q8, qs, w, rows, g, cache, logits, stride, md, s);
  }
}

// The same mode with its per-row arrays advanced by `r0` rows.
LogitsMode shift_rows(const LogitsMode& md, int64_t r0) {
  LogitsMode m = md;
  if (m.range) m.range += 2 * r0;
  if (m.thr) m.thr += r0;
  if (m.fcnt) m.fcnt += r0;
  if (m.fkey) m.fkey += r0 * m.fcap;
  if (m.fpos) m.fpos += r0 * m.fcap;
  if (m.flag) m.flag += r0;
  return m;
}

template <int FMT>
hipError_t launch_fmt(const uint8_t* q8, const float* qs, const float* w, RowsView rows, PagesView pg,
                      const uint8_t* cache, float* logits, int64_t stride, const LogitsMode& md, hipStream_t s) {
  if (rows.n <= 0) return hipSuccess;
  DevPages g{pg.pt, pg.pt_stride, pg.num_reqs, pg.num_pages};
  // one request's long group (a prefill chunk): its first 8 * floor(n / 8) rows go in
  // sub-groups of eight (each page read once per eight rows) and the last one to seven rows in
  // a second launch; sub-groups of the largest divisor of n could shrink to one row, which
  // re-reads every key once per row
  if (rows.group == rows.n && rows.n > kLongGroupRG) {
    const int32_t head = rows.n - rows.n % kLongGroupRG;
    RowsView a = rows, b = rows;
    a.n = a.group = head;
    b.req += head;
    b.pos += head;
    b.n = b.group = rows.n - head;
    const hipError_t e = launch_kind<kLongGroupRG, FMT>(q8, qs, w, a, g, cache, logits, stride, md, s);
    if (e != hipSuccess || b.n == 0) return e;
    return launch_fmt<FMT>(q8 + (int64_t)head * kIdxHeads * kIdxDim, qs + (int64_t)head * kIdxHeads,
                           w + (int64_t)head * kIdxHeads, b, pg, cache, logits + (int64_t)head * stride, stride,
                           shift_rows(md, head), s);
  }
  // rows of a group are processed in sub-groups of the largest divisor of `group` <= 6
  // (the q operands of six rows fill the register file without spilling)
  int rg = 1;
  for (int d = 6; d >= 1; d--)
    if (rows.group % d == 0) { rg = d; break; }
  switch (rg) {
    case 6: return launch_kind<6, FMT>(q8, qs, w, rows, g, cache, logits, stride, md, s);
    case 5: return launch_kind<5, FMT>(q8, qs, w, rows, g, cache, logits, stride, md, s);
    case 4: return launch_kind<4, FMT>(q8, qs, w, rows, g, cache, logits, stride, md, s);
    case 3: return launch_kind<3, FMT>(q8, qs, w, rows, g, cache, logits, stride, md, s);
    case 2: return launch_kind<2, FMT>(q8, qs, w, rows, g, cache, logits, stride, md, s);
    default: return launch_kind<1, FMT>(q8, qs, w, rows, g, cache, logits, stride, md, s);
  }
}

}  // namespace

hipError_t launch_indexer_logits(const uint8_t* q8, const float* qs, const float* w, RowsView rows, PagesView pg,
                                 const uint8_t* cache, float* logits, int64_t stride, const LogitsMode& md, int fmt,
                                 hipStream_t s) {
  return fmt == kIdxMxfp4 ? launch_fmt<kIdxMxfp4>(q8, qs, w, rows, pg, cache, logits, stride, md, s)
                          : launch_fmt<kIdxFp8>(q8, qs, w, rows, pg, cache, logits, stride, md, s);
}

DSA_DEFINE_ERROR_ACCESSOR(take_device_errors_indexer)

}  // namespace dsa
