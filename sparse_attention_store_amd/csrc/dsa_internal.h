// dsa_internal.h -- host-side launchers implemented by each kernel file of libdsa.
// The C ABI layer (dsa_abi.hip) validates arguments and then calls these.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct RowsView {        // device rows + host-known shape
  const int32_t* req;
  const int32_t* pos;
  int32_t n, group, max_pos;
};
struct PagesView {
  const int32_t* pt;
  int64_t pt_stride;
  int32_t num_reqs;
  int64_t num_pages;
};

hipError_t launch_quant_fp8(const uint16_t* x, int64_t n_blocks, uint8_t* y, float* scale, hipStream_t s);
hipError_t launch_index_k_store(const uint16_t* k, RowsView tok, PagesView pg, uint8_t* cache,
                                double eps, const double* inv_freq32, hipStream_t s);
hipError_t launch_latent_store(const uint16_t* kv, RowsView tok, PagesView pg, uint8_t* cache, hipStream_t s);
hipError_t launch_index_k_store_mxfp4(const uint16_t* k, RowsView tok, PagesView pg, uint8_t* cache,
                                      double eps, const double* inv_freq32, hipStream_t s);

// Fused norm + RoPE + cache writes: arguments as the C entry point validated them, plus the two
// inverse-frequency tables evaluated on the host.
struct FusedStoreParams {
  const uint16_t* kv;
  int64_t kv_stride;
  const uint16_t* gamma;
  const uint16_t* k_idx;
  uint8_t* latent_cache;
  uint8_t* index_cache;
  uint16_t* q_pe;
  int64_t q_row_stride, q_head_stride;
  double rms_eps, ln_eps;
  double inv_freq[32], index_inv_freq[32];
};
hipError_t launch_fused_norm_rope_store(const FusedStoreParams& f, RowsView tok, PagesView pg, hipStream_t s);

// Index-K cache formats: FP8 (132 B per token) and MXFP4 (68 B per token).
enum { kIdxFp8 = 0, kIdxMxfp4 = 1 };

// What a launch of the indexer-logits kernel does with the scores.
enum { kLogitsPlain = 0, kLogitsSample = 1, kLogitsFilter = 2, kLogitsFallback = 3 };
struct LogitsMode {
  int kind = kLogitsPlain;
  // plain / sample: per-row [min, max] order-preserving keys of the visible scores, merged
  // with atomicMin / atomicMax (nullable; the caller initialises it)
  uint32_t* range = nullptr;
  // row groups whose rows all have pos + 1 <= skip_upto are not scored, nothing written
  int skip_upto = 0;
  // sample: only every page_step-th page of each request is scored (and written)
  int page_step = 1;
  // filter: no logits are written; scores with key >= thr[row] are appended (key, position)
  // to the row's list fkey / fpos [R][fcap], counted in fcnt[row] (a count above fcap means
  // the list overflowed)
  const uint32_t* thr = nullptr;
  int* fcnt = nullptr;
  uint32_t* fkey = nullptr;
  int* fpos = nullptr;
  int fcap = 0;
  // filter: pages p with p % sampled_step == 0 already hold their scores in `logits` (the sample
  // pass wrote them); when it is > 1 and divides the chunk, those pages are not scored again
  int sampled_step = 0;
  // fallback: plain scores for the row groups with a flagged row only
  const int* flag = nullptr;
};
hipError_t launch_indexer_logits(const uint8_t* q8, const float* qs, const float* w, RowsView rows,
                                 PagesView pg, const uint8_t* cache, float* logits, int64_t stride,
                                 const LogitsMode& md, int fmt, hipStream_t s);

size_t topk_workspace_bytes(int32_t R, int64_t stride, int32_t k);
hipError_t launch_topk(const float* logits, int64_t stride, RowsView rows, int32_t k, int32_t* idx,
                       void* ws, hipStream_t s);
// Rows of at most 32,768 visible scores: one work-group per row selects the whole row (no
// workspace, one launch); launch_topk takes it by itself for such rows.
bool topk_single_group_rows(int64_t max_pos);
hipError_t launch_row_topk(const float* logits, int64_t stride, RowsView rows, int32_t k, int32_t* idx,
                           hipStream_t s);
// Pieces of the top-k used by the fused indexer + top-k entry (threshold-filtered):
//  init; sample scores (logits kernel, sample mode, with the row ranges); per-row threshold;
//  filtered scores (logits kernel, filter mode); exact top-k over each row's candidates,
//  flagging rows whose candidate list is short or overflowed; for the flagged rows only,
//  full scores (logits kernel, fallback mode) and the radix top-k passes.
constexpr int kTopkSampleStep = 16;        // one page in sixteen is sampled
// flag_all: every row is flagged for the radix passes (the fused call's small-array path);
// zero_hist: clear the radix histograms (the filtered path clears only those of flagged rows)
hipError_t launch_topk_init(int32_t R, int32_t k, void* ws, hipStream_t s, bool flag_all, bool zero_hist);
LogitsMode topk_sample_mode(void* ws, int32_t R, int32_t k, int32_t skip_upto);
hipError_t launch_topk_threshold(const float* logits, int64_t stride, RowsView rows, int32_t k, void* ws,
                                 hipStream_t s);
LogitsMode topk_filter_mode(void* ws, int32_t R, int32_t k, int32_t skip_upto);
hipError_t launch_topk_filtered_final(RowsView rows, int64_t stride, int32_t k, int32_t* idx, void* ws,
                                      hipStream_t s);
LogitsMode topk_fallback_mode(void* ws, int32_t R, int32_t k, int32_t skip_upto = 0);
// all_flagged: every row takes the radix passes (the direct path), so they get full grids
hipError_t launch_topk_fallback(const float* logits, int64_t stride, RowsView rows, int32_t k, int32_t* idx,
                                void* ws, bool all_flagged, hipStream_t s);

size_t mla_workspace_bytes(int32_t R, int32_t k);
// The allocation-free entry point's fixed scratch: its size, and its device address on the
// current device (looked up once per device).
size_t mla_static_scratch_bytes();
hipError_t mla_static_scratch(void** ptr);
hipError_t launch_sparse_mla(const uint16_t* q, RowsView rows, PagesView pg, const uint8_t* cache,
                             const int32_t* idx, int32_t k, float sm_scale, uint16_t* out, float* lse,
                             void* ws, size_t ws_bytes, bool prefill, hipStream_t s);

// Reference-rate probes of the benchmark (k_probe.hip).
hipError_t launch_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_gather_records(const uint8_t* pool, int64_t pool_records, int32_t rec_bytes,
                                       const int32_t* ids, int64_t n, uint32_t* sink, hipStream_t s);

// Read-and-clear of each translation unit's device error flag (synchronous).
int take_device_errors_store();
int take_device_errors_indexer();
int take_device_errors_topk();
int take_device_errors_mla();

}  // namespace dsa
