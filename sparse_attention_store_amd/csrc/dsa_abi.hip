// dsa_abi.hip -- the C ABI of libdsa (declared in include/dsa.h): host-side argument
// validation, workspace sizing, layer rule, error reporting, and dispatch to the
// kernel launchers.  Nothing here allocates device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/dsa.h"
#include "dsa_internal.h"

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

dsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

dsa_status check_rows(const dsa_rows* r, const char* what, bool need_group) {
  if (!r) return fail(DSA_ERR_ARG, "%s: rows is NULL", what);
  if (r->n < 0) return fail(DSA_ERR_ARG, "%s: rows->n = %d < 0", what, r->n);
  if (r->n > 0 && (!r->req || !r->pos)) return fail(DSA_ERR_ARG, "%s: rows->req/pos is NULL", what);
  if (need_group) {
    if (r->group < 1) return fail(DSA_ERR_ARG, "%s: rows->group = %d < 1", what, r->group);
    if (r->n % r->group) return fail(DSA_ERR_ARG, "%s: rows->n = %d not a multiple of group %d", what, r->n, r->group);
  }
  if (r->max_pos < -1) return fail(DSA_ERR_ARG, "%s: rows->max_pos = %d", what, r->max_pos);
  return DSA_OK;
}

dsa_status check_pages(const dsa_pages* p, int32_t max_pos, const char* what) {
  if (!p) return fail(DSA_ERR_ARG, "%s: pages is NULL", what);
  if (!p->page_table) return fail(DSA_ERR_ARG, "%s: page_table is NULL", what);
  if (p->num_reqs < 1 || p->num_pages < 1) return fail(DSA_ERR_ARG, "%s: empty page pool", what);
  if (p->num_pages > (int64_t)(INT32_MAX / 64)) return fail(DSA_ERR_UNSUPPORTED, "%s: num_pages too large", what);
  if (p->pt_stride < (int64_t)(max_pos + 1 + 63) / 64)
    return fail(DSA_ERR_ARG, "%s: pt_stride %lld < pages needed for max_pos %d", what, (long long)p->pt_stride, max_pos);
  return DSA_OK;
}

dsa::RowsView view(const dsa_rows* r) { return dsa::RowsView{r->req, r->pos, r->n, r->group, r->max_pos}; }
dsa::PagesView view(const dsa_pages* p) { return dsa::PagesView{p->page_table, p->pt_stride, p->num_reqs, p->num_pages}; }

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_last_error(void) { return g_err; }

int dsa_layer_is_shared(const dsa_layer_rule* rule, int32_t layer_id) {
  if (!rule || layer_id < 0) return -1;
  if (rule->indexer_types) return layer_id < rule->n_types && rule->indexer_types[layer_id] == 'S';
  if (rule->cli_factor > 1) return layer_id % rule->cli_factor != 0;
  if (rule->topk_pattern) return layer_id < rule->n_pattern && rule->topk_pattern[layer_id] == 'S';
  if (rule->topk_freq < 1) return -1;
  int32_t v = layer_id - rule->skip_topk_offset + 1;
  return (v > 0 ? v : 0) % rule->topk_freq != 0;
}

int32_t dsa_mtp_seed_width(int32_t index_topk, int32_t index_kpool) {
  if (index_topk < 1 || index_topk > DSA_TOPK_MAX || index_kpool < 1) return -1;
  return index_topk + index_kpool - 1;
}

int dsa_mtp_carry_allowed(int32_t eagle_topk) {
  if (eagle_topk < 1) return -1;
  return eagle_topk == 1;
}

dsa_status dsa_quant_fp8(const uint16_t* x, int64_t n_blocks, uint8_t* y, float* scale, void* stream) {
  if (n_blocks < 0) return fail(DSA_ERR_ARG, "dsa_quant_fp8: n_blocks < 0");
  if (n_blocks == 0) return DSA_OK;
  if (!x || !y || !scale) return fail(DSA_ERR_ARG, "dsa_quant_fp8: NULL pointer");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(scale, 4)) return fail(DSA_ERR_ARG, "dsa_quant_fp8: misaligned pointer");
  return hip_status(dsa::launch_quant_fp8(x, n_blocks, y, scale, (hipStream_t)stream), "dsa_quant_fp8");
}

static dsa_status index_k_store_impl(const uint16_t* k, const dsa_rows* tok, const dsa_pages* pt, uint8_t* cache,
                                     double ln_eps, double rope_theta, void* stream, int fmt, const char* name) {
  dsa_status st = check_rows(tok, name, false);
  if (st) return st;
  if (!cache) return DSA_OK;              // shared layer: owns no index-K pages
  if ((st = check_pages(pt, tok->max_pos, name))) return st;
  if (tok->n > 0 && !k) return fail(DSA_ERR_ARG, "%s: k is NULL", name);
  if (!aligned(k, 16) || !aligned(cache, 16)) return fail(DSA_ERR_ARG, "%s: misaligned pointer", name);
  if (!(ln_eps >= 0.0) || !(rope_theta > 0.0)) return fail(DSA_ERR_ARG, "%s: bad eps/theta", name);
  double inv_freq[32];
  for (int i = 0; i < 32; i++) inv_freq[i] = pow(rope_theta, -(2.0 * i) / 64.0);
  const hipError_t e =
      fmt == dsa::kIdxMxfp4
          ? dsa::launch_index_k_store_mxfp4(k, view(tok), view(pt), cache, ln_eps, inv_freq, (hipStream_t)stream)
          : dsa::launch_index_k_store(k, view(tok), view(pt), cache, ln_eps, inv_freq, (hipStream_t)stream);
  return hip_status(e, name);
}

dsa_status dsa_index_k_store(const uint16_t* k, const dsa_rows* tok, const dsa_pages* pt, uint8_t* cache,
                             double ln_eps, double rope_theta, void* stream) {
  return index_k_store_impl(k, tok, pt, cache, ln_eps, rope_theta, stream, dsa::kIdxFp8, "dsa_index_k_store");
}

dsa_status dsa_index_k_store_mxfp4(const uint16_t* k, const dsa_rows* tok, const dsa_pages* pt, uint8_t* cache,
                                   double ln_eps, double rope_theta, void* stream) {
  return index_k_store_impl(k, tok, pt, cache, ln_eps, rope_theta, stream, dsa::kIdxMxfp4,
                            "dsa_index_k_store_mxfp4");
}

dsa_status dsa_latent_store(const uint16_t* kv, const dsa_rows* tok, const dsa_pages* pt, uint8_t* cache,
                            void* stream) {
  dsa_status st = check_rows(tok, "dsa_latent_store", false);
  if (st) return st;
  if ((st = check_pages(pt, tok->max_pos, "dsa_latent_store"))) return st;
  if (!cache || (tok->n > 0 && !kv)) return fail(DSA_ERR_ARG, "dsa_latent_store: NULL pointer");
  if (!aligned(kv, 16) || !aligned(cache, 16)) return fail(DSA_ERR_ARG, "dsa_latent_store: misaligned pointer");
  return hip_status(dsa::launch_latent_store(kv, view(tok), view(pt), cache, (hipStream_t)stream), "dsa_latent_store");
}

dsa_status dsa_fused_norm_rope_store(const uint16_t* kv, int64_t kv_stride, const uint16_t* gamma,
                                     const uint16_t* k_idx, const dsa_rows* tok, const dsa_pages* pt,
                                     uint8_t* latent_cache, uint8_t* index_cache, uint16_t* q_pe,
                                     int64_t q_row_stride, int64_t q_head_stride, double rms_eps, double ln_eps,
                                     double rope_theta, double index_rope_theta, void* stream) {
  const char* name = "dsa_fused_norm_rope_store";
  dsa_status st = check_rows(tok, name, false);
  if (st) return st;
  if ((st = check_pages(pt, tok->max_pos, name))) return st;
  if (!latent_cache) return fail(DSA_ERR_ARG, "%s: latent_cache is NULL", name);
  if (tok->n > 0 && !kv) return fail(DSA_ERR_ARG, "%s: kv is NULL", name);
  if (index_cache && tok->n > 0 && !k_idx) return fail(DSA_ERR_ARG, "%s: index_cache given without k_idx", name);
  if (kv_stride < DSA_LATENT_DIM || kv_stride % 8) return fail(DSA_ERR_ARG, "%s: kv_stride must be >= 576 and a multiple of 8", name);
  if (!aligned(kv, 16) || !aligned(gamma, 16) || !aligned(latent_cache, 16) ||
      (index_cache && (!aligned(k_idx, 16) || !aligned(index_cache, 16))))
    return fail(DSA_ERR_ARG, "%s: misaligned pointer", name);
  if (q_pe) {
    if (!aligned(q_pe, 16) || q_head_stride < 64 || q_head_stride % 8 || q_row_stride % 8 ||
        q_row_stride < 63 * q_head_stride + 64)
      return fail(DSA_ERR_ARG, "%s: q_pe must be 16-B aligned with head stride >= 64, rows not overlapping, "
                  "strides multiples of 8", name);
  }
  if (!(rms_eps >= 0.0) || !(ln_eps >= 0.0) || !(rope_theta > 0.0) || !(index_rope_theta > 0.0))
    return fail(DSA_ERR_ARG, "%s: bad eps/theta", name);
  dsa::FusedStoreParams f{kv, kv_stride, gamma, index_cache ? k_idx : nullptr, latent_cache, index_cache,
                          q_pe, q_row_stride, q_head_stride, rms_eps, ln_eps, {}, {}};
  for (int i = 0; i < 32; i++) {
    f.inv_freq[i] = pow(rope_theta, -(2.0 * i) / 64.0);
    f.index_inv_freq[i] = pow(index_rope_theta, -(2.0 * i) / 64.0);
  }
  return hip_status(dsa::launch_fused_norm_rope_store(f, view(tok), view(pt), (hipStream_t)stream), name);
}

int64_t dsa_logits_stride(int32_t max_pos) {
  if (max_pos < 0) return 256;
  return ((int64_t)max_pos + 1 + 255) / 256 * 256;
}

int64_t dsa_logits_rows_per_chunk(int64_t num_rows, int64_t row_bytes, int64_t budget_bytes) {
  if (num_rows * row_bytes <= budget_bytes) return 0;
  int64_t rows = budget_bytes / (row_bytes > 1 ? row_bytes : 1);
  if (rows < 1) rows = 1;
  return rows < num_rows ? rows : 0;
}

static dsa_status indexer_logits_impl(const uint8_t* q8, const float* qs, const float* w, const dsa_rows* rows,
                                      const dsa_pages* pt, const uint8_t* cache, float* logits, int64_t stride,
                                      void* stream, int fmt, const char* name) {
  dsa_status st = check_rows(rows, name, true);
  if (st) return st;
  if (!cache) return DSA_OK;              // shared layer: no indexer
  if (rows->n == 0) return DSA_OK;
  if ((st = check_pages(pt, rows->max_pos, name))) return st;
  if (!q8 || !qs || !w || !logits) return fail(DSA_ERR_ARG, "%s: NULL pointer", name);
  if (!aligned(q8, 16) || !aligned(cache, 16) || !aligned(logits, 16) || !aligned(qs, 4) || !aligned(w, 4))
    return fail(DSA_ERR_ARG, "%s: misaligned pointer", name);
  if (stride < dsa_logits_stride(rows->max_pos) || stride % 256)
    return fail(DSA_ERR_ARG, "%s: stride %lld < %lld or not a multiple of 256", name, (long long)stride,
                (long long)dsa_logits_stride(rows->max_pos));
  return hip_status(dsa::launch_indexer_logits(q8, qs, w, view(rows), view(pt), cache, logits, stride, dsa::LogitsMode{}, fmt,
                                               (hipStream_t)stream),
                    name);
}

dsa_status dsa_indexer_logits(const uint8_t* q8, const float* qs, const float* w, const dsa_rows* rows,
                              const dsa_pages* pt, const uint8_t* cache, float* logits, int64_t stride,
                              void* stream) {
  return indexer_logits_impl(q8, qs, w, rows, pt, cache, logits, stride, stream, dsa::kIdxFp8, "dsa_indexer_logits");
}

dsa_status dsa_indexer_logits_mxfp4(const uint8_t* q8, const float* qs, const float* w, const dsa_rows* rows,
                                    const dsa_pages* pt, const uint8_t* cache, float* logits, int64_t stride,
                                    void* stream) {
  return indexer_logits_impl(q8, qs, w, rows, pt, cache, logits, stride, stream, dsa::kIdxMxfp4,
                             "dsa_indexer_logits_mxfp4");
}

// Score-array size (rows x stride) up to which the fused indexer + top-k writes every score and
// takes the radix passes directly instead of the sampled-threshold filter.  Measured on the
// device: a 32-row decode batch of 8K-32K contexts (1M scores) takes 59 us directly against 68
// filtered, one 1M-context row 74 against 94; a 64-row batch at 128K (8M scores) 273 against
// 243, and 384 rows at 128K 482 against 352.
#ifndef DSA_INDEXER_TOPK_DIRECT
#define DSA_INDEXER_TOPK_DIRECT (int64_t{1} << 22)
#endif
static std::atomic<int64_t> g_topk_direct_limit{DSA_INDEXER_TOPK_DIRECT};

extern "C" int64_t dsa_set_topk_direct_limit(int64_t max_scores) {
  return max_scores < 0 ? g_topk_direct_limit.load() : g_topk_direct_limit.exchange(max_scores);
}

static dsa_status indexer_topk_impl(const uint8_t* q8, const float* qs, const float* w, const dsa_rows* rows,
                                    const dsa_pages* pt, const uint8_t* cache, float* logits, int64_t stride,
                                    int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream, int fmt,
                                    const char* name) {
  dsa_status st = check_rows(rows, name, true);
  if (st) return st;
  if (!cache) return fail(DSA_ERR_ARG, "%s: a shared layer has no indexer (reuse the full layer's idx)", name);
  if (k < 1 || k > DSA_TOPK_MAX) return fail(DSA_ERR_ARG, "%s: k = %d not in [1, %d]", name, k, DSA_TOPK_MAX);
  if (rows->n == 0) return DSA_OK;
  if ((st = check_pages(pt, rows->max_pos, name))) return st;
  if (!q8 || !qs || !w || !logits || !idx) return fail(DSA_ERR_ARG, "%s: NULL pointer", name);
  if (!aligned(q8, 16) || !aligned(cache, 16) || !aligned(logits, 16) || !aligned(qs, 4) || !aligned(w, 4) ||
      !aligned(idx, 4))
    return fail(DSA_ERR_ARG, "%s: misaligned pointer", name);
  if (stride < dsa_logits_stride(rows->max_pos) || stride % 256)
    return fail(DSA_ERR_ARG, "%s: stride %lld too small or not a multiple of 256", name, (long long)stride);
  const size_t need = dsa_topk_workspace_size(rows->n, stride, k);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu B < %zu B (256-B aligned)", name, ws_bytes, need);
  // threshold-filtered: scores of one page in sixteen set a per-row threshold; the full pass
  // keeps only the scores at or above it (the logits are not written); the exact top-k runs
  // over those candidates; rows whose candidates turn out short (fewer than k) or overflow
  // get full scores and the exact radix top-k instead, so the result never depends on the
  // sample
  hipStream_t s = (hipStream_t)stream;
  const dsa::RowsView rv = view(rows);
  const dsa::PagesView pv = view(pt);
  const int R = rows->n;
  if ((int64_t)R * stride <= g_topk_direct_limit.load(std::memory_order_relaxed)) {
    // few scores: writing them all and selecting with the radix passes costs less than the
    // filtered path's extra launches and single-work-group steps.  Rows of at most 32,768
    // scores are selected by one work-group each, straight from the plain scores.
    if (dsa::topk_single_group_rows(rows->max_pos)) {
      dsa::LogitsMode m;
      m.skip_upto = k;                 // row groups whose rows are all short need no score
      hipError_t e = dsa::launch_indexer_logits(q8, qs, w, rv, pv, cache, logits, stride, m, fmt, s);
      if (e == hipSuccess) e = dsa::launch_row_topk(logits, stride, rv, k, idx, s);
      return hip_status(e, name);
    }
    // Longer rows: every row is flagged, so the exact path's kernels (full scores with the row
    // ranges, histogram, select, final) take it; row groups whose rows are all short are still
    // not scored.
    hipError_t e = dsa::launch_topk_init(R, k, ws, s, true, true);
    if (e == hipSuccess)
      e = dsa::launch_indexer_logits(q8, qs, w, rv, pv, cache, logits, stride, dsa::topk_fallback_mode(ws, R, k, k), fmt,
                                     s);
    if (e == hipSuccess) e = dsa::launch_topk_fallback(logits, stride, rv, k, idx, ws, true, s);
    return hip_status(e, name);
  }
  hipError_t e = dsa::launch_topk_init(R, k, ws, s, false, false);
  if (e == hipSuccess)
    e = dsa::launch_indexer_logits(q8, qs, w, rv, pv, cache, logits, stride, dsa::topk_sample_mode(ws, R, k, k), fmt, s);
  if (e == hipSuccess) e = dsa::launch_topk_threshold(logits, stride, rv, k, ws, s);
  if (e == hipSuccess)
    e = dsa::launch_indexer_logits(q8, qs, w, rv, pv, cache, logits, stride, dsa::topk_filter_mode(ws, R, k, k), fmt, s);
  if (e == hipSuccess) e = dsa::launch_topk_filtered_final(rv, stride, k, idx, ws, s);
  if (e == hipSuccess)
    e = dsa::launch_indexer_logits(q8, qs, w, rv, pv, cache, logits, stride, dsa::topk_fallback_mode(ws, R, k), fmt, s);
  if (e == hipSuccess) e = dsa::launch_topk_fallback(logits, stride, rv, k, idx, ws, false, s);
  return hip_status(e, name);
}

dsa_status dsa_indexer_topk(const uint8_t* q8, const float* qs, const float* w, const dsa_rows* rows,
                            const dsa_pages* pt, const uint8_t* cache, float* logits, int64_t stride, int32_t k,
                            int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return indexer_topk_impl(q8, qs, w, rows, pt, cache, logits, stride, k, idx, ws, ws_bytes, stream, dsa::kIdxFp8,
                           "dsa_indexer_topk");
}

dsa_status dsa_indexer_topk_mxfp4(const uint8_t* q8, const float* qs, const float* w, const dsa_rows* rows,
                                  const dsa_pages* pt, const uint8_t* cache, float* logits, int64_t stride,
                                  int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return indexer_topk_impl(q8, qs, w, rows, pt, cache, logits, stride, k, idx, ws, ws_bytes, stream, dsa::kIdxMxfp4,
                           "dsa_indexer_topk_mxfp4");
}

size_t dsa_topk_workspace_size(int32_t R, int64_t stride, int32_t k) {
  if (R <= 0 || k < 1 || k > DSA_TOPK_MAX) return 0;
  return dsa::topk_workspace_bytes(R, stride, k);
}

dsa_status dsa_topk(const float* logits, int64_t stride, const dsa_rows* rows, int32_t k, int32_t* idx, void* ws,
                    size_t ws_bytes, void* stream) {
  dsa_status st = check_rows(rows, "dsa_topk", false);
  if (st) return st;
  if (k < 1 || k > DSA_TOPK_MAX) return fail(DSA_ERR_ARG, "dsa_topk: k = %d not in [1, %d]", k, DSA_TOPK_MAX);
  if (rows->n == 0) return DSA_OK;
  if (!idx || !logits) return fail(DSA_ERR_ARG, "dsa_topk: NULL pointer");
  if (!aligned(logits, 16) || !aligned(idx, 4)) return fail(DSA_ERR_ARG, "dsa_topk: misaligned pointer");
  if (stride < dsa_logits_stride(rows->max_pos) || stride % 256)
    return fail(DSA_ERR_ARG, "dsa_topk: stride %lld too small or not a multiple of 256", (long long)stride);
  const size_t need = dsa_topk_workspace_size(rows->n, stride, k);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(DSA_ERR_WORKSPACE, "dsa_topk: workspace %zu B < %zu B (256-B aligned)", ws_bytes, need);
  return hip_status(dsa::launch_topk(logits, stride, view(rows), k, idx, ws, (hipStream_t)stream), "dsa_topk");
}

size_t dsa_sparse_mla_workspace_size(int32_t R, int32_t k) {
  if (R <= 0 || k < 1 || k > DSA_TOPK_MAX) return 0;
  return dsa::mla_workspace_bytes(R, k);
}

static dsa_status mla_common(const uint16_t* q, const dsa_rows* rows, const dsa_pages* pt, const uint8_t* cache,
                             const int32_t* idx, int32_t k, float sm_scale, uint16_t* out, float* lse, void* ws,
                             size_t ws_bytes, bool prefill, void* stream, const char* what) {
  dsa_status st = check_rows(rows, what, false);
  if (st) return st;
  if (k < 1 || k > DSA_TOPK_MAX) return fail(DSA_ERR_ARG, "%s: k = %d not in [1, %d]", what, k, DSA_TOPK_MAX);
  if (rows->n == 0) return DSA_OK;
  if ((st = check_pages(pt, rows->max_pos, what))) return st;
  if (!q || !cache || !idx || !out) return fail(DSA_ERR_ARG, "%s: NULL pointer", what);
  if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(out, 16) || !aligned(idx, 4) || (lse && !aligned(lse, 4)))
    return fail(DSA_ERR_ARG, "%s: misaligned pointer", what);
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return fail(DSA_ERR_ARG, "%s: sm_scale must be > 0", what);
  const size_t need = dsa::mla_workspace_bytes(rows->n, k);
  if (need && (!ws || ws_bytes < need || !aligned(ws, 16)))
    return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu B < %zu B", what, ws_bytes, need);
  return hip_status(dsa::launch_sparse_mla(q, view(rows), view(pt), cache, idx, k, sm_scale, out, lse, ws, ws_bytes,
                                           prefill, (hipStream_t)stream),
                    what);
}

dsa_status dsa_sparse_mla_decode(const uint16_t* q, const dsa_rows* rows, const dsa_pages* pt, const uint8_t* cache,
                                 const int32_t* idx, int32_t k, float sm_scale, uint16_t* out, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  return mla_common(q, rows, pt, cache, idx, k, sm_scale, out, lse, ws, ws_bytes, false, stream,
                    "dsa_sparse_mla_decode");
}

dsa_status dsa_sparse_mla_prefill(const uint16_t* q, const dsa_rows* rows, const dsa_pages* pt, const uint8_t* cache,
                                  const int32_t* idx, int32_t k, float sm_scale, uint16_t* out, float* lse, void* ws,
                                  size_t ws_bytes, void* stream) {
  return mla_common(q, rows, pt, cache, idx, k, sm_scale, out, lse, ws, ws_bytes, true, stream,
                    "dsa_sparse_mla_prefill");
}

dsa_status dsa_sparse_mla_decode_noalloc(const uint16_t* q, const dsa_rows* rows, const dsa_pages* pt,
                                         const uint8_t* cache, const int32_t* idx, int32_t k, float sm_scale,
                                         uint16_t* out, float* lse, void* stream) {
  const char* what = "dsa_sparse_mla_decode_noalloc";
  dsa_status st = check_rows(rows, what, false);
  if (st) return st;
  if (k < 1 || k > DSA_TOPK_MAX) return fail(DSA_ERR_ARG, "%s: k = %d not in [1, %d]", what, k, DSA_TOPK_MAX);
  if (rows->n == 0) return DSA_OK;
  if ((st = check_pages(pt, rows->max_pos, what))) return st;
  if (!q || !cache || !idx || !out) return fail(DSA_ERR_ARG, "%s: NULL pointer", what);
  if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(out, 16) || !aligned(idx, 4) || (lse && !aligned(lse, 4)))
    return fail(DSA_ERR_ARG, "%s: misaligned pointer", what);
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return fail(DSA_ERR_ARG, "%s: sm_scale must be > 0", what);
  // the fixed array serves the stream-K schedule (256 rows or more) in full; fewer rows take
  // as many splits as it holds.  A need beyond it is refused before anything runs.
  const size_t cap = dsa::mla_static_scratch_bytes();
  if (rows->n >= 256 && dsa::mla_workspace_bytes(rows->n, k) > cap)
    return fail(DSA_ERR_WORKSPACE, "%s: %d rows need %zu B of scratch, the fixed array holds %zu B", what, rows->n,
                dsa::mla_workspace_bytes(rows->n, k), cap);
  void* ws = nullptr;
  hipError_t e = dsa::mla_static_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "dsa_sparse_mla_decode_noalloc: scratch address");
  return hip_status(dsa::launch_sparse_mla(q, view(rows), view(pt), cache, idx, k, sm_scale, out, lse, ws, cap, false,
                                           (hipStream_t)stream),
                    what);
}

dsa_status dsa_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(DSA_ERR_ARG, "dsa_probe_stream_read: bytes %lld not a multiple of 16", (long long)bytes);
  if (!buf || !sink) return fail(DSA_ERR_ARG, "dsa_probe_stream_read: NULL pointer");
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(DSA_ERR_ARG, "dsa_probe_stream_read: misaligned pointer");
  return hip_status(dsa::launch_probe_stream_read(buf, bytes, sink, (hipStream_t)stream), "dsa_probe_stream_read");
}

dsa_status dsa_probe_gather_records(const uint8_t* pool, int64_t pool_records, int32_t rec_bytes, const int32_t* ids,
                                    int64_t n, uint32_t* sink, void* stream) {
  if (n < 0 || pool_records < 1 || rec_bytes < 16 || rec_bytes % 16)
    return fail(DSA_ERR_ARG, "dsa_probe_gather_records: n %lld, pool_records %lld, rec_bytes %d", (long long)n,
                (long long)pool_records, rec_bytes);
  if (!pool || !ids || !sink) return fail(DSA_ERR_ARG, "dsa_probe_gather_records: NULL pointer");
  if (!aligned(pool, 16) || !aligned(ids, 4) || !aligned(sink, 4))
    return fail(DSA_ERR_ARG, "dsa_probe_gather_records: misaligned pointer");
  return hip_status(dsa::launch_probe_gather_records(pool, pool_records, rec_bytes, ids, n, sink, (hipStream_t)stream),
                    "dsa_probe_gather_records");
}

dsa_status dsa_check_device_errors(void) {
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_status(e, "dsa_check_device_errors");
  int v = dsa::take_device_errors_store() | dsa::take_device_errors_indexer() | dsa::take_device_errors_topk() |
          dsa::take_device_errors_mla();
  if (v < 0) return fail(DSA_ERR_HIP, "dsa_check_device_errors: cannot read the device flag");
  if (v) return fail(DSA_ERR_DEVICE_CHECK, "device range check failed (flags 0x%x: 1 page id, 2 index, 4 request/table column)", v);
  return DSA_OK;
}

}  // extern "C"
