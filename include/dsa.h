/*
 * dsa.h -- C ABI of libdsa: the hot path of one DeepSeek-V3.2 / GLM-5.3-style
 * DSA attention layer on one AMD Instinct MI355X (gfx950).
 *
 * Pages the operations follow (cited by title and section):
 *   [IDXC] "GLM-5.3 推理全链路(十一): 索引器缓存的跨层读写" (pinghaoyang.com.cn)
 *   [REQ]  "GLM-5.3 推理全链路(一): 一个请求在 SGLang 里经过哪些算子、哪些通信"
 *   [VLLM] "vLLM 推理链路概览: 以 GLM-5.2 为例" (xpengzhao.github.io)
 *
 * Conventions (apply to every call):
 *  - Plain C types only.  Pointers marked "device" point to GPU memory; everything
 *    else is host memory.  Every buffer is owned by the caller; no call allocates
 *    or frees device memory, and no call keeps a pointer after it returns.
 *  - Every compute call is asynchronous and ordered on `stream` (a hipStream_t
 *    passed as void*; NULL = the default stream).  No call synchronises.
 *  - Calls return dsa_status.  Argument errors are detected on the host before any
 *    launch, and nothing is written then.  dsa_last_error() describes the last
 *    failure of the calling thread.
 *  - Fixed shapes (DSA_ERR_UNSUPPORTED if a caller asks for others): page size 64,
 *    indexer head dim 128 with 32 indexer heads, MLA with 64 heads over a 576-dim
 *    latent (512 latent + 64 rope) and a 512-dim value, top-k width <= 2048.
 *  - Device data that the host cannot validate (page ids, positions, selected
 *    indices) is range-checked inside the kernels: an out-of-range page id or
 *    index is never dereferenced; the offending element is skipped and a device
 *    error flag is raised, reported by dsa_check_device_errors().
 *
 * Byte layouts:
 *  - Index-K cache, one per full layer: uint8 [num_pages][8448].  A page holds 64
 *    tokens: [64 x 128 B fp8 E4M3 keys, token-major][64 x fp32 ue8m0 scale]
 *    ([IDXC] §索引器缓存里存的是什么: 128 B + one 4-B scale per 128 dims per token,
 *    64 x 132 = 8448 B per page; the keys-then-scales split inside the page is this
 *    library's reading, so a 64-token key block is one contiguous 8 KiB run).
 *  - Latent (MLA KV) cache, one per layer: uint8 [num_pages][41984], 64 records of
 *    656 B: [512 B fp8 latent (4 blocks of 128)][4 x fp32 ue8m0 scale][64 x bf16 rope]
 *    ([IDXC] §主 KV 缓存里存的是什么: 576 dims, fp8 with 4-B scales per 128 dims,
 *    656 B/token/layer; the rope tail stays bf16 in this reading).
 *  - Page table: int32 [num_reqs][pt_stride]; logical position p of request b is
 *    page page_table[b][p / 64], slot p % 64.  One table serves both caches and all
 *    layers ([REQ] §第九阶段, 细节二: both pools share page ids).
 *  - FP8 is OCP E4M3 (e4m3fn), round-to-nearest-even, saturating at +-448; a ue8m0
 *    scale is the smallest power of two s with max|x| <= 448 s (1 for an all-zero
 *    block), stored as fp32.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1
#define DSA_PAGE_SIZE 64
#define DSA_INDEX_DIM 128
#define DSA_INDEX_HEADS 32
#define DSA_INDEX_PAGE_BYTES 8448
#define DSA_INDEX_MXFP4_PAGE_BYTES 4352
#define DSA_MLA_HEADS 64
#define DSA_LATENT_DIM 576
#define DSA_VALUE_DIM 512
#define DSA_LATENT_RECORD_BYTES 656
#define DSA_LATENT_PAGE_BYTES 41984
#define DSA_TOPK_MAX 2048

typedef enum {
  DSA_OK = 0,
  DSA_ERR_ARG = 1,          /* null / misaligned pointer, bad size or stride */
  DSA_ERR_UNSUPPORTED = 2,  /* a fixed dimension was asked to change */
  DSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than *_workspace_size() */
  DSA_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed */
  DSA_ERR_DEVICE_CHECK = 5  /* a kernel met an out-of-range page id / index */
} dsa_status;

/* Library version of this header (DSA_ABI_VERSION). */
int dsa_abi_version(void);

/* Message for the calling thread's last failed call; valid until its next call. */
const char* dsa_last_error(void);

/* Page table shared by the index-K and latent caches (device). */
typedef struct {
  const int32_t* page_table;  /* device [num_reqs][pt_stride] */
  int64_t pt_stride;          /* entries per request row, >= ceil((max_pos+1)/64) */
  int32_t num_reqs;
  int64_t num_pages;          /* pages in each cache pool; page ids must be < num_pages */
} dsa_pages;

/* Query rows or new tokens: request id and absolute position of each (device).
 * pos < 0 marks a padded row: it is stored nowhere and selects nothing.
 * `group` consecutive rows belong to the same request (1 for plain decode, the
 * number of draft tokens for speculative verify, all rows for one prefill chunk);
 * rows of a group share one pass over the request's index-K pages.  n must be a
 * multiple of group.  max_pos is a host-known upper bound of pos (it sizes grids). */
typedef struct {
  const int32_t* req;   /* device [n] */
  const int32_t* pos;   /* device [n] */
  int32_t n;
  int32_t group;
  int32_t max_pos;
} dsa_rows;

/* Full/shared layer rule ([IDXC] §配置里的 78 个字符).  Precedence: an explicit
 * per-layer list (indexer_types, 'F'/'S'; layers beyond it are full), else
 * cli_factor > 1 (full iff layer % cli_factor == 0), else an explicit pattern
 * ('F'/'S'; beyond it full), else shared iff max(layer - skip_topk_offset + 1, 0)
 * % topk_freq != 0.  GLM-5.3: topk_freq 4, skip_topk_offset 3 -> 21 full layers
 * {0,1,2,6,...,74} and 57 shared of 78.  Strings are host memory, nullable. */
typedef struct {
  const char* indexer_types;
  int32_t n_types;
  int32_t cli_factor;
  const char* topk_pattern;
  int32_t n_pattern;
  int32_t topk_freq;
  int32_t skip_topk_offset;
} dsa_layer_rule;

/* 1 if layer_id reuses the previous full layer's top-k (shared), 0 if it runs its
 * own indexer (full), < 0 on a bad rule or layer id.  A shared layer owns no
 * index-K pages and skips store, logits and top-k; its sparse MLA takes the last
 * full layer's index tensor unchanged (zero copy) ([IDXC] §空壳 and
 * §模型侧的另一道门:should_run_indexer). */
int dsa_layer_is_shared(const dsa_layer_rule* rule, int32_t layer_id);

/* MTP draft-step top-k carry ([IDXC] §优化三:MTP 迭代内复用 topk).  The draft steps of one
 * MTP iteration reuse the top-k seed of its first step instead of scoring the MTP layer's own
 * index-K cache again: step 0 runs dsa_indexer_topk, steps 1.. pass that idx tensor (the same
 * device pointer, no copy) to dsa_sparse_mla_decode, as a shared layer does.  The saving is
 * (steps - 1) x 132 L bytes of indexer reads per iteration.
 * dsa_mtp_seed_width: the seed's width, index_topk + index_kpool - 1 (2048 with index_kpool
 * 1); -1 if index_topk is not in [1, 2048] or index_kpool < 1.
 * dsa_mtp_carry_allowed: 1 when the carry is valid, which needs a single draft chain
 * (eagle_topk == 1: wider drafts reorder rows and the seed no longer lines up); 0 otherwise;
 * -1 if eagle_topk < 1.  Host-only; no device work. */
int32_t dsa_mtp_seed_width(int32_t index_topk, int32_t index_kpool);
int dsa_mtp_carry_allowed(int32_t eagle_topk);

/* ---------------------------------------------------------------- quantisation */

/* Per-128-element block FP8 quantisation with a ue8m0 scale (the indexer query
 * format, [IDXC] §读取路径里的两条"非缓存"字节: fp8 q plus one scale per 128 dims).
 * x_bf16: device [n_blocks][128] bf16; y_fp8: device [n_blocks][128];
 * scale: device [n_blocks] fp32.  Bit-exact (bf16 / 2^e is exact). */
dsa_status dsa_quant_fp8(const uint16_t* x_bf16, int64_t n_blocks, uint8_t* y_fp8, float* scale,
                         void* stream);

/* Index-K store ([IDXC] §索引器缓存里存的是什么; [REQ] §4.5): for each token,
 * LayerNorm over 128 dims (no affine, biased variance, eps ln_eps), interleaved
 * RoPE on dims 0..63 at the token's position (pairs (2i, 2i+1), angle
 * pos * rope_theta^(-i/32) evaluated in double), ue8m0 + fp8, written to the
 * token's page slot.  k_bf16: device [tok->n][128].  index_cache: device
 * [pt->num_pages][8448], or NULL for a shared layer (then the call does nothing
 * and returns DSA_OK, like the pages' ownership gate).  Tokens with pos < 0 are
 * skipped. */
dsa_status dsa_index_k_store(const uint16_t* k_bf16, const dsa_rows* tok, const dsa_pages* pt,
                             uint8_t* index_cache, double ln_eps, double rope_theta, void* stream);

/* MXFP4 index-K store: the compressed indexer-cache format ([IDXC] §读取路径里的两条
 * "非缓存"字节, the paragraph on vLLM's two indexer-cache formats: 128/2 code bytes plus
 * 128/32 ue8m0 scales, 68 B per token).  Same LayerNorm and RoPE as dsa_index_k_store;
 * then per 32 dims the smallest power of two 2^e with amax <= 6 * 2^e, stored as the byte
 * e + 127 (E8M0), and e2m1 codes (OCP MX FP4) of x / 2^e, round to nearest even, two per
 * byte with the lower dim in the low nibble.  Page layout (4352 B): [64 tokens x 64 code
 * bytes][64 tokens x 4 scale bytes].  index_cache: device [pt->num_pages][4352], or NULL
 * (shared layer: no-op).  Tokens with pos < 0 are skipped.  Same argument errors as
 * dsa_index_k_store. */
dsa_status dsa_index_k_store_mxfp4(const uint16_t* k_bf16, const dsa_rows* tok, const dsa_pages* pt,
                                   uint8_t* index_cache, double ln_eps, double rope_theta, void* stream);

/* Latent store: 576 bf16 -> one 656-B record per token (layout above).
 * kv_bf16: device [tok->n][576]; latent_cache: device [pt->num_pages][41984].
 * Bit-exact.  Tokens with pos < 0 are skipped. */
dsa_status dsa_latent_store(const uint16_t* kv_bf16, const dsa_rows* tok, const dsa_pages* pt,
                            uint8_t* latent_cache, void* stream);

/* Fused norm + RoPE + dual-cache write: the step after the KV A projection, one pass per
 * token ([VLLM] §KV 低秩投影与缓存: RMSNorm of the 512-dim KV latent and RoPE of the 64-dim
 * rope key are what the main cache holds; [REQ] §4.3 两个 RMSNorm 与 RoPE: fused_norm_rope also
 * rotates the query's rope part and, with has_indexer, writes the indexer key too).
 * For each token with pos >= 0, in double precision:
 *   c^ = c / sqrt(mean(c^2) + rms_eps) * gamma over the 512 latent dims (kv[0..511]);
 *   k~ = RoPE_pos(kv[512..575]) (interleaved pairs, angle pos * rope_theta^(-i/32));
 * the token's 656-B record gets c^ as four ue8m0-scaled fp8 blocks (one rounding from double)
 * and k~ rounded once to bf16.  With index_cache (a layer that runs its own indexer) the
 * token's index key k_idx is stored exactly as dsa_index_k_store stores it (ln_eps,
 * index_rope_theta).  With q_pe, the token's 64 query heads have their 64 rope dims rotated in
 * place with the same angles as k~ (one rounding to bf16).
 *   kv:           device bf16, row t at kv + t * kv_stride (kv_stride >= 576, multiple of 8;
 *                 e.g. the latent columns of the A projection's output row).
 *   gamma:        device bf16 [512], or NULL for gamma = 1.
 *   k_idx:        device bf16 [tok->n][128]; required when index_cache is given, else unused.
 *   latent_cache: device [pt->num_pages][41984].
 *   index_cache:  device [pt->num_pages][8448], or NULL (no indexer of its own: no index write).
 *   q_pe:         device bf16, head h of token t at q_pe + t * q_row_stride + h * q_head_stride
 *                 (64 contiguous dims; strides multiples of 8, q_head_stride >= 64 and heads of
 *                 different tokens not overlapping), or NULL.  Rewritten in place.
 * Pointers are 16-B aligned.  Padded tokens (pos < 0) are left alone everywhere, their q
 * included.  Argument errors: DSA_ERR_ARG (NULL latent_cache or kv, index_cache without
 * k_idx, bad strides or alignment, eps < 0 or theta <= 0). */
dsa_status dsa_fused_norm_rope_store(const uint16_t* kv, int64_t kv_stride, const uint16_t* gamma,
                                     const uint16_t* k_idx, const dsa_rows* tok, const dsa_pages* pt,
                                     uint8_t* latent_cache, uint8_t* index_cache, uint16_t* q_pe,
                                     int64_t q_row_stride, int64_t q_head_stride, double rms_eps, double ln_eps,
                                     double rope_theta, double index_rope_theta, void* stream);

/* ---------------------------------------------------------------- indexer */

/* Logits row stride: (max_pos + 1) rounded up to 256 elements ([IDXC]
 * §临时缓冲:logits 矩阵, rows aligned to 256 columns). */
int64_t dsa_logits_stride(int32_t max_pos);

/* Rows per chunk when R rows of row_bytes exceed budget_bytes, else 0 (no
 * chunking) ([IDXC] §临时缓冲:logits 矩阵, mqa_logits_rows_per_chunk). */
int64_t dsa_logits_rows_per_chunk(int64_t num_rows, int64_t row_bytes, int64_t budget_bytes);

/* Lightning-indexer scores ([VLLM] §DSA Indexer):
 *   logits[r][s] = sum_h w[r][h] * ReLU(q_scale[r][h] * k_scale[s] * <q_fp8[r][h], k_fp8[s]>)
 * for s <= pos[r]; -inf for pos[r] < s < stride (and the whole row if pos[r] < 0).
 * q_fp8: device [R][32][128]; q_scale, w: device fp32 [R][32]; logits: device fp32
 * [R][stride], stride >= dsa_logits_stride(rows->max_pos).  index_cache NULL =
 * shared layer: no-op.  Rows of one group read the request's pages once. */
dsa_status dsa_indexer_logits(const uint8_t* q_fp8, const float* q_scale, const float* w,
                              const dsa_rows* rows, const dsa_pages* pt, const uint8_t* index_cache,
                              float* logits, int64_t stride, void* stream);

/* The same scores against an MXFP4 index-K cache (written by dsa_index_k_store_mxfp4):
 *   logits[r][s] = sum_h w[r][h] * ReLU(q_scale[r][h] * sum_b 2^(e_b[s]-127) * <q_fp8[r][h], k4[s]>_b)
 * over the four 32-dim blocks b.  index_cache: device [pt->num_pages][4352].  Other
 * arguments, layout and errors as dsa_indexer_logits. */
dsa_status dsa_indexer_logits_mxfp4(const uint8_t* q_fp8, const float* q_scale, const float* w,
                                    const dsa_rows* rows, const dsa_pages* pt, const uint8_t* index_cache,
                                    float* logits, int64_t stride, void* stream);

/* ---------------------------------------------------------------- top-k */

/* Workspace for dsa_topk, in bytes. */
size_t dsa_topk_workspace_size(int32_t R, int64_t stride, int32_t k);

/* Per-row top-k ([VLLM] §DSA Indexer, TopK over positions; [REQ] §4.5 top-2048
 * into topk_indices_buffer).  idx: device int32 [R][k], the k positions with the
 * largest logits among s <= pos[r], written in ascending position order.  If
 * pos[r] + 1 <= k the row is [0, 1, ..., pos[r], -1, ...] without reading logits
 * ([IDXC] §优化二:短上下文直接跳过打分); a padded row is all -1.  Among exactly
 * equal scores at the threshold the lower positions are kept.  k in [1, 2048].  Rows of at
 * most 32,768 visible scores are selected by one work-group each, which uses no workspace;
 * ws is still checked. */
dsa_status dsa_topk(const float* logits, int64_t stride, const dsa_rows* rows, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* Fused indexer + top-k: the same idx as dsa_indexer_logits followed by dsa_topk, without
 * writing the full logits.  Scores of one page in sixteen set a per-row threshold; the
 * full scoring pass keeps only the (score, position) pairs at or above it, and the exact
 * top-k runs over those.  A row whose pairs come out fewer than k or more than the list
 * holds is scored in full and takes the radix top-k instead, so the selection never
 * depends on the sample.  `logits` is scratch: on return it holds the sampled pages'
 * scores and the full scores of rows that fell back (on the direct path below, the scores of
 * every scored row group); other entries are unspecified.  A
 * row group (rows->group consecutive rows) whose rows all have pos + 1 <= k is not scored
 * ([IDXC] §优化二:短上下文直接跳过打分).  A call whose R x stride is at most the direct
 * limit (dsa_set_topk_direct_limit; 4,194,304 scores by default) writes every score and takes
 * the radix top-k directly (the filter's extra steps cost more than they save there); the
 * result is the same.  Arguments as for the two calls; ws sized by
 * dsa_topk_workspace_size(R, stride, k).  index_cache must not be NULL (a shared layer
 * reuses the full layer's idx instead). */
dsa_status dsa_indexer_topk(const uint8_t* q_fp8, const float* q_scale, const float* w,
                            const dsa_rows* rows, const dsa_pages* pt, const uint8_t* index_cache,
                            float* logits, int64_t stride, int32_t k, int32_t* idx,
                            void* ws, size_t ws_bytes, void* stream);

/* Tuning: the score-array size (R x stride) up to which dsa_indexer_topk and
 * dsa_indexer_topk_mxfp4 write every score and take the radix top-k directly instead of the
 * sampled-threshold filter (both give the same idx; which is faster depends on the shape).
 * Sets the limit for the process and returns the previous one; a negative argument only
 * returns the current limit.  0 sends every call with a row longer than k through the filter.
 * Takes effect for calls issued after it returns. */
int64_t dsa_set_topk_direct_limit(int64_t max_scores);

/* The fused indexer + top-k against an MXFP4 index-K cache: the same idx as
 * dsa_indexer_logits_mxfp4 followed by dsa_topk.  Arguments and errors as dsa_indexer_topk. */
dsa_status dsa_indexer_topk_mxfp4(const uint8_t* q_fp8, const float* q_scale, const float* w,
                                  const dsa_rows* rows, const dsa_pages* pt, const uint8_t* index_cache,
                                  float* logits, int64_t stride, int32_t k, int32_t* idx,
                                  void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- sparse MLA */

/* Workspace for dsa_sparse_mla_decode / _prefill, in bytes (may be 0).  Its contents need no
 * initialisation: with 256 rows or more, rows split between two work-groups are merged through
 * per-slot tag words that each call sets to a random 64-bit value and clears again before it
 * ends, so a workspace can be reused by any number of calls, also from a captured graph
 * replayed many times.  Calls that share one workspace must not overlap (on one stream, or
 * ordered by events). */
size_t dsa_sparse_mla_workspace_size(int32_t R, int32_t k);

/* Sparse MLA in absorbed (MQA) form ([VLLM] §Sparse MLA Attention; [REQ]
 * §decode:MQA 形态与吸收): for each row r and head h,
 *   l_j = sm_scale * <q[r][h][0:576], [c_j ; kr_j]>,  o[r][h] = sum_j softmax_j(l) c_j
 * over the positions j = idx[r][*] with 0 <= j <= pos[r] (causal mask; -1 entries
 * skipped; a repeated position counts once per occurrence), c_j the dequantised
 * 512-dim latent and kr_j its 64 bf16 rope dims.  q_bf16: device [R][64][576];
 * idx: device int32 [R][k] (logical positions, any order); out_bf16: device
 * [R][64][512]; lse (nullable): device fp32 [R][64], natural-log sum of exp of l
 * (-inf and o = 0 when nothing is selected).  Shared layers pass the last full
 * layer's idx pointer unchanged.  _decode is tuned for few rows per call,
 * _prefill for many (chunked prefill); both compute the same function. */
dsa_status dsa_sparse_mla_decode(const uint16_t* q_bf16, const dsa_rows* rows, const dsa_pages* pt,
                                 const uint8_t* latent_cache, const int32_t* idx, int32_t k,
                                 float sm_scale, uint16_t* out_bf16, float* lse,
                                 void* ws, size_t ws_bytes, void* stream);
dsa_status dsa_sparse_mla_prefill(const uint16_t* q_bf16, const dsa_rows* rows, const dsa_pages* pt,
                                  const uint8_t* latent_cache, const int32_t* idx, int32_t k,
                                  float sm_scale, uint16_t* out_bf16, float* lse,
                                  void* ws, size_t ws_bytes, void* stream);

/* dsa_sparse_mla_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It computes the same function as dsa_sparse_mla_decode, within the same
 * tolerance (fewer than 256 rows may run in fewer splits).  Its scratch is a fixed array of
 * 67,636,232 B (64.5 MiB) in device memory, one per GPU, that the library holds from the first
 * call on that GPU until the process ends; the call itself allocates nothing (no hipMalloc or
 * allocating library routine).  The array serves any row count: 256 rows or more take the
 * stream-K schedule, whose need is exactly its size; fewer rows take at most as many splits as
 * it holds.  A need beyond the array returns DSA_ERR_WORKSPACE before any launch.  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (on different streams, or from
 * different threads, without ordering) race and give wrong results; calls ordered on one stream
 * do not.  The array keeps the last call's contents; no call needs it cleared.  The current
 * device must be the GPU of `stream`.  Arguments and other errors as dsa_sparse_mla_decode. */
dsa_status dsa_sparse_mla_decode_noalloc(const uint16_t* q_bf16, const dsa_rows* rows, const dsa_pages* pt,
                                         const uint8_t* latent_cache, const int32_t* idx, int32_t k,
                                         float sm_scale, uint16_t* out_bf16, float* lse, void* stream);

/* ---------------------------------------------------------------- reference-rate probes
 * Not steps of the layer: they measure, on the device at hand, the plain access patterns the
 * hot kernels perform, so that a kernel's rate can be stated beside a measured one as well as
 * beside the nominal HBM peak.  Both read every byte they are given once, with non-temporal
 * 16-B loads, and write the XOR of the words each work-group read to sink[0 ..
 * DSA_PROBE_SINK_WORDS) (device uint32; every word is written), so that no load is optimised
 * away: the XOR of the sink's words is the XOR of every word read.  Errors: DSA_ERR_ARG for
 * sizes or pointers as stated; DSA_ERR_HIP for launch failures.
 *
 * dsa_probe_stream_read: `bytes` (a multiple of 16) of device memory at buf (16-B aligned),
 * as a grid-stride stream of 16-B loads, several in flight per thread: the shape of the
 * indexer's index-K scan ("GLM-5.3 推理全链路(十一)", section on the read bandwidth).
 *
 * dsa_probe_gather_records: the n records of rec_bytes (a multiple of 16) at record indices
 * ids[0..n) (device int32; values outside [0, pool_records) are clamped into the pool) of
 * pool (device, 16-B aligned), each read whole: the shape of the sparse MLA's gather of its
 * selected 656-B latent records ("vLLM 推理链路概览: 以 GLM-5.2 为例", section Sparse MLA
 * Attention). */
#define DSA_PROBE_SINK_WORDS 2048
dsa_status dsa_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);
dsa_status dsa_probe_gather_records(const uint8_t* pool, int64_t pool_records, int32_t rec_bytes,
                                    const int32_t* ids, int64_t n, uint32_t* sink, void* stream);

/* ---------------------------------------------------------------- diagnostics */

/* Synchronises the current device and reports (then clears) the device error flag
 * raised by in-kernel range checks: DSA_OK or DSA_ERR_DEVICE_CHECK. */
dsa_status dsa_check_device_errors(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
