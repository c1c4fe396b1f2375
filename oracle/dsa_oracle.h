/*
 * dsa_oracle.h -- plain CPU reference of the DSA attention-layer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links or
 * calls this code; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source with the HIP path.
 *
 * Every floating-point step is evaluated in double precision and rounded once
 * to the storage type (fp8 E4M3, fp32 or bf16) at the end.
 *
 * Pages this code follows (cited by title and section):
 *   [IDXC] "GLM-5.3 推理全链路(十一): 索引器缓存的跨层读写" (pinghaoyang.com.cn)
 *   [REQ]  "GLM-5.3 推理全链路(一): 一个请求在 SGLang 里经过哪些算子、哪些通信"
 *   [VLLM] "vLLM 推理链路概览: 以 GLM-5.2 为例" (xpengzhao.github.io)
 *
 * Fixed shapes: page of 64 tokens; indexer head dim 128, 32 indexer heads;
 * MLA: 64 heads, latent 512 + 64 rope dims; top-k width 2048.
 *
 * Byte layouts (readings of the pages, stated once here):
 *   index-K page  (8448 B)  = [64 x 128 B fp8 keys, token-major][64 x fp32 scale]
 *   latent record ( 656 B)  = [512 B fp8 latent][4 x fp32 block scale][64 x bf16 rope]
 *   latent page   (41984 B) = 64 latent records, token-major
 *   MXFP4 index-K page (4352 B) = [64 x 64 B packed e2m1 codes, token-major, lower dim in
 *                    the low nibble][64 x 4 E8M0 scale bytes, one per 32 dims]
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* FP8 E4M3 (OCP e4m3fn): decode, RNE encode with saturation to +-448. */
double  orc_fp8_decode(uint8_t code);
uint8_t orc_fp8_encode(double x);
/* Same encode by exhaustive nearest search over all finite codes (a pin for the above). */
uint8_t orc_fp8_encode_bruteforce(double x);

/* ue8m0 block scale: smallest power of two s with amax <= 448*s; amax==0 -> 1. */
double  orc_ue8m0_scale(double amax);

/* MXFP4 elements (OCP e2m1, a 4-bit code): decode; RNE encode saturating to +-6; the
 * same encode by exhaustive search; the scale rule with 6 in place of 448. */
double  orc_fp4_decode(uint8_t code);
uint8_t orc_fp4_encode(double x);
uint8_t orc_fp4_encode_bruteforce(double x);
double  orc_ue8m0_scale_fp4(double amax);

/* bf16 <-> double; double -> bf16 rounds to nearest even (directly, no fp32 step). */
double   orc_bf16_to_double(uint16_t h);
uint16_t orc_double_to_bf16(double x);

/* Interleaved RoPE on dims [0,64) of a 128-vector, in place.  inverse != 0 rotates by -angle. */
void orc_rope64(double* y, int64_t pos, double theta, int inverse);

/* LayerNorm over 128 dims, no affine, biased variance. */
void orc_layernorm128(const double* x, double* y, double eps);

/* Per-128-block quantisation: n_blocks blocks of 128 bf16 -> fp8 codes + fp32 scale. */
void orc_quant_fp8(const uint16_t* x_bf16, int64_t n_blocks, uint8_t* y_fp8, float* scale);

/* Index-K store: LN -> RoPE(dims 0..63) -> ue8m0 + fp8, written into the paged cache.
 * Rows with pos < 0 are skipped.  pre_quant (nullable, [n][128]) receives y/scale before rounding. */
void orc_index_k_store(const uint16_t* k_bf16, const int32_t* req, const int32_t* pos, int64_t n,
                       const int32_t* page_table, int64_t pt_stride,
                       uint8_t* cache, double eps, double theta, double* pre_quant);

/* Fused norm + RoPE + cache writes: RMSNorm(kv[0:512]) * gamma -> 4 scaled fp8 blocks,
 * RoPE(kv[512:576]) -> bf16 tail of the 656-B record; the index-K entry when index_cache and
 * k_idx are given; q_pe (nullable) rotated in place, 64 heads x 64 dims per token. */
void orc_fused_norm_rope_store(const uint16_t* kv, int64_t kv_stride, const uint16_t* gamma,
                               const uint16_t* k_idx, const int32_t* req, const int32_t* pos, int64_t n,
                               const int32_t* page_table, int64_t pt_stride, uint8_t* latent_cache,
                               uint8_t* index_cache, uint16_t* q_pe, int64_t q_row_stride,
                               int64_t q_head_stride, double rms_eps, double ln_eps, double rope_theta,
                               double index_rope_theta);

/* Latent store: 576 bf16 -> 656-B record (4 scaled fp8 blocks + bf16 rope tail). */
void orc_latent_store(const uint16_t* kv_bf16, const int32_t* req, const int32_t* pos, int64_t n,
                      const int32_t* page_table, int64_t pt_stride, uint8_t* cache);

/* Indexer logits I[r][s] for s <= pos[r]; -inf elsewhere (s < stride). */
void orc_indexer_logits(const uint8_t* q_fp8, const float* q_scale, const float* w,
                        const int32_t* req, const int32_t* pos, int64_t R,
                        const int32_t* page_table, int64_t pt_stride, const uint8_t* cache,
                        float* logits, int64_t stride);

/* MXFP4 index-K store: LN -> RoPE(dims 0..63) -> per-32-dim ue8m0 (max 6) + e2m1 codes,
 * written into a 4352-B page. */
void orc_index_k_store_mxfp4(const uint16_t* k_bf16, const int32_t* req, const int32_t* pos, int64_t n,
                             const int32_t* page_table, int64_t pt_stride,
                             uint8_t* cache, double eps, double theta);

/* Indexer logits against an MXFP4 index-K cache. */
void orc_indexer_logits_mxfp4(const uint8_t* q_fp8, const float* q_scale, const float* w,
                              const int32_t* req, const int32_t* pos, int64_t R,
                              const int32_t* page_table, int64_t pt_stride, const uint8_t* cache,
                              float* logits, int64_t stride);

/* Top-k as a set: the k largest by (score desc, position asc), written ascending by
 * position; -1 tail.  If pos[r]+1 <= k all visible positions are returned.
 * kth (nullable, [R]) receives the k-th largest score (NaN when no selection happened). */
void orc_topk(const float* logits, int64_t stride, const int32_t* pos, int64_t R, int32_t k,
              int32_t* idx, float* kth);

/* Sparse MLA (absorbed, MQA form) over the given logical positions. */
void orc_sparse_mla(const uint16_t* q_bf16, const int32_t* req, const int32_t* pos, int64_t R,
                    const int32_t* page_table, int64_t pt_stride, const uint8_t* latent_cache,
                    const int32_t* idx, int32_t k, double sm_scale,
                    uint16_t* out_bf16, float* lse);

/* Full/shared layer rule.  types / pattern: nullable strings of 'F'/'S'. */
int orc_layer_is_shared(const char* types, int32_t n_types, int32_t cli_factor,
                        const char* pattern, int32_t n_pattern,
                        int32_t topk_freq, int32_t skip_topk_offset, int32_t layer_id);

/* Array helpers used by the tests. */
void orc_fp8_encode_array(const double* x, int64_t n, uint8_t* out, int brute);
void orc_fp8_decode_array(const uint8_t* c, int64_t n, double* out);
void orc_bf16_from_double_array(const double* x, int64_t n, uint16_t* out);
void orc_ue8m0_array(const double* amax, int64_t n, double* out);
/* LN (optional) then RoPE (or its inverse) per 128-vector at position pos[t]. */
void orc_ln_rope_array(const double* x, const int64_t* pos, int64_t n, double eps, double theta,
                       int do_ln, int inverse, double* out);

#ifdef __cplusplus
}
#endif
#endif
