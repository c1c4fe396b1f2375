/*
 * dsa_oracle.c -- plain, slow, obviously-correct CPU reference of the DSA
 * attention-layer hot path (index-K store, indexer scoring, top-k, sparse MLA,
 * layer rule).
 *
 * TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the product library.  It shares
 * no code, header, table or constant generator with the HIP path.
 *
 * Arithmetic: double precision throughout; one rounding at the end of each
 * stage to the stored type.  OpenMP is used only across independent rows or
 * tokens (never inside a reduction), so results do not depend on thread count.
 *
 * Page citations use the tags defined in dsa_oracle.h ([IDXC], [REQ], [VLLM]).
 */
#include "dsa_oracle.h"
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define PAGE          64
#define IDX_DIM       128
#define IDX_HEADS     32
#define IDX_PAGE_B    8448      /* 64 * (128 + 4): [IDXC] §索引器缓存里存的是什么 */
#define IDX_SCALE_OFF 8192      /* scales follow the 64 keys inside a page */
#define MLA_HEADS     64
#define LAT_DIM       512
#define ROPE_DIM      64
#define LAT_REC_B     656       /* [IDXC] §主 KV 缓存里存的是什么 */
#define LAT_PAGE_B    (PAGE * LAT_REC_B)
#define FP8_MAX       448.0

/* ------------------------------------------------------------------ FP8 E4M3
 * OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinity;
 * S.1111.111 is NaN; largest finite 448.  The pages name the format "FP8 E4M3"
 * ([REQ] launch flags, --kv-cache-dtype fp8_e4m3). */
double orc_fp8_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);            /* subnormal */
    else        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round to nearest, ties to even code; saturate to 448; NaN -> 0x7F. */
uint8_t orc_fp8_encode(double x) {
    uint8_t sign;
    double a, r;
    int e, m;
    if (isnan(x)) return 0x7F;
    sign = signbit(x) ? 0x80 : 0x00;
    a = fabs(x);
    if (a >= FP8_MAX) return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: quantum 2^-9; m == 8 lands on the smallest normal (code 8) */
        r = nearbyint(a / ldexp(1.0, -9));
        return sign | (uint8_t)r;
    }
    frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1) -> unbiased exponent e-1 */
    e -= 1;
    r = nearbyint((a / ldexp(1.0, e) - 1.0) * 8.0);   /* mantissa in eighths, RNE */
    m = (int)r;
    if (m == 8) { m = 0; e += 1; }
    if (e + 7 > 15 || (e + 7 == 15 && m == 7)) return sign | 0x7E;  /* rounds past 448 */
    return sign | (uint8_t)(((e + 7) << 3) | m);
}

uint8_t orc_fp8_encode_bruteforce(double x) {
    uint8_t sign, best = 0;
    double a, bd = INFINITY;
    int c;
    if (isnan(x)) return 0x7F;
    sign = signbit(x) ? 0x80 : 0x00;
    a = fabs(x);
    if (a >= FP8_MAX) return sign | 0x7E;
    for (c = 0; c < 0x7F; c++) {
        double d = fabs(a - orc_fp8_decode((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = (uint8_t)c; }
    }
    return sign | best;
}

/* ue8m0 scale: a power of two chosen so that the block's largest magnitude
 * fits the FP8 range ([IDXC] §索引器缓存里存的是什么: one 4-byte ue8m0 factor
 * per 128 dims).  Smallest such power, found by exact comparisons. */
double orc_ue8m0_scale(double amax) {
    int e;
    if (!(amax > 0.0)) return 1.0;
    e = ilogb(amax) - 8;
    while (amax > ldexp(FP8_MAX, e)) e++;
    while (amax <= ldexp(FP8_MAX, e - 1)) e--;
    return ldexp(1.0, e);
}

/* ------------------------------------------------------------------ bf16 */
double orc_bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

uint16_t orc_double_to_bf16(double x) {
    double a, q, r;
    int e;
    float f;
    uint32_t u;
    if (isnan(x)) return 0x7FC0;
    a = fabs(x);
    if (a == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    e = ilogb(a);
    if (e < -126) e = -126;                 /* subnormal quantum 2^-133 */
    q = ldexp(1.0, e - 7);                  /* 8 significant bits */
    r = nearbyint(a / q) * q;
    if (r > ldexp(255.0 / 128.0, 127)) return signbit(x) ? 0xFF80 : 0x7F80;
    f = (float)r;                           /* exact: r has <= 8 significant bits */
    memcpy(&u, &f, 4);
    return (uint16_t)((u >> 16) | (signbit(x) ? 0x8000 : 0));
}

/* ------------------------------------------------------------------ LN, RoPE
 * Index-K preparation ([IDXC] §索引器缓存里存的是什么): the indexer key passes
 * through k_norm (a LayerNorm), then RoPE acting on its first 64 dims only, then
 * FP8 quantisation.  [REQ] §4.5 states the indexer RoPE is interleaved. */
void orc_layernorm128(const double* x, double* y, double eps) {
    double mu = 0.0, var = 0.0, inv;
    int d;
    for (d = 0; d < IDX_DIM; d++) mu += x[d];
    mu /= IDX_DIM;
    for (d = 0; d < IDX_DIM; d++) var += (x[d] - mu) * (x[d] - mu);
    var /= IDX_DIM;
    inv = 1.0 / sqrt(var + eps);
    for (d = 0; d < IDX_DIM; d++) y[d] = (x[d] - mu) * inv;
}

void orc_rope64(double* y, int64_t pos, double theta, int inverse) {
    int i;
    for (i = 0; i < ROPE_DIM / 2; i++) {
        double inv_freq = pow(theta, -(2.0 * i) / (double)ROPE_DIM);
        double ang = (double)pos * inv_freq;
        double c = cos(ang), s = inverse ? -sin(ang) : sin(ang);
        double a = y[2 * i], b = y[2 * i + 1];
        y[2 * i]     = a * c - b * s;
        y[2 * i + 1] = a * s + b * c;
    }
}

/* One 128-block: scale + codes.  pre (nullable) receives x/scale before rounding. */
static float quant_block(const double* x, uint8_t* codes, double* pre) {
    double amax = 0.0, s;
    int d;
    for (d = 0; d < 128; d++) if (fabs(x[d]) > amax) amax = fabs(x[d]);
    s = orc_ue8m0_scale(amax);
    for (d = 0; d < 128; d++) {
        double v = x[d] / s;             /* exact: s is a power of two */
        if (pre) pre[d] = v;
        codes[d] = orc_fp8_encode(v);
    }
    return (float)s;
}

void orc_quant_fp8(const uint16_t* x_bf16, int64_t n_blocks, uint8_t* y_fp8, float* scale) {
    int64_t b;
#pragma omp parallel for schedule(static)
    for (b = 0; b < n_blocks; b++) {
        double x[128];
        int d;
        for (d = 0; d < 128; d++) x[d] = orc_bf16_to_double(x_bf16[b * 128 + d]);
        scale[b] = quant_block(x, y_fp8 + b * 128, NULL);
    }
}

/* ------------------------------------------------------------------ paging
 * A logical position p of request b lives in page page_table[b][p / 64], slot
 * p % 64 ([IDXC] §优化一:按页分块打分: 64-token pages; one page table serves
 * both caches because their pages share ids, [REQ] §prefix cache). */
static int64_t page_of(const int32_t* pt, int64_t pt_stride, int32_t req, int64_t p) {
    return (int64_t)pt[(int64_t)req * pt_stride + p / PAGE];
}

/* One token's index-K entry: LN, RoPE at p, ue8m0 + fp8 into its page slot. */
static void index_k_entry(const uint16_t* k_row, int32_t r, int64_t p, const int32_t* page_table,
                          int64_t pt_stride, uint8_t* cache, double eps, double theta, double* pre) {
    double x[IDX_DIM], y[IDX_DIM];
    uint8_t* base;
    int d;
    float s;
    for (d = 0; d < IDX_DIM; d++) x[d] = orc_bf16_to_double(k_row[d]);
    orc_layernorm128(x, y, eps);
    orc_rope64(y, p, theta, 0);
    base = cache + page_of(page_table, pt_stride, r, p) * IDX_PAGE_B;
    s = quant_block(y, base + (p % PAGE) * IDX_DIM, pre);
    memcpy(base + IDX_SCALE_OFF + (p % PAGE) * 4, &s, 4);
}

void orc_index_k_store(const uint16_t* k_bf16, const int32_t* req, const int32_t* pos, int64_t n,
                       const int32_t* page_table, int64_t pt_stride,
                       uint8_t* cache, double eps, double theta, double* pre_quant) {
    int64_t t;
    if (!cache) return;                    /* shared layer: no index-K of its own */
#pragma omp parallel for schedule(static)
    for (t = 0; t < n; t++) {
        if (pos[t] < 0) continue;          /* padded row: nothing written */
        index_k_entry(k_bf16 + t * IDX_DIM, req[t], pos[t], page_table, pt_stride, cache, eps, theta,
                      pre_quant ? pre_quant + t * IDX_DIM : NULL);
    }
}

void orc_latent_store(const uint16_t* kv_bf16, const int32_t* req, const int32_t* pos, int64_t n,
                      const int32_t* page_table, int64_t pt_stride, uint8_t* cache) {
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < n; t++) {
        double x[LAT_DIM];
        int64_t p = pos[t];
        uint8_t* rec;
        int b, d;
        if (p < 0) continue;
        rec = cache + page_of(page_table, pt_stride, req[t], p) * LAT_PAGE_B + (p % PAGE) * LAT_REC_B;
        for (d = 0; d < LAT_DIM; d++) x[d] = orc_bf16_to_double(kv_bf16[t * 576 + d]);
        for (b = 0; b < 4; b++) {
            float s = quant_block(x + 128 * b, rec + 128 * b, NULL);
            memcpy(rec + LAT_DIM + 4 * b, &s, 4);
        }
        memcpy(rec + LAT_DIM + 16, kv_bf16 + t * 576 + LAT_DIM, ROPE_DIM * 2);  /* rope tail stays bf16 */
    }
}

/* ------------------------------------------------------------------ fused norm + RoPE + cache writes
 * The step after the KV A projection ([VLLM] §KV 低秩投影与缓存; [REQ] §4.3 两个 RMSNorm 与
 * RoPE, the fused_norm_rope kernel with its has_indexer switch), per token at position p:
 *   c^ = c / sqrt(mean(c^2) + eps) * gamma      over the 512 latent dims (RMSNorm as in
 *                                              [VLLM] §RMSNorm 与残差路径; gamma = 1 if NULL)
 *   k~ = RoPE_p(k_R)                            over the 64 rope dims (interleaved pairs)
 * c^ goes into the 656-B record as four ue8m0-scaled fp8 blocks, rounded once from double;
 * k~ is rounded once to bf16 into the record's tail.  With an index-K cache (a layer that
 * runs its own indexer) the token's index key is stored exactly as orc_index_k_store does;
 * q_pe (NULL to skip) holds the token's 64 per-head 64-dim rope parts, rotated in place with
 * the same angles as k~.  Padded tokens (p < 0) are left alone. */
void orc_fused_norm_rope_store(const uint16_t* kv, int64_t kv_stride, const uint16_t* gamma,
                               const uint16_t* k_idx, const int32_t* req, const int32_t* pos, int64_t n,
                               const int32_t* page_table, int64_t pt_stride, uint8_t* latent_cache,
                               uint8_t* index_cache, uint16_t* q_pe, int64_t q_row_stride,
                               int64_t q_head_stride, double rms_eps, double ln_eps, double rope_theta,
                               double index_rope_theta) {
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < n; t++) {
        double c[LAT_DIM], kr[ROPE_DIM], ms = 0.0, rms;
        int64_t p = pos[t];
        const uint16_t* src = kv + t * kv_stride;
        uint8_t* rec;
        int b, d, h;
        if (p < 0) continue;
        for (d = 0; d < LAT_DIM; d++) {
            c[d] = orc_bf16_to_double(src[d]);
            ms += c[d] * c[d];
        }
        rms = sqrt(ms / LAT_DIM + rms_eps);
        for (d = 0; d < LAT_DIM; d++) c[d] = c[d] / rms * (gamma ? orc_bf16_to_double(gamma[d]) : 1.0);
        rec = latent_cache + page_of(page_table, pt_stride, req[t], p) * LAT_PAGE_B + (p % PAGE) * LAT_REC_B;
        for (b = 0; b < 4; b++) {
            float s = quant_block(c + 128 * b, rec + 128 * b, NULL);
            memcpy(rec + LAT_DIM + 4 * b, &s, 4);
        }
        for (d = 0; d < ROPE_DIM; d++) kr[d] = orc_bf16_to_double(src[LAT_DIM + d]);
        orc_rope64(kr, p, rope_theta, 0);
        for (d = 0; d < ROPE_DIM; d++) {
            uint16_t hb = orc_double_to_bf16(kr[d]);
            memcpy(rec + LAT_DIM + 16 + 2 * d, &hb, 2);
        }
        if (index_cache && k_idx)
            index_k_entry(k_idx + t * IDX_DIM, req[t], p, page_table, pt_stride, index_cache, ln_eps,
                          index_rope_theta, NULL);
        if (q_pe)
            for (h = 0; h < MLA_HEADS; h++) {
                uint16_t* q = q_pe + t * q_row_stride + h * q_head_stride;
                double v[ROPE_DIM];
                for (d = 0; d < ROPE_DIM; d++) v[d] = orc_bf16_to_double(q[d]);
                orc_rope64(v, p, rope_theta, 0);
                for (d = 0; d < ROPE_DIM; d++) q[d] = orc_double_to_bf16(v[d]);
            }
    }
}

/* ------------------------------------------------------------------ indexer
 * Score of query row r against visible position s ([VLLM] §DSA Indexer):
 *   I[r][s] = sum_h w[r][h] * ReLU(<q[r][h], k[s]>)
 * with q and k dequantised from FP8 by their block scales.  Positions after the
 * row's own position are masked ([VLLM] §Sparse MLA Attention, causal j <= i). */
void orc_indexer_logits(const uint8_t* q_fp8, const float* q_scale, const float* w,
                        const int32_t* req, const int32_t* pos, int64_t R,
                        const int32_t* page_table, int64_t pt_stride, const uint8_t* cache,
                        float* logits, int64_t stride) {
    double tab[256];
    int64_t r;
    int c;
    for (c = 0; c < 256; c++) tab[c] = orc_fp8_decode((uint8_t)c);
    for (r = 0; r < R; r++) {
        double q[IDX_HEADS][IDX_DIM];
        int64_t p = pos[r], s;
        int h, d;
        for (h = 0; h < IDX_HEADS; h++)
            for (d = 0; d < IDX_DIM; d++)
                q[h][d] = tab[q_fp8[(r * IDX_HEADS + h) * IDX_DIM + d]] * (double)q_scale[r * IDX_HEADS + h];
#pragma omp parallel for schedule(static)
        for (s = 0; s < stride; s++) {
            const uint8_t* page;
            const uint8_t* key;
            float ks;
            double k[IDX_DIM], acc = 0.0;
            int hh, dd;
            if (p < 0 || s > p) { logits[r * stride + s] = -INFINITY; continue; }
            page = cache + page_of(page_table, pt_stride, req[r], s) * IDX_PAGE_B;
            key = page + (s % PAGE) * IDX_DIM;
            memcpy(&ks, page + IDX_SCALE_OFF + (s % PAGE) * 4, 4);
            for (dd = 0; dd < IDX_DIM; dd++) k[dd] = tab[key[dd]] * (double)ks;
            for (hh = 0; hh < IDX_HEADS; hh++) {
                double dot = 0.0;
                for (dd = 0; dd < IDX_DIM; dd++) dot += q[hh][dd] * k[dd];
                acc += (double)w[r * IDX_HEADS + hh] * (dot > 0.0 ? dot : 0.0);
            }
            logits[r * stride + s] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------ top-k
 * The k best-scoring visible positions ([VLLM] §DSA Indexer, TopK over j).
 * When no more than k positions are visible every one of them is selected and
 * the tail is -1 ([IDXC] §优化二:短上下文直接跳过打分). */
typedef struct { float v; int32_t p; } orc_pair;

static int cmp_score_desc(const void* a, const void* b) {
    const orc_pair* x = (const orc_pair*)a;
    const orc_pair* y = (const orc_pair*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->p > y->p) - (x->p < y->p);
}

static int cmp_int_asc(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

void orc_topk(const float* logits, int64_t stride, const int32_t* pos, int64_t R, int32_t k,
              int32_t* idx, float* kth) {
    int64_t r;
#pragma omp parallel for schedule(dynamic)
    for (r = 0; r < R; r++) {
        int64_t n = (int64_t)pos[r] + 1, s;
        int32_t* out = idx + r * k;
        int32_t j;
        for (j = 0; j < k; j++) out[j] = -1;
        if (kth) kth[r] = NAN;
        if (n <= 0) continue;
        if (n <= k) {
            for (s = 0; s < n; s++) out[s] = (int32_t)s;
            continue;
        }
        {
            orc_pair* v = (orc_pair*)malloc((size_t)n * sizeof(orc_pair));
            for (s = 0; s < n; s++) { v[s].v = logits[r * stride + s]; v[s].p = (int32_t)s; }
            qsort(v, (size_t)n, sizeof(orc_pair), cmp_score_desc);
            for (j = 0; j < k; j++) out[j] = v[j].p;
            if (kth) kth[r] = v[k - 1].v;
            free(v);
            qsort(out, (size_t)k, sizeof(int32_t), cmp_int_asc);
        }
    }
}

/* ------------------------------------------------------------------ sparse MLA
 * Absorbed (MQA-form) MLA over the selected positions ([VLLM] §Sparse MLA
 * Attention; [REQ] §decode:MQA 形态与吸收): all 64 heads share the 576-dim
 * latent (512 latent + 64 rope) as key; the 512-dim latent is the value.
 *   logit_j = sm_scale * <q_h, [c_j ; kr_j]>,  o_h = sum_j softmax(logit)_j c_j
 * over selected j that are >= 0 and <= the row's position. */
void orc_sparse_mla(const uint16_t* q_bf16, const int32_t* req, const int32_t* pos, int64_t R,
                    const int32_t* page_table, int64_t pt_stride, const uint8_t* latent_cache,
                    const int32_t* idx, int32_t k, double sm_scale,
                    uint16_t* out_bf16, float* lse) {
    double tab[256];
    int64_t r;
    int c;
    for (c = 0; c < 256; c++) tab[c] = orc_fp8_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic)
    for (r = 0; r < R; r++) {
        int64_t p = pos[r];
        double* kv = (double*)malloc((size_t)k * 576 * sizeof(double));
        double* lg = (double*)malloc((size_t)k * sizeof(double));
        int32_t nv = 0, j;
        int h, d, b;
        for (j = 0; j < k; j++) {
            int64_t s = idx[r * k + j];
            const uint8_t* rec;
            if (p < 0 || s < 0 || s > p) continue;
            rec = latent_cache + page_of(page_table, pt_stride, req[r], s) * LAT_PAGE_B + (s % PAGE) * LAT_REC_B;
            for (b = 0; b < 4; b++) {
                float sc;
                memcpy(&sc, rec + LAT_DIM + 4 * b, 4);
                for (d = 0; d < 128; d++) kv[(int64_t)nv * 576 + 128 * b + d] = tab[rec[128 * b + d]] * (double)sc;
            }
            for (d = 0; d < ROPE_DIM; d++) {
                uint16_t hbits;
                memcpy(&hbits, rec + LAT_DIM + 16 + 2 * d, 2);
                kv[(int64_t)nv * 576 + LAT_DIM + d] = orc_bf16_to_double(hbits);
            }
            nv++;
        }
        for (h = 0; h < MLA_HEADS; h++) {
            const uint16_t* qh = q_bf16 + (r * MLA_HEADS + h) * 576;
            double q[576], m = -INFINITY, z = 0.0, o[LAT_DIM];
            for (d = 0; d < 576; d++) q[d] = orc_bf16_to_double(qh[d]);
            for (j = 0; j < nv; j++) {
                double dot = 0.0;
                for (d = 0; d < 576; d++) dot += q[d] * kv[(int64_t)j * 576 + d];
                lg[j] = sm_scale * dot;
                if (lg[j] > m) m = lg[j];
            }
            for (d = 0; d < LAT_DIM; d++) o[d] = 0.0;
            for (j = 0; j < nv; j++) {
                double e = exp(lg[j] - m);
                z += e;
                for (d = 0; d < LAT_DIM; d++) o[d] += e * kv[(int64_t)j * 576 + d];
            }
            for (d = 0; d < LAT_DIM; d++)
                out_bf16[(r * MLA_HEADS + h) * LAT_DIM + d] = orc_double_to_bf16(nv ? o[d] / z : 0.0);
            if (lse) lse[r * MLA_HEADS + h] = nv ? (float)(m + log(z)) : -INFINITY;
        }
        free(kv);
        free(lg);
    }
}

/* ------------------------------------------------------------------ layer rule
 * Which layers run their own indexer ([IDXC] §配置里的 78 个字符):
 * an explicit per-layer list wins; otherwise a cli_factor > 1 keeps every
 * cli_factor-th layer; otherwise an explicit 'S'/'F' pattern; otherwise a
 * frequency with an alignment offset, shared <=> max(l - offset + 1, 0) % freq != 0.
 * Layers beyond an explicit list or pattern count as full. */
int orc_layer_is_shared(const char* types, int32_t n_types, int32_t cli_factor,
                        const char* pattern, int32_t n_pattern,
                        int32_t topk_freq, int32_t skip_topk_offset, int32_t layer_id) {
    int32_t v;
    if (layer_id < 0) return -1;
    if (types) return layer_id < n_types && types[layer_id] == 'S';
    if (cli_factor > 1) return layer_id % cli_factor != 0;
    if (pattern) return layer_id < n_pattern && pattern[layer_id] == 'S';
    if (topk_freq < 1) return -1;
    v = layer_id - skip_topk_offset + 1;
    if (v < 0) v = 0;
    return v % topk_freq != 0;
}

/* ------------------------------------------------------------------ MXFP4 index-K
 * The compressed indexer-cache format ([IDXC] §读取路径里的两条"非缓存"字节, the
 * paragraph on vLLM's kv_cache_as_quant_view): head_dim/2 bytes of packed 4-bit codes
 * plus one ue8m0 scale per block of 32 dims, 128/2 + 128/32 = 68 B per token.
 * Readings (the page names the format only): the elements are OCP MX e2m1 (1 sign,
 * 2 exponent bits with bias 1, 1 mantissa bit; largest finite 6), rounded to nearest
 * with ties to the even code; each scale is the smallest power of two s with
 * amax <= 6*s (the same rule as the FP8 path with 6 in place of 448, so nothing
 * saturates), stored as its biased exponent byte (E8M0: 2^(byte-127)).  Two codes
 * per byte, the lower dim in the low nibble.  Page: [64 x 64 B codes][64 x 4 scale
 * bytes] = 4352 B (planar, like the FP8 page). */
#define FP4_MAX        6.0
#define MX4_TOKEN_B    64
#define MX4_PAGE_B     (PAGE * (MX4_TOKEN_B + 4))
#define MX4_SCALE_OFF  (PAGE * MX4_TOKEN_B)

double orc_fp4_decode(uint8_t c) {
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* RNE over the magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}: within each binade the step is a
 * quarter, half or one unit; the rounding is done on the mantissa, as for FP8. */
uint8_t orc_fp4_encode(double x) {
    uint8_t sign;
    double a, r;
    int e, m;
    if (isnan(x)) return 0x7;              /* no NaN code: the largest magnitude */
    sign = signbit(x) ? 0x8 : 0x0;
    a = fabs(x);
    if (a >= FP4_MAX) return sign | 0x7;
    if (a < 1.0) {                         /* subnormal binade: quantum 0.5; 2 -> code 2 (1.0) */
        r = nearbyint(a / 0.5);
        return sign | (uint8_t)r;
    }
    frexp(a, &e);
    e -= 1;                                /* a = f * 2^e, f in [1, 2) */
    r = nearbyint((a / ldexp(1.0, e) - 1.0) * 2.0);   /* mantissa in halves, RNE */
    m = (int)r;
    if (m == 2) { m = 0; e += 1; }
    if (e + 1 > 3) return sign | 0x7;      /* rounds past 6 */
    return sign | (uint8_t)(((e + 1) << 1) | m);
}

uint8_t orc_fp4_encode_bruteforce(double x) {
    uint8_t sign, best = 0;
    double a, bd = INFINITY;
    int c;
    if (isnan(x)) return 0x7;
    sign = signbit(x) ? 0x8 : 0x0;
    a = fabs(x);
    for (c = 0; c < 8; c++) {
        double d = fabs(a - orc_fp4_decode((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = (uint8_t)c; }
    }
    return sign | best;
}

/* Smallest power of two s with amax <= 6*s; amax == 0 -> 1. */
double orc_ue8m0_scale_fp4(double amax) {
    int e;
    if (!(amax > 0.0)) return 1.0;
    e = ilogb(amax) - 2;
    while (amax > ldexp(FP4_MAX, e)) e++;
    while (amax <= ldexp(FP4_MAX, e - 1)) e--;
    return ldexp(1.0, e);
}

void orc_index_k_store_mxfp4(const uint16_t* k_bf16, const int32_t* req, const int32_t* pos, int64_t n,
                             const int32_t* page_table, int64_t pt_stride,
                             uint8_t* cache, double eps, double theta) {
    int64_t t;
    if (!cache) return;                    /* shared layer: no index-K of its own */
#pragma omp parallel for schedule(static)
    for (t = 0; t < n; t++) {
        double x[IDX_DIM], y[IDX_DIM];
        int64_t p = pos[t], page;
        uint8_t* base;
        uint8_t* codes;
        int d, b;
        if (p < 0) continue;
        for (d = 0; d < IDX_DIM; d++) x[d] = orc_bf16_to_double(k_bf16[t * IDX_DIM + d]);
        orc_layernorm128(x, y, eps);
        orc_rope64(y, p, theta, 0);
        page = page_of(page_table, pt_stride, req[t], p);
        base = cache + page * MX4_PAGE_B;
        codes = base + (p % PAGE) * MX4_TOKEN_B;
        for (b = 0; b < IDX_DIM / 32; b++) {
            double amax = 0.0, s;
            int e;
            for (d = 32 * b; d < 32 * b + 32; d++) if (fabs(y[d]) > amax) amax = fabs(y[d]);
            s = orc_ue8m0_scale_fp4(amax);
            frexp(s, &e);                  /* s = 2^(e-1) */
            base[MX4_SCALE_OFF + (p % PAGE) * 4 + b] = (uint8_t)(e - 1 + 127);
            for (d = 32 * b; d < 32 * b + 32; d += 2) {
                uint8_t lo = orc_fp4_encode(y[d] / s), hi = orc_fp4_encode(y[d + 1] / s);
                codes[d / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/* The indexer score against an MXFP4 cache: as orc_indexer_logits, with each key dim
 * dequantised as its 4-bit code times its block's scale. */
void orc_indexer_logits_mxfp4(const uint8_t* q_fp8, const float* q_scale, const float* w,
                              const int32_t* req, const int32_t* pos, int64_t R,
                              const int32_t* page_table, int64_t pt_stride, const uint8_t* cache,
                              float* logits, int64_t stride) {
    double tab[256];
    int64_t r;
    int c;
    for (c = 0; c < 256; c++) tab[c] = orc_fp8_decode((uint8_t)c);
    for (r = 0; r < R; r++) {
        double q[IDX_HEADS][IDX_DIM];
        int64_t p = pos[r], s;
        int h, d;
        for (h = 0; h < IDX_HEADS; h++)
            for (d = 0; d < IDX_DIM; d++)
                q[h][d] = tab[q_fp8[(r * IDX_HEADS + h) * IDX_DIM + d]] * (double)q_scale[r * IDX_HEADS + h];
#pragma omp parallel for schedule(static)
        for (s = 0; s < stride; s++) {
            const uint8_t* page;
            const uint8_t* key;
            double k[IDX_DIM], acc = 0.0;
            int hh, dd;
            if (p < 0 || s > p) { logits[r * stride + s] = -INFINITY; continue; }
            page = cache + page_of(page_table, pt_stride, req[r], s) * MX4_PAGE_B;
            key = page + (s % PAGE) * MX4_TOKEN_B;
            for (dd = 0; dd < IDX_DIM; dd++) {
                uint8_t code = (uint8_t)((key[dd / 2] >> (4 * (dd & 1))) & 0xF);
                double sc = ldexp(1.0, (int)page[MX4_SCALE_OFF + (s % PAGE) * 4 + dd / 32] - 127);
                k[dd] = orc_fp4_decode(code) * sc;
            }
            for (hh = 0; hh < IDX_HEADS; hh++) {
                double dot = 0.0;
                for (dd = 0; dd < IDX_DIM; dd++) dot += q[hh][dd] * k[dd];
                acc += (double)w[r * IDX_HEADS + hh] * (dot > 0.0 ? dot : 0.0);
            }
            logits[r * stride + s] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------ array helpers (for tests) */
void orc_fp8_encode_array(const double* x, int64_t n, uint8_t* out, int brute) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; i++) out[i] = brute ? orc_fp8_encode_bruteforce(x[i]) : orc_fp8_encode(x[i]);
}

void orc_fp8_decode_array(const uint8_t* c, int64_t n, double* out) {
    int64_t i;
    for (i = 0; i < n; i++) out[i] = orc_fp8_decode(c[i]);
}

void orc_bf16_from_double_array(const double* x, int64_t n, uint16_t* out) {
    int64_t i;
    for (i = 0; i < n; i++) out[i] = orc_double_to_bf16(x[i]);
}

void orc_ue8m0_array(const double* amax, int64_t n, double* out) {
    int64_t i;
    for (i = 0; i < n; i++) out[i] = orc_ue8m0_scale(amax[i]);
}

void orc_ln_rope_array(const double* x, const int64_t* pos, int64_t n, double eps, double theta,
                       int do_ln, int inverse, double* out) {
    int64_t t;
    for (t = 0; t < n; t++) {
        int d;
        if (do_ln) orc_layernorm128(x + t * 128, out + t * 128, eps);
        else for (d = 0; d < 128; d++) out[t * 128 + d] = x[t * 128 + d];
        orc_rope64(out + t * 128, pos[t], theta, inverse);
    }
}

void orc_fp4_encode_array(const double* x, int64_t n, uint8_t* out, int brute) {
    int64_t i;
    for (i = 0; i < n; i++) out[i] = brute ? orc_fp4_encode_bruteforce(x[i]) : orc_fp4_encode(x[i]);
}

void orc_fp4_decode_array(const uint8_t* c, int64_t n, double* out) {
    int64_t i;
    for (i = 0; i < n; i++) out[i] = orc_fp4_decode(c[i]);
}

void orc_ue8m0_fp4_array(const double* amax, int64_t n, double* out) {
    int64_t i;
    for (i = 0; i < n; i++) out[i] = orc_ue8m0_scale_fp4(amax[i]);
}
