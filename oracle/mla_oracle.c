/*
 * CPU oracle for weight-absorbed MLA decode over a paged latent cache.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The product path never calls it.
 * It shares no code, header or table with the HIP library.
 *
 * Everything is computed in IEEE double from the exact input values: bfloat16
 * and fp8 e4m3fn codes are widened exactly. The softmax is materialised, as in
 * the plain "three kernel" form the FlashAttention paragraph of the SGLang
 * attention-backends page describes. No blocking, no online rescaling and no
 * fusion: one (query row, head) pair at a time.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_LATENT 512 /* kv_lora_rank: the part of each row that is also V */
#define ORACLE_ROPE 64    /* qk_rope_head_dim */
#define ORACLE_ROW (ORACLE_LATENT + ORACLE_ROPE)

enum { ORACLE_CACHE_BF16 = 0, ORACLE_CACHE_F64 = 1, ORACLE_CACHE_E4M3FN = 2 };

/* bfloat16: the upper 16 bits of an IEEE binary32. Widening is exact. */
double oracle_bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP fp8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; exponent 0 encodes subnormals m/8 * 2^-6. */
double oracle_e4m3fn_to_double(uint8_t code) {
    int sign = code >> 7;
    int exp = (code >> 3) & 0xF;
    int man = code & 0x7;
    double v;
    if (exp == 0xF && man == 0x7) return NAN;
    if (exp == 0)
        v = ldexp((double)man / 8.0, -6);
    else
        v = ldexp(1.0 + (double)man / 8.0, exp - 7);
    return sign ? -v : v;
}

void oracle_decode_elements(int32_t dtype, const void* src, int64_t n, double* dst) {
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == ORACLE_CACHE_BF16)
            dst[i] = oracle_bf16_to_double(((const uint16_t*)src)[i]);
        else if (dtype == ORACLE_CACHE_E4M3FN)
            dst[i] = oracle_e4m3fn_to_double(((const uint8_t*)src)[i]);
        else
            dst[i] = ((const double*)src)[i];
    }
}

static double cache_value(const void* cache, int32_t dtype, double kv_scale, int64_t row, int d) {
    int64_t i = row * ORACLE_ROW + d;
    if (dtype == ORACLE_CACHE_BF16) return oracle_bf16_to_double(((const uint16_t*)cache)[i]);
    if (dtype == ORACLE_CACHE_E4M3FN)
        return oracle_e4m3fn_to_double(((const uint8_t*)cache)[i]) * kv_scale;
    return ((const double*)cache)[i];
}

/* Tokens of request b: pages kv_indices[kv_indptr[b] .. kv_indptr[b+1]), every
 * page full except the last, which holds kv_last_page_len[b] tokens
 * ("Paged, ragged batches", SGLang attention-backends page). A NULL
 * kv_last_page_len means the last page is full. */
static int64_t request_len(int32_t b, int32_t page_size, const int32_t* kv_indptr,
                           const int32_t* kv_last_page_len) {
    int64_t np = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
    if (np <= 0) return 0;
    int64_t last = kv_last_page_len ? kv_last_page_len[b] : page_size;
    return (np - 1) * page_size + last;
}

/* Pool row that holds token t of request b: the page is kv_indices at the
 * request's offset plus t / page_size, the slot in the page is t % page_size. */
static int64_t token_row(int32_t b, int64_t t, int32_t page_size, const int32_t* kv_indptr,
                         const int32_t* kv_indices) {
    int64_t page = kv_indices[(int64_t)kv_indptr[b] + t / page_size];
    return page * page_size + t % page_size;
}

int32_t oracle_num_threads(void) {
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the next calls use (the CPU baseline times one core as well as all
 * of them). n <= 0 restores the OpenMP default. */
void oracle_set_num_threads(int32_t n) {
#ifdef _OPENMP
    static int32_t dflt = 0;
    if (dflt == 0) dflt = (int32_t)omp_get_max_threads();
    omp_set_num_threads(n > 0 ? n : dflt);
#else
    (void)n;
#endif
}

/*
 * Absorbed-MLA decode.
 *
 * For query row n of request b, head h, and each token t < L_b with cache row c_t:
 *   score:  s_t = sm_scale * ( sum_{d<512} q_nope[n,h,d] c_t[d] + sum_{d<64} q_rope[n,h,d] c_t[512+d] )
 *           (the two-path score of the tpu-inference MLA kernel core loop, section 2.4 of the
 *            sglang-jax MLA gap page; the absorbed query of section 2.1 there)
 *   softmax: m = max_t s_t, p_t = exp(s_t - m), l = sum_t p_t, P_t = p_t / l
 *   output: out[n,h,:] = sum_t P_t c_t[0:512]   (the latent is reused as the value: section 2.1
 *           and the MLA paragraph of the attention-backends page, 576 wide for k and 512 for v)
 *   lse:    lse[n,h] = m + ln l                  (natural log)
 * An empty request gives out = 0 and lse = -inf.
 *
 * q_nope [N,H,512] and q_rope [N,H,64] are doubles; cache rows are 576 values of
 * the given dtype; fp8 codes are multiplied by kv_scale. qo_indptr may be NULL
 * (one query row per request). out is [N,H,512] and lse is [N,H].
 * Returns 0, or -1 on a malformed layout.
 */
int32_t oracle_mla_decode(int32_t batch, int32_t num_heads, int32_t page_size,
                          const int32_t* qo_indptr, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_last_page_len,
                          const double* q_nope, const double* q_rope, const void* cache,
                          int32_t cache_dtype, double kv_scale, double sm_scale, double* out,
                          double* lse) {
    if (batch < 0 || num_heads <= 0 || page_size <= 0) return -1;
    int64_t num_rows = qo_indptr ? qo_indptr[batch] : batch;
    int64_t max_len = 0;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t L = request_len(b, page_size, kv_indptr, kv_last_page_len);
        if (L < 0) return -1;
        if (L > max_len) max_len = L;
    }
    /* Row n -> request b. */
    int32_t* row_req = (int32_t*)malloc(sizeof(int32_t) * (size_t)(num_rows > 0 ? num_rows : 1));
    if (!row_req) return -1;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t r0 = qo_indptr ? qo_indptr[b] : b, r1 = qo_indptr ? qo_indptr[b + 1] : b + 1;
        for (int64_t n = r0; n < r1; ++n) row_req[n] = b;
    }
    int64_t pairs = num_rows * num_heads;
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t pr = 0; pr < pairs; ++pr) {
            if (!s) continue;
            int64_t n = pr / num_heads;
            int32_t h = (int32_t)(pr % num_heads);
            int32_t b = row_req[n];
            int64_t L = request_len(b, page_size, kv_indptr, kv_last_page_len);
            const double* qa = q_nope + (n * num_heads + h) * ORACLE_LATENT;
            const double* qr = q_rope + (n * num_heads + h) * ORACLE_ROPE;
            double* o = out + (n * num_heads + h) * ORACLE_LATENT;
            for (int d = 0; d < ORACLE_LATENT; ++d) o[d] = 0.0;
            if (L == 0) {
                lse[n * num_heads + h] = -INFINITY;
                continue;
            }
            /* Scores. */
            for (int64_t t = 0; t < L; ++t) {
                int64_t row = token_row(b, t, page_size, kv_indptr, kv_indices);
                double nope = 0.0, rope = 0.0;
                for (int d = 0; d < ORACLE_LATENT; ++d)
                    nope += qa[d] * cache_value(cache, cache_dtype, kv_scale, row, d);
                for (int d = 0; d < ORACLE_ROPE; ++d)
                    rope += qr[d] * cache_value(cache, cache_dtype, kv_scale, row, ORACLE_LATENT + d);
                s[t] = (nope + rope) * sm_scale;
            }
            /* Softmax, materialised. */
            double m = s[0];
            for (int64_t t = 1; t < L; ++t)
                if (s[t] > m) m = s[t];
            double l = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                s[t] = exp(s[t] - m);
                l += s[t];
            }
            /* Output: probabilities times the latent part of each row. */
            for (int64_t t = 0; t < L; ++t) {
                int64_t row = token_row(b, t, page_size, kv_indptr, kv_indices);
                double P = s[t] / l;
                for (int d = 0; d < ORACLE_LATENT; ++d)
                    o[d] += P * cache_value(cache, cache_dtype, kv_scale, row, d);
            }
            lse[n * num_heads + h] = m + log(l);
        }
        free(s);
    }
    free(row_req);
    return failed ? -1 : 0;
}

/*
 * Merge of two attention states over disjoint token sets, each given as a
 * normalised output v and its log-sum-exp s (the cascade merge of the PR 49477
 * analysis, introduction; the Flash-Decoding rescaling of the attention-backends
 * page):  s = ln(e^{s_a} + e^{s_b}),  v = e^{s_a - s} v_a + e^{s_b - s} v_b.
 * A side with s = -inf holds no tokens and drops out; both empty gives v = 0,
 * s = -inf. Rows are [n, d] contiguous.
 */
void oracle_merge_states(int64_t n, int32_t d, const double* v_a, const double* s_a,
                         const double* v_b, const double* s_b, double* v_out, double* s_out) {
    for (int64_t i = 0; i < n; ++i) {
        double a = s_a[i], b = s_b[i];
        if (isinf(a) && a < 0 && isinf(b) && b < 0) {
            s_out[i] = -INFINITY;
            for (int32_t k = 0; k < d; ++k) v_out[i * d + k] = 0.0;
            continue;
        }
        double m = a > b ? a : b;
        double s = m + log(exp(a - m) + exp(b - m));
        double wa = exp(a - s), wb = exp(b - s);
        for (int32_t k = 0; k < d; ++k) v_out[i * d + k] = wa * v_a[i * d + k] + wb * v_b[i * d + k];
        s_out[i] = s;
    }
}
