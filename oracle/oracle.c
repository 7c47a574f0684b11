/*
 * oracle.c -- plain, slow, fp64 CPU reference for one paged-KV decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the tests, the smoke check and the bench's CPU
 * baseline do.  It shares no code, header, table or helper with the HIP
 * library: it decodes f16/bf16 bit patterns itself and walks the page table
 * itself.
 *
 * What it computes (one decode step of one attention layer):
 *
 *  - Each decode request contributes exactly one new query token per head and
 *    reads all of its K/V history ("Disaggregated LLM Serving：从 PD 分离到
 *    Attention 卸载", section 1 and section 2.1: a decode step both reads the
 *    existing KV cache and appends the new token's KV; each decode request
 *    brings one query token).
 *  - The history is found through the request's own page table: logical token
 *    t lives in physical block table[t / block_size] at slot t % block_size,
 *    and blocks need not be contiguous ("从 PagedAttention 到 Prefill-Decode
 *    分离的深度解析", section 2.2, steps one and two).
 *  - The attention itself is never written out on the pages; we take the
 *    textbook scaled-dot-product softmax attention of the one query over all n
 *    history tokens, with `scale` passed in (1/sqrt(D) in every workload), and
 *    query head h reading KV head h / (H_q / H_kv) (contiguous grouping).
 *  - The new token's K/V are written into the block and slot its position maps
 *    to ("从 PagedAttention 到 Prefill-Decode 分离的深度解析", section 2.2,
 *    step three: blocks are handed out as new tokens need them; the caller has
 *    already placed that block in the table).
 *
 * Pool layout: k_pool / v_pool are [n_blocks][H_kv][block_size][D] in the
 * storage dtype; q is [B][H_q][D] with a row stride (elements) between
 * requests; block tables are [B][bt_stride] int32.
 *
 * Every function validates what it reads and returns a negative code instead
 * of reading out of bounds.
 *
 * Pins: tests/test_oracle.py checks this file against torch's
 * scaled_dot_product_attention in float64 on contiguous inputs, exhaustive
 * f16/bf16 decoding against numpy/torch, closed forms (one token, equal V rows,
 * zero query), invariance under block relocation, and the log-sum-exp merge
 * identity on sub-ranges.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_OK = 0, ORC_ERR_ARG = -1, ORC_ERR_RANGE = -2, ORC_ERR_NOMEM = -3 };

static int elem_size(int dtype) {
    switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    default: return 0;
    }
}

/* IEEE 754 binary16 -> double, written from the format's definition. */
static double half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (ex == 0) {
        v = ldexp((double)man, -24);                 /* zero or subnormal */
    } else if (ex == 31) {
        v = man ? NAN : INFINITY;
    } else {
        v = ldexp((double)(man + 1024), ex - 25);    /* 1.man * 2^(ex-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 is the top half of a binary32. */
static double bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(int dtype, const void* base, int64_t i) {
    switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[i];
    case ORC_F16: return half_to_double(((const uint16_t*)base)[i]);
    default: return bf16_to_double(((const uint16_t*)base)[i]);
    }
}

/* Decode n storage elements to double (exposed so the tests can pin the decoders). */
int oracle_decode(int dtype, const void* src, double* dst, int64_t n) {
    if (!elem_size(dtype) || (!src && n) || (!dst && n) || n < 0) return ORC_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(dtype, src, i);
    return ORC_OK;
}

/*
 * Append: for every request b, copy the bits of k_new[b][g][:] and
 * v_new[b][g][:] (all KV heads g) into slot positions[b] % block_size of
 * physical block block_tables[b][positions[b] / block_size].
 */
int oracle_kv_append(int dtype, const void* k_new, const void* v_new, int64_t new_row_stride,
                     void* k_pool, void* v_pool, const int32_t* block_tables, int32_t bt_stride,
                     const int32_t* positions, int32_t B, int32_t H_kv, int32_t D,
                     int32_t block_size, int32_t n_blocks) {
    int e = elem_size(dtype);
    if (!e || B < 0 || H_kv <= 0 || D <= 0 || block_size <= 0 || n_blocks <= 0 || bt_stride <= 0)
        return ORC_ERR_ARG;
    if (B == 0) return ORC_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !positions) return ORC_ERR_ARG;
    if (new_row_stride < (int64_t)H_kv * D) return ORC_ERR_ARG;
    /* validate every target before writing anything */
    for (int32_t b = 0; b < B; ++b) {
        int32_t p = positions[b];
        if (p < 0 || p / block_size >= bt_stride) return ORC_ERR_RANGE;
        int32_t blk = block_tables[(int64_t)b * bt_stride + p / block_size];
        if (blk < 0 || blk >= n_blocks) return ORC_ERR_RANGE;
    }
    size_t row_bytes = (size_t)D * (size_t)e;
    for (int32_t b = 0; b < B; ++b) {
        int32_t p = positions[b];
        int32_t blk = block_tables[(int64_t)b * bt_stride + p / block_size];
        int32_t slot = p % block_size;
        for (int32_t g = 0; g < H_kv; ++g) {
            int64_t dst = (((int64_t)blk * H_kv + g) * block_size + slot) * D;
            int64_t src = (int64_t)b * new_row_stride + (int64_t)g * D;
            memcpy((char*)k_pool + dst * e, (const char*)k_new + src * e, row_bytes);
            memcpy((char*)v_pool + dst * e, (const char*)v_new + src * e, row_bytes);
        }
    }
    return ORC_OK;
}

/*
 * Attention of one decode query per (request, query head) over the request's
 * whole paged history:
 *   s_t   = scale * sum_d q[b][h][d] * K_t[d]          t = 0 .. n-1
 *   out   = sum_t softmax(s)_t * V_t
 * computed as exp(s_t - max s) / sum exp(s - max s), all in double.
 * n = context_lens[b]; n == 0 gives a zero row.  If lse is not NULL it receives
 * log(sum_t exp(s_t)) per (b, h) (-inf for n == 0).
 */
int oracle_paged_decode_attention(int dtype, double* out, double* lse,
                                  const void* q, int64_t q_row_stride,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, int32_t bt_stride,
                                  const int32_t* context_lens,
                                  int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                  int32_t block_size, int32_t n_blocks, float scale,
                                  int32_t nthreads) {
    if (!elem_size(dtype) || B < 0 || H_q <= 0 || H_kv <= 0 || D <= 0 || block_size <= 0 ||
        n_blocks <= 0 || bt_stride <= 0 || H_q % H_kv != 0)
        return ORC_ERR_ARG;
    if (B == 0) return ORC_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return ORC_ERR_ARG;
    if (q_row_stride < (int64_t)H_q * D) return ORC_ERR_ARG;
    int32_t max_n = 0;
    for (int32_t b = 0; b < B; ++b) {
        int32_t n = context_lens[b];
        if (n < 0 || (n > 0 && (n - 1) / block_size >= bt_stride)) return ORC_ERR_RANGE;
        for (int32_t j = 0; j * block_size < n; ++j) {
            int32_t blk = block_tables[(int64_t)b * bt_stride + j];
            if (blk < 0 || blk >= n_blocks) return ORC_ERR_RANGE;
        }
        if (n > max_n) max_n = n;
    }
    const int32_t G = H_q / H_kv;
    const int64_t pairs = (int64_t)B * H_q;
    int status = ORC_OK;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_n > 0 ? max_n : 1));
        double* qd = (double*)malloc(sizeof(double) * (size_t)D);
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        const int ok = (s && qd && acc);
        if (!ok) {
#pragma omp atomic write
            status = ORC_ERR_NOMEM;
        }
        /* every thread reaches the loop; one without buffers does no work */
#pragma omp for schedule(dynamic, 1)
        for (int64_t pr = 0; pr < pairs; ++pr) {
            if (ok) {
                int32_t b = (int32_t)(pr / H_q);
                int32_t h = (int32_t)(pr % H_q);
                int32_t g = h / G;
                int32_t n = context_lens[b];
                double* o = out + pr * D;
                if (n == 0) {
                    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
                    if (lse) lse[pr] = -INFINITY;
                    continue;   /* next (b, h) */
                }
                for (int32_t d = 0; d < D; ++d)
                    qd[d] = load_elem(dtype, q, (int64_t)b * q_row_stride + (int64_t)h * D + d);
                const int32_t* table = block_tables + (int64_t)b * bt_stride;
                /* scores */
                for (int32_t t = 0; t < n; ++t) {
                    int64_t row = (((int64_t)table[t / block_size] * H_kv + g) * block_size +
                                   t % block_size) * D;
                    double dot = 0.0;
                    for (int32_t d = 0; d < D; ++d) dot += qd[d] * load_elem(dtype, k_pool, row + d);
                    s[t] = (double)scale * dot;
                }
                /* softmax */
                double m = s[0];
                for (int32_t t = 1; t < n; ++t) if (s[t] > m) m = s[t];
                double l = 0.0;
                for (int32_t t = 0; t < n; ++t) { s[t] = exp(s[t] - m); l += s[t]; }
                /* weighted sum of V */
                for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
                for (int32_t t = 0; t < n; ++t) {
                    int64_t row = (((int64_t)table[t / block_size] * H_kv + g) * block_size +
                                   t % block_size) * D;
                    for (int32_t d = 0; d < D; ++d) acc[d] += s[t] * load_elem(dtype, v_pool, row + d);
                }
                for (int32_t d = 0; d < D; ++d) o[d] = acc[d] / l;
                if (lse) lse[pr] = m + log(l);
            }
        }
        free(s);
        free(qd);
        free(acc);
    }
    return status;
}

/* Threads an OpenMP parallel region gets with the given request (0 = default). */
int oracle_threads(int32_t nthreads) {
#ifdef _OPENMP
    int got = 1;
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
    {
#pragma omp single
        got = omp_get_num_threads();
    }
    return got;
#else
    (void)nthreads;
    return 1;
#endif
}
