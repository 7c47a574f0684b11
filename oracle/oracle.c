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
enum { ORC_OK = 0, ORC_ERR_ARG = -1, ORC_ERR_RANGE = -2, ORC_ERR_NOMEM = -3, ORC_ERR_ALIAS = -4 };

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

static int cmp_i64(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/*
 * The requests of one append step write distinct slots: each new token is given a
 * slot of its own ("从 PagedAttention 到 Prefill-Decode 分离的深度解析", section
 * 2.2, step three), so two requests naming the same (block, slot) is an error and
 * nothing is written.  Targets are range-checked before this is called.
 */
static int check_distinct_targets(const int32_t* block_tables, int32_t bt_stride, const int32_t* positions,
                                  int32_t B, int32_t block_size) {
    int64_t* key = (int64_t*)malloc((size_t)B * sizeof(int64_t));
    if (!key) return ORC_ERR_NOMEM;
    for (int32_t b = 0; b < B; ++b) {
        int32_t p = positions[b];
        int32_t blk = block_tables[(int64_t)b * bt_stride + p / block_size];
        key[b] = (int64_t)blk * block_size + p % block_size;
    }
    qsort(key, (size_t)B, sizeof(int64_t), cmp_i64);
    int rc = ORC_OK;
    for (int32_t b = 1; b < B; ++b)
        if (key[b] == key[b - 1]) rc = ORC_ERR_ALIAS;
    free(key);
    return rc;
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
    int rc_alias = check_distinct_targets(block_tables, bt_stride, positions, B, block_size);
    if (rc_alias != ORC_OK) return rc_alias;
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

/*
 * ---------------------------------------------------------------------------
 * FP8 K/V cache
 * ---------------------------------------------------------------------------
 * "从 PagedAttention 到 Prefill-Decode 分离的深度解析", section 6.2: a
 * low-precision KV cache stores K/V in a few bits with fine-grained block
 * scales and dequantizes them before attention.  Reading taken here (the page
 * gives no layout): 8-bit OCP E4M3 codes (sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, S.1111.111 = NaN, largest finite 448; the
 * format gfx950 decodes in hardware), with one power-of-two scale per token row
 * and KV head, so that each appended row is quantized on its own:
 *   amax  = max_d |x_d|                       (x the row in its source dtype)
 *   E     = max(floor(log2 amax) - 8, -126)   (E = 0 when amax = 0)
 *   scale = 2^E                               (so amax / scale lies in [256, 512))
 *   code  = the E4M3 value nearest to x_d / scale, magnitudes above 448 taken
 *           as 448, ties to the even code; the sign bit is the sign of x_d
 * and the dequantized value is value(code) * scale (exact in double and f32).
 * Dividing by a power of two is exact, so the only rounding is the one to the
 * E4M3 grid, done here by searching the grid.
 */

/* OCP E4M3 code -> double, from the format's definition. */
static double e4m3_value(uint8_t c) {
    int sign = (c >> 7) & 1;
    int ex = (c >> 3) & 15;
    int man = c & 7;
    double v;
    if (ex == 15 && man == 7) return NAN;
    if (ex == 0) v = ldexp((double)man, -9);              /* zero or subnormal: man/8 * 2^-6 */
    else v = ldexp(1.0 + man / 8.0, ex - 7);
    return sign ? -v : v;
}

int oracle_e4m3_decode(const uint8_t* codes, double* dst, int64_t n) {
    if (n < 0 || (n && (!codes || !dst))) return ORC_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) dst[i] = e4m3_value(codes[i]);
    return ORC_OK;
}

/* The non-negative code (0x00 .. 0x7E) whose value is nearest to a, 0 <= a; ties to the even code. */
static uint8_t e4m3_nearest_magnitude(double a) {
    if (a > 448.0) a = 448.0;
    int best = 0;
    double best_err = fabs(a - e4m3_value(0));
    for (int c = 1; c <= 0x7E; ++c) {
        double err = fabs(a - e4m3_value((uint8_t)c));
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)best;
}

/* Quantize one row of D source elements: codes[0 .. D) and its scale. */
int oracle_e4m3_quantize_row(int src_dtype, const void* src, int32_t D, uint8_t* codes, float* scale) {
    if (!elem_size(src_dtype) || D <= 0 || !src || !codes || !scale) return ORC_ERR_ARG;
    double amax = 0.0;
    for (int32_t d = 0; d < D; ++d) {
        double x = load_elem(src_dtype, src, d);
        if (!isfinite(x)) return ORC_ERR_RANGE;
        if (fabs(x) > amax) amax = fabs(x);
    }
    int E = 0;
    if (amax > 0.0) {
        int e2;
        frexp(amax, &e2);               /* amax = f * 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
        E = e2 - 1 - 8;
        if (E < -126) E = -126;
    }
    const double s = ldexp(1.0, E);
    for (int32_t d = 0; d < D; ++d) {
        double v = load_elem(src_dtype, src, d) / s;
        uint8_t mag = e4m3_nearest_magnitude(fabs(v));
        codes[d] = (uint8_t)(signbit(v) ? (mag | 0x80) : mag);
    }
    *scale = (float)s;
    return ORC_OK;
}

/*
 * FP8 append: quantize k_new[b][g][:] and v_new[b][g][:] (source dtype) and
 * write the codes to slot positions[b] % block_size of block
 * block_tables[b][positions[b] / block_size], the scales to the same
 * (block, head, slot) of k_scale / v_scale ([n_blocks][H_kv][block_size] f32).
 */
int oracle_kv_append_fp8(int src_dtype, const void* k_new, const void* v_new, int64_t new_row_stride,
                         uint8_t* k_pool, uint8_t* v_pool, float* k_scale, float* v_scale,
                         const int32_t* block_tables, int32_t bt_stride, const int32_t* positions,
                         int32_t B, int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks) {
    int e = elem_size(src_dtype);
    if (!e || B < 0 || H_kv <= 0 || D <= 0 || block_size <= 0 || n_blocks <= 0 || bt_stride <= 0)
        return ORC_ERR_ARG;
    if (B == 0) return ORC_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !k_scale || !v_scale || !block_tables || !positions)
        return ORC_ERR_ARG;
    if (new_row_stride < (int64_t)H_kv * D) return ORC_ERR_ARG;
    for (int32_t b = 0; b < B; ++b) {
        int32_t p = positions[b];
        if (p < 0 || p / block_size >= bt_stride) return ORC_ERR_RANGE;
        int32_t blk = block_tables[(int64_t)b * bt_stride + p / block_size];
        if (blk < 0 || blk >= n_blocks) return ORC_ERR_RANGE;
    }
    int rc_alias = check_distinct_targets(block_tables, bt_stride, positions, B, block_size);
    if (rc_alias != ORC_OK) return rc_alias;
    for (int32_t b = 0; b < B; ++b) {
        int32_t p = positions[b];
        int32_t blk = block_tables[(int64_t)b * bt_stride + p / block_size];
        int32_t slot = p % block_size;
        for (int32_t g = 0; g < H_kv; ++g) {
            int64_t row = ((int64_t)blk * H_kv + g) * block_size + slot;
            const char* ks = (const char*)k_new + ((int64_t)b * new_row_stride + (int64_t)g * D) * e;
            const char* vs = (const char*)v_new + ((int64_t)b * new_row_stride + (int64_t)g * D) * e;
            int st = oracle_e4m3_quantize_row(src_dtype, ks, D, k_pool + row * D, k_scale + row);
            if (st == ORC_OK) st = oracle_e4m3_quantize_row(src_dtype, vs, D, v_pool + row * D, v_scale + row);
            if (st != ORC_OK) return st;
        }
    }
    return ORC_OK;
}

/*
 * Dequantize n_rows rows of D codes with one scale per row into float32:
 * dst[r][d] = value(codes[r][d]) * scale[r] (exact for every finite code and
 * power-of-two scale >= 2^-126).  The FP8 attention is the float32 attention
 * above on pools dequantized this way.
 */
int oracle_e4m3_dequantize_rows(const uint8_t* codes, const float* scale, int64_t n_rows, int32_t D, float* dst) {
    if (n_rows < 0 || D <= 0 || (n_rows && (!codes || !scale || !dst))) return ORC_ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int32_t d = 0; d < D; ++d)
            dst[r * D + d] = (float)(e4m3_value(codes[r * D + d]) * (double)scale[r]);
    return ORC_OK;
}

/*
 * ---------------------------------------------------------------------------
 * MXFP4 K/V cache
 * ---------------------------------------------------------------------------
 * The same page, section 6.2, names a 4-bit KV cache with fine-grained block
 * scales.  Reading taken here: the OCP microscaling format MXFP4 (OCP
 * Microscaling Formats (MX) Specification v1.0, section 5: a block of 32
 * elements shares one scale).  Elements are E2M1 codes (sign, 2 exponent bits
 * with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no
 * infinity or NaN); the shared scale is E8M0 (an 8-bit biased exponent, value
 * 2^(s - 127), s = 255 is NaN).  Per block of 32 consecutive elements of a row:
 *   amax = max_i |x_i|                    (x in its source dtype)
 *   E    = floor(log2 amax) - 2           (2: the exponent of E2M1's largest
 *          value 6 = 1.5 * 2^2), clamped to [-127, 127]; E = -127 when amax = 0
 *   code = the E2M1 value nearest to x_i / 2^E, magnitudes above 6 taken as 6,
 *          ties to the even code; the sign bit is the sign of x_i
 *   s    = E + 127
 * and the dequantized value is value(code) * 2^E (exact in double and in f32
 * for every E a finite f32 input produces).  Dividing by 2^E is exact for the
 * E range used here, so the only rounding is the one to the E2M1 grid, done
 * here by searching the grid.  Storage: codes two per byte, element 2k in the
 * low nibble of byte k; one scale byte per block of 32.
 */

static double e2m1_value(uint8_t c) {
    int sign = (c >> 3) & 1;
    int ex = (c >> 1) & 3;
    int man = c & 1;
    double v = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
    return sign ? -v : v;
}

static double e8m0_value(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

/* packed MXFP4 codes (n elements, two per byte) -> doubles, unscaled */
int oracle_e2m1_decode(const uint8_t* packed, double* dst, int64_t n) {
    if (n < 0 || (n & 1) || (n && (!packed || !dst))) return ORC_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) dst[i] = e2m1_value((uint8_t)((packed[i >> 1] >> (4 * (i & 1))) & 15));
    return ORC_OK;
}

/* The non-negative code (0 .. 7) whose value is nearest to a, 0 <= a; ties to the even code. */
static uint8_t e2m1_nearest_magnitude(double a) {
    if (a > 6.0) a = 6.0;
    int best = 0;
    double best_err = fabs(a - e2m1_value(0));
    for (int c = 1; c <= 7; ++c) {
        double err = fabs(a - e2m1_value((uint8_t)c));
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)best;
}

/* Quantize one row of D source elements (D a multiple of 32): codes[0 .. D/2), scales[0 .. D/32). */
int oracle_mxfp4_quantize_row(int src_dtype, const void* src, int32_t D, uint8_t* codes, uint8_t* scales) {
    if (!elem_size(src_dtype) || D <= 0 || D % 32 || !src || !codes || !scales) return ORC_ERR_ARG;
    for (int32_t d = 0; d < D; ++d)
        if (!isfinite(load_elem(src_dtype, src, d))) return ORC_ERR_RANGE;
    for (int32_t blk = 0; blk < D / 32; ++blk) {
        double amax = 0.0;
        for (int32_t i = 0; i < 32; ++i) {
            double x = fabs(load_elem(src_dtype, src, blk * 32 + i));
            if (x > amax) amax = x;
        }
        int E = -127;
        if (amax > 0.0) {
            int e2;
            frexp(amax, &e2);               /* amax = f * 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
            E = e2 - 1 - 2;
            if (E < -127) E = -127;
            if (E > 127) E = 127;
        }
        for (int32_t i = 0; i < 32; ++i) {
            const int32_t d = blk * 32 + i;
            double v = ldexp(load_elem(src_dtype, src, d), -E);
            uint8_t c = e2m1_nearest_magnitude(fabs(v));
            if (signbit(v)) c |= 8;
            if (i & 1) codes[d >> 1] = (uint8_t)((codes[d >> 1] & 0x0F) | (c << 4));
            else codes[d >> 1] = c;
        }
        scales[blk] = (uint8_t)(E + 127);
    }
    return ORC_OK;
}

/*
 * MXFP4 append: quantize k_new[b][g][:] and v_new[b][g][:] into slot
 * positions[b] % block_size of block block_tables[b][positions[b] / block_size]:
 * codes into k_pool / v_pool ([n_blocks][H_kv][block_size][D/2] bytes), scales
 * into k_scale / v_scale ([n_blocks][H_kv][block_size][D/32] bytes).
 */
int oracle_kv_append_mxfp4(int src_dtype, const void* k_new, const void* v_new, int64_t new_row_stride,
                           uint8_t* k_pool, uint8_t* v_pool, uint8_t* k_scale, uint8_t* v_scale,
                           const int32_t* block_tables, int32_t bt_stride, const int32_t* positions,
                           int32_t B, int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks) {
    int e = elem_size(src_dtype);
    if (!e || B < 0 || H_kv <= 0 || D <= 0 || D % 32 || block_size <= 0 || n_blocks <= 0 || bt_stride <= 0)
        return ORC_ERR_ARG;
    if (B == 0) return ORC_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !k_scale || !v_scale || !block_tables || !positions)
        return ORC_ERR_ARG;
    if (new_row_stride < (int64_t)H_kv * D) return ORC_ERR_ARG;
    for (int32_t b = 0; b < B; ++b) {
        int32_t p = positions[b];
        if (p < 0 || p / block_size >= bt_stride) return ORC_ERR_RANGE;
        int32_t blk = block_tables[(int64_t)b * bt_stride + p / block_size];
        if (blk < 0 || blk >= n_blocks) return ORC_ERR_RANGE;
    }
    int rc_alias = check_distinct_targets(block_tables, bt_stride, positions, B, block_size);
    if (rc_alias != ORC_OK) return rc_alias;
    for (int32_t b = 0; b < B; ++b) {
        int32_t p = positions[b];
        int32_t blk = block_tables[(int64_t)b * bt_stride + p / block_size];
        int32_t slot = p % block_size;
        for (int32_t g = 0; g < H_kv; ++g) {
            int64_t row = ((int64_t)blk * H_kv + g) * block_size + slot;
            const char* ks = (const char*)k_new + ((int64_t)b * new_row_stride + (int64_t)g * D) * e;
            const char* vs = (const char*)v_new + ((int64_t)b * new_row_stride + (int64_t)g * D) * e;
            int st = oracle_mxfp4_quantize_row(src_dtype, ks, D, k_pool + row * (D / 2), k_scale + row * (D / 32));
            if (st == ORC_OK)
                st = oracle_mxfp4_quantize_row(src_dtype, vs, D, v_pool + row * (D / 2), v_scale + row * (D / 32));
            if (st != ORC_OK) return st;
        }
    }
    return ORC_OK;
}

/*
 * Dequantize n_rows rows of D elements into float32: dst[r][d] =
 * value(code of element d of row r) * 2^(scale byte of its block - 127) (exact;
 * NaN where the scale byte is 255).  The MXFP4 attention is the float32
 * attention above on pools dequantized this way.
 */
int oracle_mxfp4_dequantize_rows(const uint8_t* codes, const uint8_t* scales, int64_t n_rows, int32_t D,
                                 float* dst) {
    if (n_rows < 0 || D <= 0 || D % 32 || (n_rows && (!codes || !scales || !dst))) return ORC_ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int32_t d = 0; d < D; ++d) {
            const uint8_t c = (uint8_t)((codes[r * (D / 2) + (d >> 1)] >> (4 * (d & 1))) & 15);
            dst[r * D + d] = (float)(e2m1_value(c) * e8m0_value(scales[r * (D / 32) + d / 32]));
        }
    return ORC_OK;
}
