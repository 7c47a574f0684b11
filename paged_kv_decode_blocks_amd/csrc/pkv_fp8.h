// pkv_fp8.h -- device helpers for the FP8 K/V cache (internal to libpkv).
//
// Format: OCP E4M3 codes (bias 7, no infinities, S.1111.111 = NaN, largest
// finite 448), the 8-bit float gfx950 converts in hardware, with one
// power-of-two scale per token row and KV head.  A row x is stored as
//   E = max(floor(log2 max|x|) - 8, -126)  (0 for an all-zero row),
//   scale = 2^E, code_d = nearest E4M3 value to x_d / scale (ties to even,
//   magnitudes above 448 clamped), sign kept,
// so a row is quantized on its own when it is appended, and both x / scale
// and code * scale are exact: the only rounding is to the E4M3 grid.
#pragma once

#include "pkv_device.h"

namespace pkv {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// 16 codes (one 16-byte lane vector) -> 16 floats.
__device__ __forceinline__ void fp8x16_to_f32(const uint4& v, float (&f)[16]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);   // bytes 0, 1
        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);    // bytes 2, 3
        f[4 * i] = lo[0];
        f[4 * i + 1] = lo[1];
        f[4 * i + 2] = hi[0];
        f[4 * i + 3] = hi[1];
    }
}

// sum_i q[i] * value(code_i), float32
__device__ __forceinline__ float dot_fp8x16(const float (&q)[16], const uint4& k) {
    float f[16];
    fp8x16_to_f32(k, f);
    float s = q[0] * f[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) s = fmaf(q[i], f[i], s);
    return s;
}

// o[0 .. 16) += p * value(code)
__device__ __forceinline__ void axpy_fp8x16(float* o, float p, const uint4& v) {
    float f[16];
    fp8x16_to_f32(v, f);
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = fmaf(p, f[e], o[e]);
}

// 16 consecutive elements of a row in storage dtype QDT -> floats (exact).
template <int QDT>
__device__ __forceinline__ void load16_f32(const char* p, float (&f)[16]) {
    if constexpr (QDT == DT_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 u = ld16_cached(p + 16 * i);
            f[4 * i] = __uint_as_float(u.x);
            f[4 * i + 1] = __uint_as_float(u.y);
            f[4 * i + 2] = __uint_as_float(u.z);
            f[4 * i + 3] = __uint_as_float(u.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 u = ld16_cached(p + 16 * i);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (QDT == DT_F16) {
                    const half2_t h = __builtin_bit_cast(half2_t, w[j]);
                    f[8 * i + 2 * j] = (float)h.x;
                    f[8 * i + 2 * j + 1] = (float)h.y;
                } else {
                    f[8 * i + 2 * j] = bf16lo(w[j]);
                    f[8 * i + 2 * j + 1] = bf16hi(w[j]);
                }
            }
        }
    }
}

// Max over aligned groups of N lanes (N a power of two, 1..64); every lane gets it.
template <int N>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (N >= 2) v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp_f<kDppRowMirror>(v));
    if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
    if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

// 2^e as a float, e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// E of a row's scale from the row's largest magnitude (finite, >= 0).
__device__ __forceinline__ int fp8_row_exponent(float amax) {
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
    if (ef == 0) return amax == 0.0f ? 0 : -126;   // zero row, or a maximum below the normal range
    return max(ef - 127 - 8, -126);
}

// Nearest E4M3 code to v (|v| < 512), magnitudes above 448 clamped, ties to the
// even code, sign bit from v.  Below 2^-6 the grid step is 2^-9; above, a
// value a in [2^e, 2^(e+1)) has grid step 2^(e-3).  Both scalings by powers of
// two are exact, so rintf (round to nearest even) makes the only rounding, and
// an integer tie lands on an even integer, i.e. an even code.
__device__ __forceinline__ uint32_t fp8_encode(float v) {
    const float a = fminf(fabsf(v), 448.0f);
    uint32_t mag;
    if (a < 0.015625f) {
        mag = (uint32_t)__builtin_rintf(a * 512.0f);                     // 0 .. 8 (8 = 2^-6, code 0x08)
    } else {
        const int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;    // -6 .. 8
        const float t = a * pow2f(3 - e);                                  // [8, 16)
        mag = (uint32_t)((e + 7) * 8) + (uint32_t)__builtin_rintf(t) - 8u;   // 16 carries into the exponent
    }
    return mag | ((__float_as_uint(v) >> 24) & 0x80u);
}

}  // namespace pkv
