// pkv_mxfp4.h -- device helpers for the MXFP4 K/V cache.
//
// A low-precision cache stores K/V in a few bits with fine-grained block scales
// ("从 PagedAttention 到 Prefill-Decode 分离的深度解析", section 6.2).  This one
// follows the OCP microscaling format MXFP4: every 32 consecutive elements of a
// row share one E8M0 scale (a power of two, 2^(s - 127)), each element is an
// E2M1 code (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), packed two per byte with
// element 2k in the low nibble of byte k.  For a block with largest magnitude
// amax the scale exponent is E = floor(log2 amax) - 2 (E2M1's largest value is
// 1.5 * 2^2), clamped to [-127, 127], -127 for an all-zero block; codes are the
// nearest grid value to x / 2^E, ties to the even code, saturating at 6.
//
// gfx950 decodes codes in hardware: v_cvt_scalef32_pk_f32_fp4 turns byte `sel`
// of a word into two floats (low nibble first) multiplied by 2^(exponent field
// of its f32 scale operand) -- exact for every E8M0 scale (checked over all
// codes and the extreme scales on the GPU).
#pragma once
#include "pkv_fp8.h"

namespace pkv {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// E8M0 scale byte -> the f32 operand whose exponent field the conversion uses
// (2^-127 as the denormal 0x00400000; 255, NaN in E8M0, gives +inf).
__device__ __forceinline__ float mx_scale_operand(uint32_t s) {
    return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// 8 codes of word w -> f[0 .. 8), each times 2^E of the scale operand (exact).
__device__ __forceinline__ void e2m1x8_to_f32(uint32_t w, float sc, float* f) {
    const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
    const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
    const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
    const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
    f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
    f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

// Scale exponent of a block from its largest magnitude (finite, >= 0): a
// maximum below the normal range (or zero) gives the smallest, -127.
__device__ __forceinline__ int mx_block_exponent(float amax) {
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
    return ef == 0 ? -127 : max(ef - 127 - 2, -127);
}

// Nearest E2M1 code to v (already divided by 2^E), ties to the even code,
// magnitudes above 6 saturating; the sign bit from v.  Each comparison counts a
// grid midpoint below |v|; at a midpoint between an even and an odd code the
// strict test keeps the even one, the non-strict test moves to the even one.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
    const float a = fabsf(v);
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// One row quantized by one wave: lane l holds elements 2l and 2l + 1 (zeros for
// lanes >= D/2); returns the lane's code byte and, in E, its 32-element block's
// scale exponent (the block's max from a 16-lane reduction).
__device__ __forceinline__ uint32_t mx4_quantize_pair(float x0, float x1, int& E) {
    const float amax = group_max<16>(fmaxf(fabsf(x0), fabsf(x1)));
    E = mx_block_exponent(amax);
    // 2^-E as a float: -E in [-125, 127]
    const float inv = __uint_as_float((uint32_t)(127 - E) << 23);
    return e2m1_encode(x0 * inv) | (e2m1_encode(x1 * inv) << 4);
}

}  // namespace pkv
