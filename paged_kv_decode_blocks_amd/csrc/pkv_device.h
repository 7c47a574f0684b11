// pkv_device.h -- device helpers shared by the gfx950 kernels of libpkv.
//
// Storage types, 16-byte vector loads, wave64 DPP row reductions and the
// argument block every attention kernel takes.  Nothing here is used by the
// CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };   // storage dtypes of q, K/V and new rows

constexpr int kBlockSize = 16;   // tokens per physical KV block (the only size built)
constexpr int kGqaWindowTokens = 256 * kBlockSize;   // block ids a grouped workgroup stages in LDS at a time
constexpr int kGqaSpanTokens = 512 * kBlockSize;     // the same for the 16-bit grouped kernel with K in LDS
constexpr int kMhaWindowTokens = 256 * kBlockSize;   // the same for the per-head kernel
// Even split of a grouped batch (one run of blocks per wave, see decode_gqa.hip):
constexpr int kEvenMaxBatch = 1024;       // requests whose block counts a workgroup prefix-sums in LDS
constexpr int kEvenMaxWaveBlocks = 256;   // longest run of blocks one wave takes
constexpr int kEvenMinWaveBlocks = 16;    // shortest run worth a wave of its own (default)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -3.0e38f;   // "no score yet": exp2(kNegBig - m) == 0 for any real m

template <int DT> struct Dt;
template <> struct Dt<DT_F32>  { static constexpr int bytes = 4; };
template <> struct Dt<DT_F16>  { static constexpr int bytes = 2; };
template <> struct Dt<DT_BF16> { static constexpr int bytes = 2; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// 16-byte loads and stores.  KV rows are read exactly once per step, so the
// loads carry the non-temporal hint; they still go through the vector memory
// path (global_load_dwordx4).
// ---------------------------------------------------------------------------
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Work unit of workgroup `x` out of `units` (units numbered head-fastest), for
// the per-head FP8 kernel.  Workgroups are dealt to the 8 XCDs round-robin by
// index, so units 2k and 2k+1 -- KV heads 2k' and 2k'+1, whose 64-byte row-scale
// pieces share one 128-byte line -- would land on two XCDs and each fetch that
// line from HBM.  Within every full group of 16 indices, index 8m + j takes unit
// 2 (8 i + j) + m (i the group): a head pair shares an XCD and starts together.
// A bijection on [0, units); the last partial group keeps its order.  (Measured
// on the 16-bit kernels, which have no scale lines, it helped one workload and
// hurt another, so they keep the plain order.)
__device__ __forceinline__ int xcd_pair_unit(int x, int units) {
    if (x >= (units & ~15)) return x;
    const int r = x & 15;
    return ((x >> 4) * 8 + (r & 7)) * 2 + (r >> 3);
}

__device__ __forceinline__ uint4 ld16(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16_cached(const void* p) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void* p, const uint4& v) {
    *reinterpret_cast<u32x4_t*>(p) = u32x4_t{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ uint2 ld8(const void* p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st8(void* p, const uint2& v) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{v.x, v.y};
}

// ---------------------------------------------------------------------------
// Element conversion helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// dot product of the 16 bytes `k` with the 16 bytes `q` (same storage dtype),
// accumulated in float32.
template <int DT>
__device__ __forceinline__ float dot16(const uint4& q, const uint4& k);

template <>
__device__ __forceinline__ float dot16<DT_F32>(const uint4& q, const uint4& k) {
    float s = __uint_as_float(q.x) * __uint_as_float(k.x);
    s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
    s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
    s = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
    return s;
}

template <>
__device__ __forceinline__ float dot16<DT_F16>(const uint4& q, const uint4& k) {
    float s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.x), __builtin_bit_cast(half2_t, k.x), 0.0f, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.y), __builtin_bit_cast(half2_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.z), __builtin_bit_cast(half2_t, k.z), s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.w), __builtin_bit_cast(half2_t, k.w), s, false);
    return s;
}

template <>
__device__ __forceinline__ float dot16<DT_BF16>(const uint4& q, const uint4& k) {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.x), __builtin_bit_cast(bf162_t, k.x), 0.0f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.y), __builtin_bit_cast(bf162_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.z), __builtin_bit_cast(bf162_t, k.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.w), __builtin_bit_cast(bf162_t, k.w), s, false);
    return s;
}

// o[0 .. E) += p * v, v the 16 bytes of one row chunk (E = 16 / element bytes)
template <int DT>
__device__ __forceinline__ void axpy16(float* o, float p, const uint4& v);

template <>
__device__ __forceinline__ void axpy16<DT_F32>(float* o, float p, const uint4& v) {
    o[0] = fmaf(p, __uint_as_float(v.x), o[0]);
    o[1] = fmaf(p, __uint_as_float(v.y), o[1]);
    o[2] = fmaf(p, __uint_as_float(v.z), o[2]);
    o[3] = fmaf(p, __uint_as_float(v.w), o[3]);
}

template <>
__device__ __forceinline__ void axpy16<DT_F16>(float* o, float p, const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        half2_t h = __builtin_bit_cast(half2_t, w[i]);
        o[2 * i] = fmaf(p, (float)h.x, o[2 * i]);
        o[2 * i + 1] = fmaf(p, (float)h.y, o[2 * i + 1]);
    }
}

template <>
__device__ __forceinline__ void axpy16<DT_BF16>(float* o, float p, const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = fmaf(p, bf16lo(w[i]), o[2 * i]);
        o[2 * i + 1] = fmaf(p, bf16hi(w[i]), o[2 * i + 1]);
    }
}

// A product that is never fused into a following add: the scaled score s is
// used both for the running max m and in exp2(s - m), and s - m must be exactly
// 0 for the maximal token (so that a one-token context returns v bit for bit).
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
    return a * b;
}

// ---------------------------------------------------------------------------
// Cross-lane reductions.  Within a 16-lane row the butterfly uses DPP
// (quad_perm for distance 1 and 2, row_half_mirror and row_mirror to fold 8
// and 16 lanes); across rows it uses ds_swizzle/bpermute through __shfl_xor.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within each group of 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within each row of 16

// Sum over aligned groups of N lanes (N a power of two, 1..64); every lane of
// the group gets the total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp_f<kDppQuadXor1>(v);
    if constexpr (N >= 4) v += dpp_f<kDppQuadXor2>(v);
    if constexpr (N >= 8) v += dpp_f<kDppRowHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_f<kDppRowMirror>(v);
    if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (N >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// ---------------------------------------------------------------------------
// Arguments shared by every attention kernel (passed by value).
// ---------------------------------------------------------------------------
struct AttnArgs {
    float* out;             // [B][H_q][D]
    float* part_o;          // [B][H_q][n_parts][D]   (split only)
    float* part_lse;        // [B][H_q][n_parts]      (split only; log2 domain)
    const char* q;          // [B][H_q][D] storage dtype, rows q_row_stride elements apart
    const char* k_pool;     // [n_blocks][H_kv][16][D]
    const char* v_pool;
    char* k_pool_w;         // same pools, written by the fused append
    char* v_pool_w;
    const int32_t* block_tables;
    const int32_t* context_lens;   // attention lengths (plain call)
    const int32_t* positions;      // appended slot (fused call); n = positions + 1
    const char* k_new;             // [B][H_kv][D] (fused call)
    const char* v_new;
    const float* k_scale;          // FP8 pools only: [n_blocks][H_kv][16] per-row scales
    const float* v_scale;
    float* k_scale_w;              // same, written by the fused FP8 append
    float* v_scale_w;
    const uint8_t* k_mx_scale;     // MXFP4 pools only: [n_blocks][H_kv][16][D/32] E8M0 scale bytes
    const uint8_t* v_mx_scale;
    uint8_t* k_mx_scale_w;         // same, written by the fused MXFP4 append
    uint8_t* v_mx_scale_w;
    int64_t q_row_stride;          // elements
    int64_t new_row_stride;        // elements
    int32_t bt_stride;
    int32_t B, H_q, H_kv, G;
    int32_t n_blocks;
    int32_t max_context_len;
    int32_t part_tokens;           // tokens per workgroup span (whole padded context when not split)
    int32_t n_parts;               // spans per (request, head); 1 = no split
    int32_t wave_tokens;           // grouped kernel: 0 = the waves share the span's chunks round-robin;
                                   // > 0 = the span is part_tokens / wave_tokens partitions of this many
                                   // tokens and wave w streams partition w alone
    int32_t part_rev;              // split kernels: 1 = deal partitions from the last to the first
    int32_t even_waves;            // grouped kernel with K in LDS: > 0 = even split over at most this many
                                   // waves (part_o / part_lse then hold one row per piece and head)
    int32_t* even_meta;            // even split: [0] blocks per workgroup's super-run, [1] runs used,
                                   // [2 + b] blocks of requests 0 .. b-1 (b = 0 .. B)
    int32_t even_min_run;          // even split: shortest run worth a wave of its own (blocks)
    float scale_log2;              // scale * log2(e)
};

// Partition of the p-th group of work units (units are numbered partition-major, so the
// dispatcher starts them in that order).  With part_rev the last partitions -- present only
// for the longest requests -- start first and every request's first partitions end the
// launch, so its final round is the batch's densest set of equal units.
__device__ __forceinline__ int unit_part(const AttnArgs& a, int p) { return a.part_rev ? a.n_parts - 1 - p : p; }

}  // namespace pkv
