// decode_mxfp4.hip -- paged decode attention over an MXFP4 K/V cache, one query
// head per workgroup.
//
// A 4-bit cache with fine-grained block scales ("从 PagedAttention 到
// Prefill-Decode 分离的深度解析", section 6.2) quarters the bytes a decode step
// reads against f16/bf16, and the step is bound by those bytes ("Injecting
// Adrenaline into LLM Serving" review, section 2.2).  Format: pkv_mxfp4.h.
//
//  * Four lanes cover a token row: lane (r, c) holds codes [c D/4, (c+1) D/4) of
//    row r (16 bytes for D = 128, 8 for D = 64), so one load instruction reads a
//    whole 16-row block of one pool; each lane also loads the one scale byte of
//    its 32-element block(s).
//  * Codes are decoded by the hardware conversions, exact: for q . k, code pairs
//    go to q's type and meet q's pairs in packed dot products accumulated in
//    float32 (bf16: v_cvt_scalef32_pk_bf16_fp4 with the block scale; f16:
//    v_cvt_scalef32_pk_f16_fp4 at unit scale, the lane's sum then times the
//    scale; an f32 q takes float32 codes and FMAs); V codes go to float32 with
//    their scale (v_cvt_scalef32_pk_f32_fp4) for the weighted sum.  The four
//    lanes of a row add their partial dot products with DPP.
//  * Block ids are staged in LDS per window; each wave takes chunks of CH
//    blocks and issues the next chunk's loads before computing the current one;
//    the online softmax runs in the log2 domain with one running max per wave,
//    moved lazily, so the wave's row groups merge by plain sums (DPP row
//    rotations and lane swaps) and the waves through LDS.
//
// The fused step runs the quantizing append kernel first; this kernel then
// reads every row, the new one included, from the pools (lengths from
// context_lens, or positions + 1 when context_lens is NULL).  Quantizing the new
// row in this kernel instead measured slower: its registers cost a wave per SIMD.
#include "pkv_mxfp4.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kMx4WindowBlocks = 256;
constexpr float kMx4Slack = 8.0f;   // log2 units: weights stay below 256
constexpr int kDppRowRor4 = 0x124;  // rotate each row of 16 lanes right by 4
constexpr int kDppRowRor8 = 0x128;  // ... by 8

// Sum / max over the 16 row groups of a wave (lanes 4 apart): row rotations by 4
// and 8 within each row of 16, then the gfx950 row and half swaps.
__device__ __forceinline__ float rows_sum(float v) {
    v += dpp_f<kDppRowRor4>(v);
    v += dpp_f<kDppRowRor8>(v);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float v) {
    v = fmaxf(v, dpp_f<kDppRowRor4>(v));
    v = fmaxf(v, dpp_f<kDppRowRor8>(v));
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// acc + q . (codes of byte X of w), as one packed dot product: the code pair is
// decoded with the block scale to bf16 (exact), or at unit scale to f16 (the code
// values are exact there; the caller applies the scale)
template <int X>
__device__ __forceinline__ float dot_codes_bf16(uint32_t q, uint32_t w, float sc, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q),
                                           __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, X), acc, false);
}
template <int X>
__device__ __forceinline__ float dot_codes_f16(uint32_t q, uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q), __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, X),
                                  acc, false);
}

template <int D>
struct Mx4Row {
    static constexpr int CPL = D / 4;          // codes per lane
    static constexpr int NWD = CPL / 8;        // 32-bit words per lane
    uint32_t w[NWD];
};

template <int D>
__device__ __forceinline__ Mx4Row<D> ld_row(const uint8_t* p) {
    Mx4Row<D> r;
    if constexpr (Mx4Row<D>::NWD == 4) {
        const uint4 v = ld16(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
        const uint2 v = ld8(p);
        r.w[0] = v.x; r.w[1] = v.y;
    }
    return r;
}

// CPL consecutive elements of a row of q in storage dtype QDT -> floats (exact).
template <int QDT, int CPL>
__device__ __forceinline__ void load_q(const char* p, float (&f)[CPL]) {
#pragma unroll
    for (int i = 0; i < CPL / 16; ++i) {
        float t[16];
        load16_f32<QDT>(p + (size_t)16 * i * Dt<QDT>::bytes, t);
#pragma unroll
        for (int e = 0; e < 16; ++e) f[16 * i + e] = t[e];
    }
}

template <int QDT, int D, int NW, int CH>
__global__ __launch_bounds__(NW * 64) void decode_mxfp4_kernel(const AttnArgs a) {
    constexpr int QES = Dt<QDT>::bytes;
    constexpr int CPL = Mx4Row<D>::CPL;
    constexpr int RB = D / 2;                  // code bytes per row
    constexpr int SB = D / 32;                 // scale bytes per row
    static_assert(D == 64 || D == 128, "head dim");

    __shared__ int32_t s_ids[kMx4WindowBlocks];
    __shared__ int s_bad;
    __shared__ float s_m[NW];
    __shared__ float s_l[NW];
    __shared__ float s_o[NW][D];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane >> 2;                   // row of the block
    const int c = lane & 3;                    // quarter of the row

    const int BH = a.B * a.H_q;
    const int unit = xcd_pair_unit(blockIdx.x, a.n_parts * BH);
    const int pg = unit / BH;
    const int part = unit_part(a, pg);
    const int bh = unit - pg * BH;
    const int b = bh / a.H_q;
    const int h = bh - b * a.H_q;
    const int g = h / a.G;

    const bool from_pos = a.context_lens == nullptr;
    const int n = from_pos ? a.positions[b] + 1 : a.context_lens[b];
    // q: float32 for an f32 q; otherwise the storage pairs as they are, for the
    // packed dot products (element pair j of the lane's piece in word j)
    constexpr bool PACKED = QDT != DT_F32;
    float qf[PACKED ? 1 : CPL];
    uint32_t qp[PACKED ? CPL / 2 : 1];
    if constexpr (PACKED) {
        const char* qs = a.q + ((int64_t)b * a.q_row_stride + (int64_t)h * D + c * CPL) * QES;
#pragma unroll
        for (int i = 0; i < CPL / 8; ++i) {
            const uint4 v = ld16_cached(qs + 16 * i);
            qp[4 * i] = v.x; qp[4 * i + 1] = v.y; qp[4 * i + 2] = v.z; qp[4 * i + 3] = v.w;
        }
    } else {
        load_q<QDT, CPL>(a.q + ((int64_t)b * a.q_row_stride + (int64_t)h * D + c * CPL) * QES, qf);
    }
    const int32_t* table = a.block_tables + (int64_t)b * a.bt_stride;
    const int first_blk = part * (a.part_tokens / kBlockSize);
    constexpr int PRE = (kMx4WindowBlocks + NW * 64 - 1) / (NW * 64);
    int pre[PRE];
    {
        const int spec = min(min(a.part_tokens / kBlockSize, kMx4WindowBlocks), a.bt_stride - first_blk);
#pragma unroll
        for (int k = 0; k < PRE; ++k) {
            const int t = threadIdx.x + k * NW * 64;
            pre[k] = t < spec ? table[first_blk + t] : 0;
        }
    }
    const bool bad_len = from_pos ? (n < 1 || n > a.max_context_len) : (n < 0 || n > a.max_context_len);
    float* out_row = a.out + (size_t)bh * D;
    if (bad_len || n == 0) {
        if (a.n_parts == 1 && part == 0)
            for (int d = threadIdx.x; d < D; d += NW * 64) out_row[d] = bad_len ? __builtin_nanf("") : 0.0f;
        return;
    }
    const int start = part * a.part_tokens;
    if (start >= n) return;
    const int end = min(start + a.part_tokens, n);
    const int lim = end;
    float m = kNegBig, l = 0.0f;
    float o[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) o[e] = 0.0f;

    const int nblk = (end - start + kBlockSize - 1) / kBlockSize;
    const size_t blk_codes = (size_t)a.H_kv * kBlockSize * RB;     // bytes of one block of one pool
    const size_t blk_sc = (size_t)a.H_kv * kBlockSize * SB;
    const uint8_t* kpool = reinterpret_cast<const uint8_t*>(a.k_pool) + (size_t)g * kBlockSize * RB + r * RB + c * (CPL / 2);
    const uint8_t* vpool = reinterpret_cast<const uint8_t*>(a.v_pool) + (size_t)g * kBlockSize * RB + r * RB + c * (CPL / 2);
    const uint8_t* kspool = a.k_mx_scale + (size_t)g * kBlockSize * SB + r * SB + (c * CPL) / 32;
    const uint8_t* vspool = a.v_mx_scale + (size_t)g * kBlockSize * SB + r * SB + (c * CPL) / 32;

    struct Buf {
        Mx4Row<D> k[CH], v[CH];
        uint32_t ks[CH], vs[CH];
    };
    auto load_chunk = [&](Buf& bf, int cb0) {
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            const size_t id = (size_t)__builtin_amdgcn_readfirstlane(s_ids[cb0 + cb]);
            bf.k[cb] = ld_row<D>(kpool + id * blk_codes);
            bf.v[cb] = ld_row<D>(vpool + id * blk_codes);
            bf.ks[cb] = kspool[id * blk_sc];
            bf.vs[cb] = vspool[id * blk_sc];
        }
    };
    // Online-softmax update with CH rows (one per block); valid[cb] masks rows at or past lim.
    auto accumulate = [&](const Buf& bf, const bool (&valid)[CH]) {
        float s[CH];
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            const float sc = mx_scale_operand(bf.ks[cb]);
            float acc = 0.0f;
            if constexpr (QDT == DT_BF16) {
                // code pairs decoded with their scale to bf16 (exact for every scale),
                // one packed dot product with q per pair, accumulated in float32
#pragma unroll
                for (int x = 0; x < Mx4Row<D>::NWD; ++x) {
                    const uint32_t w = bf.k[cb].w[x];
                    acc = dot_codes_bf16<0>(qp[4 * x], w, sc, acc);
                    acc = dot_codes_bf16<1>(qp[4 * x + 1], w, sc, acc);
                    acc = dot_codes_bf16<2>(qp[4 * x + 2], w, sc, acc);
                    acc = dot_codes_bf16<3>(qp[4 * x + 3], w, sc, acc);
                }
            } else if constexpr (QDT == DT_F16) {
                // code pairs decoded at unit scale to f16 (the code values are exact
                // there), one packed dot product with q per pair; the block scale, a
                // power of two, multiplies the lane's sum
#pragma unroll
                for (int x = 0; x < Mx4Row<D>::NWD; ++x) {
                    const uint32_t w = bf.k[cb].w[x];
                    acc = dot_codes_f16<0>(qp[4 * x], w, acc);
                    acc = dot_codes_f16<1>(qp[4 * x + 1], w, acc);
                    acc = dot_codes_f16<2>(qp[4 * x + 2], w, acc);
                    acc = dot_codes_f16<3>(qp[4 * x + 3], w, acc);
                }
                acc *= bf.ks[cb] == 255u ? __builtin_nanf("") : sc;   // 255: a NaN scale
            } else {
#pragma unroll
                for (int x = 0; x < Mx4Row<D>::NWD; ++x) {
                    float f[8];
                    e2m1x8_to_f32(bf.k[cb].w[x], sc, f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc = fmaf(qf[8 * x + e], f[e], acc);
                }
            }
            s[cb] = mul_rn(group_sum<4>(acc), a.scale_log2);
        }
        // one running max per wave, moved only when the chunk's max exceeds it by
        // more than kMx4Slack (a rare, wave-uniform branch)
        float mloc = kNegBig;
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) mloc = valid[cb] ? fmaxf(mloc, s[cb]) : mloc;
        mloc = rows_max(mloc);
        if (__builtin_amdgcn_ballot_w64(mloc > m + kMx4Slack) != 0) {
            const float m_new = fmaxf(m, mloc);
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int e = 0; e < CPL; ++e) o[e] *= alpha;
        }
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            const float p = valid[cb] ? __builtin_amdgcn_exp2f(s[cb] - m) : 0.0f;
            l += p;
            const float sc = mx_scale_operand(bf.vs[cb]);
#pragma unroll
            for (int x = 0; x < Mx4Row<D>::NWD; ++x) {
                float f[8];
                e2m1x8_to_f32(bf.v[cb].w[x], sc, f);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[8 * x + e] = fmaf(p, f[e], o[8 * x + e]);
            }
        }
    };
    bool all_valid[CH];
#pragma unroll
    for (int cb = 0; cb < CH; ++cb) all_valid[cb] = true;

    if (threadIdx.x == 0) s_bad = 0;
    for (int r0 = 0; r0 < nblk; r0 += kMx4WindowBlocks) {
        const int nr = min(kMx4WindowBlocks, nblk - r0);
        __syncthreads();
        if (r0 == 0) {
#pragma unroll
            for (int k = 0; k < PRE; ++k) {
                const int t = threadIdx.x + k * NW * 64;
                if (t < nr) {
                    int id = pre[k];
                    if ((unsigned)id >= (unsigned)a.n_blocks) {
                        s_bad = 1;
                        id = 0;
                    }
                    s_ids[t] = id;
                }
            }
        } else {
            for (int t = threadIdx.x; t < nr; t += NW * 64) {
                int id = table[first_blk + r0 + t];
                if ((unsigned)id >= (unsigned)a.n_blocks) {
                    s_bad = 1;
                    id = 0;
                }
                s_ids[t] = id;
            }
        }
        __syncthreads();
        const int nch = (nr + CH - 1) / CH;
        const int tok_r = start + r0 * kBlockSize;
        const int nfull_all = max(0, min(nch, (lim - tok_r) / (CH * kBlockSize)));
        const int nf = w < nfull_all ? (nfull_all - w + NW - 1) / NW : 0;
        auto chunk_of = [&](int i) { return (w + NW * i) * CH; };
        // chunk i lives in buf[i % 2]; the loads of chunk i + 1 go out before chunk i is used
        Buf buf[2];
        int i = 0;
        if (nf >= 3) {
            load_chunk(buf[0], chunk_of(0));   // unconditional, so the loop's waits stay exact
            for (; i + 3 <= nf; i += 2) {
                load_chunk(buf[1], chunk_of(i + 1));
                accumulate(buf[0], all_valid);
                load_chunk(buf[0], chunk_of(i + 2));
                accumulate(buf[1], all_valid);
            }
        } else if (nf > 0) {
            load_chunk(buf[0], chunk_of(0));
        }
        for (; i < nf; i += 2) {   // at most two chunks left; chunk i is loaded
            if (i + 1 < nf) load_chunk(buf[1], chunk_of(i + 1));
            accumulate(buf[0], all_valid);
            if (i + 1 < nf) {
                if (i + 2 < nf) load_chunk(buf[0], chunk_of(i + 2));
                accumulate(buf[1], all_valid);
            }
        }
        // the partial chunk: masked loads (rows at or past lim read nothing)
        for (int k = nfull_all + ((w - nfull_all) % NW + NW) % NW; k < nch; k += NW) {
            const int cb0 = k * CH;
            Buf bf;
            bool valid[CH];
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) {
                const size_t id = (size_t)__builtin_amdgcn_readfirstlane(cb0 + cb < nr ? s_ids[cb0 + cb] : 0);
                const int t = tok_r + (cb0 + cb) * kBlockSize + r;
                valid[cb] = t < lim;
#pragma unroll
                for (int x = 0; x < Mx4Row<D>::NWD; ++x) bf.k[cb].w[x] = bf.v[cb].w[x] = 0;
                bf.ks[cb] = bf.vs[cb] = 127;
                if (valid[cb]) {
                    bf.k[cb] = ld_row<D>(kpool + id * blk_codes);
                    bf.v[cb] = ld_row<D>(vpool + id * blk_codes);
                    bf.ks[cb] = kspool[id * blk_sc];
                    bf.vs[cb] = vspool[id * blk_sc];
                }
            }
            accumulate(bf, valid);
        }
    }

    // merge the 16 row groups of the wave (lanes 4 apart hold the same columns):
    // they share m, so the merge is a sum
    l = rows_sum(l);
#pragma unroll
    for (int e = 0; e < CPL; ++e) o[e] = rows_sum(o[e]);
    if (lane < 4) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) s_o[w][c * CPL + e] = o[e];
        if (lane == 0) {
            s_m[w] = m;
            s_l[w] = l;
        }
    }
    __syncthreads();
    const bool bad = s_bad != 0;
    float M = s_m[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) M = fmaxf(M, s_m[k]);
    float L = 0.0f;
#pragma unroll
    for (int k = 0; k < NW; ++k) L += s_l[k] * __builtin_amdgcn_exp2f(s_m[k] - M);
    const float inv = 1.0f / L;
    for (int d = threadIdx.x; d < D; d += NW * 64) {
        float O = 0.0f;
#pragma unroll
        for (int k = 0; k < NW; ++k) O += s_o[k][d] * __builtin_amdgcn_exp2f(s_m[k] - M);
        const float val = bad ? __builtin_nanf("") : O * inv;
        if (a.n_parts == 1) out_row[d] = val;
        else a.part_o[((size_t)bh * a.n_parts + part) * D + d] = val;
    }
    if (a.n_parts > 1 && threadIdx.x == 0)
        a.part_lse[(size_t)bh * a.n_parts + part] = bad ? __builtin_nanf("") : M + __builtin_amdgcn_logf(L);
}

template <int QDT, int D, int NW, int CH>
static hipError_t launch_t(const AttnArgs& a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((decode_mxfp4_kernel<QDT, D, NW, CH>), dim3(grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int QDT, int D>
static hipError_t launch_d(int nw, int ch, const AttnArgs& a, unsigned grid, hipStream_t s) {
    switch (nw * 10 + ch) {
    case 42: return launch_t<QDT, D, 4, 2>(a, grid, s);
    case 82: return launch_t<QDT, D, 8, 2>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_mxfp4(int q_dtype, int D, int nw, int ch, const AttnArgs& a, unsigned grid,
                               hipStream_t stream) {
    switch (q_dtype * 1000 + D) {
    case DT_F32 * 1000 + 64: return launch_d<DT_F32, 64>(nw, ch, a, grid, stream);
    case DT_F32 * 1000 + 128: return launch_d<DT_F32, 128>(nw, ch, a, grid, stream);
    case DT_F16 * 1000 + 64: return launch_d<DT_F16, 64>(nw, ch, a, grid, stream);
    case DT_F16 * 1000 + 128: return launch_d<DT_F16, 128>(nw, ch, a, grid, stream);
    case DT_BF16 * 1000 + 64: return launch_d<DT_BF16, 64>(nw, ch, a, grid, stream);
    case DT_BF16 * 1000 + 128: return launch_d<DT_BF16, 128>(nw, ch, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

bool mxfp4_variant_exists(int nw, int ch) { return nw * 10 + ch == 42 || nw * 10 + ch == 82; }

}  // namespace pkv
