// decode_fp8.hip -- paged decode attention over an FP8 (OCP E4M3) K/V cache,
// one query head per workgroup.
//
// A low-precision KV cache keeps K/V in a few bits with fine-grained scales and
// dequantizes them for attention ("从 PagedAttention 到 Prefill-Decode 分离的
// 深度解析", section 6.2); decode attention is bound by the bytes it reads
// ("Injecting Adrenaline into LLM Serving" review, section 2.2), so one-byte
// codes halve the step's traffic against f16/bf16.  The kernel has the shape
// of the f16/bf16 per-head kernel:
//
//  * 16-byte loads hold 16 codes; D / 16 lanes cover a token row and one load
//    instruction reads TPL consecutive rows of a block.  Each row also has a
//    float scale (a power of two) per KV head, loaded next to it.
//  * Codes are decoded by the hardware conversion (v_cvt_pk_f32_fp8); q stays
//    in float32 registers (16 values per lane).  The row scale multiplies the
//    row's dot product for K and the softmax weight for V, so dequantization
//    costs one exact multiply per row.
//  * Block ids are staged in LDS per window, chunks of CH blocks are streamed
//    through a PF-deep pipeline, and the online softmax runs in the log2
//    domain; lane-group and cross-wave merges as in the f16/bf16 kernel.
//
// The fused variant (APPEND) quantizes the step's new K/V row (q's dtype) in
// the lanes that hold it -- row maximum by a lane-group reduction, scale, codes
// -- uses those codes like any other row, and the KV head's first query head
// writes codes and scale to the pool.
#include "pkv_fp8.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kFp8WindowBlocks = 256;

template <int QDT, int D, int NW, int CH, int PF, bool APPEND>
__global__ __launch_bounds__(NW * 64) void decode_fp8_kernel(const AttnArgs a) {
    constexpr int QES = Dt<QDT>::bytes;
    constexpr int E = 16;                     // codes per 16-byte lane vector
    constexpr int LPT = D / E;                // lanes per token row
    constexpr int TPL = 64 / LPT;             // tokens per wave-wide load
    constexpr int LPB = kBlockSize / TPL;     // loads per block
    constexpr int NL = CH * LPB;
    static_assert(TPL * LPT == 64 && LPB * TPL == kBlockSize, "unsupported shape");

    __shared__ int32_t s_ids[kFp8WindowBlocks];
    __shared__ int s_bad;
    __shared__ float s_m[NW];
    __shared__ float s_l[NW];
    __shared__ float s_o[NW][D];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane / LPT;
    const int c = lane % LPT;

    const int BH = a.B * a.H_q;
    const int unit = xcd_pair_unit(blockIdx.x, a.n_parts * BH);
    const int pg = unit / BH;
    const int part = unit_part(a, pg);
    const int bh = unit - pg * BH;
    const int b = bh / a.H_q;
    const int h = bh - b * a.H_q;
    const int g = h / a.G;
    const bool writer = APPEND && (h % a.G) == 0;

    const int n = APPEND ? a.positions[b] + 1 : a.context_lens[b];
    float qf[E];
    load16_f32<QDT>(a.q + ((int64_t)b * a.q_row_stride + (int64_t)h * D + c * E) * QES, qf);
    const int32_t* table = a.block_tables + (int64_t)b * a.bt_stride;
    const int first_blk = part * (a.part_tokens / kBlockSize);
    constexpr int PRE = (kFp8WindowBlocks + NW * 64 - 1) / (NW * 64);
    int pre[PRE];
    {
        const int spec = min(min(a.part_tokens / kBlockSize, kFp8WindowBlocks), a.bt_stride - first_blk);
#pragma unroll
        for (int k = 0; k < PRE; ++k) {
            const int t = threadIdx.x + k * NW * 64;
            pre[k] = t < spec ? table[first_blk + t] : 0;
        }
    }
    const bool bad_len = APPEND ? (n < 1 || n > a.max_context_len) : (n < 0 || n > a.max_context_len);
    float* out_row = a.out + (size_t)bh * D;
    if (bad_len || n == 0) {
        if (a.n_parts == 1 && part == 0)
            for (int d = threadIdx.x; d < D; d += NW * 64) out_row[d] = bad_len ? __builtin_nanf("") : 0.0f;
        return;
    }
    const int start = part * a.part_tokens;
    if (start >= n) return;
    const int end = min(start + a.part_tokens, n);
    const int n_hist = APPEND ? n - 1 : n;
    const int lim = min(end, n_hist);
    const int pos_new = (APPEND && end == n) ? n - 1 : -1;

    float m = kNegBig, l = 0.0f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.0f;

    const int nblk = (end - start + kBlockSize - 1) / kBlockSize;
    const size_t blk_codes = (size_t)a.H_kv * kBlockSize * D;            // bytes of one block of one pool
    const size_t head_codes = (size_t)g * kBlockSize * D;
    const size_t blk_rows = (size_t)a.H_kv * kBlockSize;                   // scales of one block
    const size_t head_rows = (size_t)g * kBlockSize;
    int lane_off[LPB];
#pragma unroll
    for (int i = 0; i < LPB; ++i) lane_off[i] = (i * TPL + r) * D + c * E;
    const uint8_t* kpool = reinterpret_cast<const uint8_t*>(a.k_pool);
    const uint8_t* vpool = reinterpret_cast<const uint8_t*>(a.v_pool);

    auto load_full = [&](uint4 (&kv)[NL], uint4 (&vv)[NL], float (&ks)[NL], float (&vs)[NL], int cb0) {
        int id[CH];
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) id[cb] = __builtin_amdgcn_readfirstlane(s_ids[cb0 + cb]);
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
#pragma unroll
            for (int i = 0; i < LPB; ++i)
                kv[cb * LPB + i] = ld16(kpool + (size_t)id[cb] * blk_codes + head_codes + lane_off[i]);
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
#pragma unroll
            for (int i = 0; i < LPB; ++i)
                vv[cb * LPB + i] = ld16(vpool + (size_t)id[cb] * blk_codes + head_codes + lane_off[i]);
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
#pragma unroll
            for (int i = 0; i < LPB; ++i) {
                const size_t srow = (size_t)id[cb] * blk_rows + head_rows + i * TPL + r;
                ks[cb * LPB + i] = a.k_scale[srow];
                vs[cb * LPB + i] = a.v_scale[srow];
            }
    };
    auto accumulate = [&](const uint4 (&kv)[NL], const uint4 (&vv)[NL], const float (&ks)[NL],
                          const float (&vs)[NL], const bool (&valid)[NL]) {
        float s[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) s[j] = mul_rn(group_sum<LPT>(dot_fp8x16(qf, kv[j])) * ks[j], a.scale_log2);
        float mloc = kNegBig;
#pragma unroll
        for (int j = 0; j < NL; ++j) mloc = valid[j] ? fmaxf(mloc, s[j]) : mloc;
        const float m_new = fmaxf(m, mloc);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] *= alpha;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const float p = valid[j] ? __builtin_amdgcn_exp2f(s[j] - m) : 0.0f;
            l += p;
            axpy_fp8x16(o, p * vs[j], vv[j]);
        }
    };
    bool all_valid[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) all_valid[j] = true;

    if (threadIdx.x == 0) s_bad = 0;
    for (int r0 = 0; r0 < nblk; r0 += kFp8WindowBlocks) {
        const int nr = min(kFp8WindowBlocks, nblk - r0);
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
        const bool any_bad = s_bad != 0;
        const int nch = (nr + CH - 1) / CH;

        const int tok_r = start + r0 * kBlockSize;
        const int nfull_all = max(0, min(nch, (lim - tok_r) / (CH * kBlockSize)));
        const int nf = w < nfull_all ? (nfull_all - w + NW - 1) / NW : 0;
        uint4 bk[PF][NL], bv[PF][NL];
        float bks[PF][NL], bvs[PF][NL];
        auto chunk_of = [&](int i) { return (w + NW * i) * CH; };
        if (nf >= PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) load_full(bk[u], bv[u], bks[u], bvs[u], chunk_of(u));
            int i = 0;
            for (; i + 2 * PF <= nf; i += PF) {
#pragma unroll
                for (int u = 0; u < PF; ++u) {
                    accumulate(bk[u], bv[u], bks[u], bvs[u], all_valid);
                    load_full(bk[u], bv[u], bks[u], bvs[u], chunk_of(i + PF + u));
                }
            }
            const int rem = nf - i - PF;
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                accumulate(bk[u], bv[u], bks[u], bvs[u], all_valid);
                if (u < rem) load_full(bk[u], bv[u], bks[u], bvs[u], chunk_of(i + PF + u));
            }
#pragma unroll
            for (int u = 0; u < PF; ++u)
                if (u < rem) accumulate(bk[u], bv[u], bks[u], bvs[u], all_valid);
        } else {
            for (int i = 0; i < nf; ++i) {
                load_full(bk[0], bv[0], bks[0], bvs[0], chunk_of(i));
                accumulate(bk[0], bv[0], bks[0], bvs[0], all_valid);
            }
        }

        // The partial chunk: masked loads, and in the fused call the new row,
        // quantized here from k_new / v_new.
        for (int k = nfull_all + ((w - nfull_all) % NW + NW) % NW; k < nch; k += NW) {
            const int cb0 = k * CH;
            const int tok0 = start + (r0 + cb0) * kBlockSize;
            int id[CH];
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) id[cb] = __builtin_amdgcn_readfirstlane(cb0 + cb < nr ? s_ids[cb0 + cb] : 0);
            uint4 kv[NL], vv[NL];
            float ks[NL], vs[NL];
            bool valid[NL];
#pragma unroll
            for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                for (int i = 0; i < LPB; ++i) {
                    const int j = cb * LPB + i;
                    const int t = tok0 + cb * kBlockSize + i * TPL + r;
                    const size_t code_off = (size_t)id[cb] * blk_codes + head_codes + lane_off[i];
                    const size_t srow = (size_t)id[cb] * blk_rows + head_rows + i * TPL + r;
                    kv[j] = make_uint4(0, 0, 0, 0);
                    vv[j] = make_uint4(0, 0, 0, 0);
                    ks[j] = 0.0f;
                    vs[j] = 0.0f;
                    valid[j] = false;
                    if (t < lim) {
                        kv[j] = ld16(kpool + code_off);
                        vv[j] = ld16(vpool + code_off);
                        ks[j] = a.k_scale[srow];
                        vs[j] = a.v_scale[srow];
                        valid[j] = true;
                    }
                    if constexpr (APPEND) {
                        // every lane takes part in the row reductions; only the row
                        // holding the new token keeps the result
                        const bool mine = t == pos_new;
                        const size_t src = ((size_t)b * a.new_row_stride + (size_t)g * D + c * E) * QES;
                        float xk[E], xv[E];
                        if (mine) {
                            load16_f32<QDT>(a.k_new + src, xk);
                            load16_f32<QDT>(a.v_new + src, xv);
                        } else {
#pragma unroll
                            for (int e = 0; e < E; ++e) xk[e] = xv[e] = 0.0f;
                        }
                        float mk = 0.0f, mv = 0.0f;
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            mk = fmaxf(mk, fabsf(xk[e]));
                            mv = fmaxf(mv, fabsf(xv[e]));
                        }
                        mk = group_max<LPT>(mk);
                        mv = group_max<LPT>(mv);
                        if (mine) {
                            const int Ek = fp8_row_exponent(mk), Ev = fp8_row_exponent(mv);
                            const float ik = pow2f(-Ek), iv = pow2f(-Ev);
                            uint32_t wk[4], wv[4];
#pragma unroll
                            for (int q4 = 0; q4 < 4; ++q4) {
                                wk[q4] = fp8_encode(xk[4 * q4] * ik) | (fp8_encode(xk[4 * q4 + 1] * ik) << 8) |
                                         (fp8_encode(xk[4 * q4 + 2] * ik) << 16) | (fp8_encode(xk[4 * q4 + 3] * ik) << 24);
                                wv[q4] = fp8_encode(xv[4 * q4] * iv) | (fp8_encode(xv[4 * q4 + 1] * iv) << 8) |
                                         (fp8_encode(xv[4 * q4 + 2] * iv) << 16) | (fp8_encode(xv[4 * q4 + 3] * iv) << 24);
                            }
                            kv[j] = make_uint4(wk[0], wk[1], wk[2], wk[3]);
                            vv[j] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                            ks[j] = pow2f(Ek);
                            vs[j] = pow2f(Ev);
                            valid[j] = true;
                            if (writer && !any_bad) {
                                st16(reinterpret_cast<uint8_t*>(a.k_pool_w) + code_off, kv[j]);
                                st16(reinterpret_cast<uint8_t*>(a.v_pool_w) + code_off, vv[j]);
                                if (c == 0) {
                                    a.k_scale_w[srow] = ks[j];
                                    a.v_scale_w[srow] = vs[j];
                                }
                            }
                        }
                    }
                }
            accumulate(kv, vv, ks, vs, valid);
        }
    }

    // merge the TPL row groups of the wave
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
        const float m_o = __shfl_xor(m, off, 64);
        const float l_o = __shfl_xor(l, off, 64);
        const float M = fmaxf(m, m_o);
        const float fa = __builtin_amdgcn_exp2f(m - M);
        const float fb = __builtin_amdgcn_exp2f(m_o - M);
        l = l * fa + l_o * fb;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = o[e] * fa + __shfl_xor(o[e], off, 64) * fb;
        m = M;
    }
    if (lane < LPT) {
#pragma unroll
        for (int e = 0; e < E; ++e) s_o[w][c * E + e] = o[e];
        if (lane == 0) {
            s_m[w] = m;
            s_l[w] = l;
        }
    }
    __syncthreads();
    const bool bad = s_bad != 0;
    float M = s_m[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) M = fmaxf(M, s_m[i]);
    float L = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; ++i) L += s_l[i] * __builtin_amdgcn_exp2f(s_m[i] - M);
    const float inv = 1.0f / L;
    for (int d = threadIdx.x; d < D; d += NW * 64) {
        float O = 0.0f;
#pragma unroll
        for (int i = 0; i < NW; ++i) O += s_o[i][d] * __builtin_amdgcn_exp2f(s_m[i] - M);
        const float val = bad ? __builtin_nanf("") : O * inv;
        if (a.n_parts == 1) {
            out_row[d] = val;
        } else {
            a.part_o[((size_t)bh * a.n_parts + part) * D + d] = val;
        }
    }
    if (a.n_parts > 1 && threadIdx.x == 0)
        a.part_lse[(size_t)bh * a.n_parts + part] = bad ? __builtin_nanf("") : M + __builtin_amdgcn_logf(L);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <int QDT, int D, int NW, int CH, int PF>
static hipError_t launch_fp8_t(bool append, const AttnArgs& a, unsigned grid, hipStream_t stream) {
    if (append)
        hipLaunchKernelGGL((decode_fp8_kernel<QDT, D, NW, CH, PF, true>), dim3(grid), dim3(NW * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_fp8_kernel<QDT, D, NW, CH, PF, false>), dim3(grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

#define PKV_FP8_VARIANTS X(4, 2, 1) X(4, 2, 2) X(8, 2, 2) X(4, 4, 1)

template <int QDT, int D>
static hipError_t launch_fp8_d(int nw, int ch, int pf, bool append, const AttnArgs& a, unsigned grid, hipStream_t s) {
    switch (nw * 100 + ch * 10 + pf) {
#define X(NW, CH, PF) \
    case NW * 100 + CH * 10 + PF: return launch_fp8_t<QDT, D, NW, CH, PF>(append, a, grid, s);
        PKV_FP8_VARIANTS
#undef X
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_fp8(int q_dtype, int D, int nw, int ch, int pf, bool append, const AttnArgs& a,
                             unsigned grid, hipStream_t stream) {
    switch (q_dtype * 1000 + D) {
    case DT_F32 * 1000 + 64: return launch_fp8_d<DT_F32, 64>(nw, ch, pf, append, a, grid, stream);
    case DT_F32 * 1000 + 128: return launch_fp8_d<DT_F32, 128>(nw, ch, pf, append, a, grid, stream);
    case DT_F16 * 1000 + 64: return launch_fp8_d<DT_F16, 64>(nw, ch, pf, append, a, grid, stream);
    case DT_F16 * 1000 + 128: return launch_fp8_d<DT_F16, 128>(nw, ch, pf, append, a, grid, stream);
    case DT_BF16 * 1000 + 64: return launch_fp8_d<DT_BF16, 64>(nw, ch, pf, append, a, grid, stream);
    case DT_BF16 * 1000 + 128: return launch_fp8_d<DT_BF16, 128>(nw, ch, pf, append, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

bool fp8_variant_exists(int nw, int ch, int pf) {
    switch (nw * 100 + ch * 10 + pf) {
#define X(NW, CH, PF) case NW * 100 + CH * 10 + PF:
        PKV_FP8_VARIANTS
#undef X
        return true;
    default: return false;
    }
}

}  // namespace pkv
