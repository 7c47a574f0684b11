// decode_mxfp4_mfma.hip -- paged decode attention over an MXFP4 K/V cache on the
// gfx950 matrix cores, one workgroup per (partition, request, KV head) serving
// its G <= 16 query heads.
//
// A 4-bit cache with fine-grained block scales ("从 PagedAttention 到
// Prefill-Decode 分离的深度解析", section 6.2) quarters the bytes a step
// streams, and the step is bound by those bytes ("Injecting Adrenaline into LLM
// Serving" review, section 2.2).  At a quarter of the bytes the per-element
// arithmetic of a vector-unit kernel (decode, multiply-add per element for K
// and for V) becomes the limit, so both products run on MFMA tiles in bf16 with
// f32 accumulation:
//
//   scores  S^T = K Q^T   v_mfma_f32_16x16x32_bf16, D/32 steps (x2 for f16 q)
//   output  O^T = V^T P^T v_mfma_f32_16x16x32_bf16, D/16 tiles
//
// Codes are decoded with their block scale by v_cvt_scalef32_pk_bf16_fp4, which
// is exact for every code and E8M0 scale: code x 2^E is representable in bf16
// over f32's exponent range, subnormals included (6 x 2^127 overflows to inf,
// as it does in f32).  A bf16 q is used as is; an f16 q is split exactly into
// bf16 hi + lo (f16's 11 significant bits fit in two bf16 pieces), each a
// product of its own.  P is carried as bf16 hi + lo in one K=32 product.
//
// Lane l = 16 j + c.  Tile row m of the score product is token tau(m) =
// 4 (m % 4) + m / 4 of the block; the lane reads row tau(c), bytes
// [D/8 j, D/8 (j + 1)) (D/4 dims, 16 bytes for D = 128), one scale byte, and
// takes 8 of those dims per step.  The dot product does not care which dims a
// step pairs as long as q's operand pairs the same ones.  With that token order
// the score tile a lane holds (rows 4 j + i, column c -> tokens 4 i + j) is the
// P^T operand the second product needs, and the V rows it needs are tokens
// 4 i + j, elements [c D/16, (c + 1) D/16) -- D/32 bytes of codes and one scale
// byte each, and each load instruction covers four whole consecutive rows.  Row
// m of output tile T is d = m D/16 + T, so V is never transposed.
//
// Softmax is online per query head in the log2 domain with the lazy rescale of
// the 16-bit grouped kernel; waves merge through LDS; the partition's result
// goes to the output or, when split, to the log-sum-exp merge.  The quantizing
// append runs before this kernel, which reads every row from the pools.
#include "pkv_mxfp4.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

constexpr int kWin = 256;                 // block ids staged per window
constexpr float kSlack = 8.0f;            // log2 units: weights stay below 256

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx4 mma_bf16(const uint4& a, const uint4& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

// p0, p1 -> packed bf16 (hi0, hi1) and (lo0, lo1) with p ~= hi + lo (to ~2^-17)
__device__ __forceinline__ void split_bf16(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    const bf162_t h = {(__bf16)p0, (__bf16)p1};
    const bf162_t r = {(__bf16)(p0 - (float)h.x), (__bf16)(p1 - (float)h.y)};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, r);
}

// E8M0 byte -> scale operand.  The conversion reads only the exponent field of
// its f32 scale, and an exponent field of 0 means 2^-127, so the byte shifted
// into place is the operand for every scale.
__device__ __forceinline__ float mx_operand(uint32_t s) { return __uint_as_float(s << 23); }

// one 32-bit word of 8 codes -> four packed bf16 pairs (elements 2x, 2x + 1 in word x), scaled
__device__ __forceinline__ void e2m1x8_to_bf16(uint32_t w, float sc, uint32_t (&o)[4]) {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
}
// two codes of the low byte -> one packed pair (D = 64 V pieces are 2 bytes)
__device__ __forceinline__ void e2m1x4_to_bf16(uint32_t w, float sc, uint32_t (&o)[2]) {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
}

template <int D>
struct Mx4Geo {
    static constexpr int KS = D / 32;          // score steps
    static constexpr int VT = D / 16;          // output tiles
    static constexpr int KW = KS;              // K code words per lane per block (8 codes per step)
    static constexpr int VB = VT / 2;          // V code bytes per lane per token
    static constexpr int RB = D / 2;           // code bytes per row
    static constexpr int SB = D / 32;          // scale bytes per row
};

// One chunk of CH blocks as loaded: K codes of the lane's row, its scale byte,
// and the codes and scale bytes of its four V rows.
template <int D, int CH>
struct Mx4Chunk {
    uint32_t k[CH][Mx4Geo<D>::KW];
    uint32_t ks[CH];
    uint32_t v[CH][4];                         // VB bytes used (4 for D = 128, 2 for D = 64)
    uint32_t vs[CH][4];
};

template <int D>
__device__ __forceinline__ void ld_kcodes(const uint8_t* p, uint32_t (&w)[Mx4Geo<D>::KW]) {
    if constexpr (D == 128) {
        const uint4 x = ld16(p);
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    } else {
        const uint2 x = ld8(p);
        w[0] = x.x; w[1] = x.y;
    }
}
template <int D>
__device__ __forceinline__ uint32_t ld_vcodes(const uint8_t* p) {
    if constexpr (D == 128) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    else return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}

template <int QDT, int D>
struct Mx4Lane {
    using Geo = Mx4Geo<D>;
    static constexpr int KS = Geo::KS, VT = Geo::VT, NQ = QDT == DT_F16 ? 2 : 1;
    int j, c;
    uint4 qf[NQ][KS];          // B operand of step s (bf16; [1] = lo part of an f16 q)
    floatx4 acc[VT];
    float m, l, scale_log2;

    __device__ __forceinline__ void init(const AttnArgs& a, int lane, int b, int g) {
        j = lane >> 4;
        c = lane & 15;
        scale_log2 = a.scale_log2;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[0][s] = make_uint4(0, 0, 0, 0);
            if constexpr (NQ == 2) qf[1][s] = make_uint4(0, 0, 0, 0);
        }
        if (c < a.G) {
            const char* qp = a.q + ((int64_t)b * a.q_row_stride + (int64_t)(g * a.G + c) * D + 8 * KS * j) * 2;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint4 x = ld16_cached(qp + 16 * s);
                if constexpr (QDT == DT_BF16) {
                    qf[0][s] = x;
                } else {
                    uint32_t hi[4], lo[4];
                    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const half2_t h = __builtin_bit_cast(half2_t, w[e]);
                        split_bf16((float)h.x, (float)h.y, hi[e], lo[e]);   // exact: f16 -> bf16 hi + lo
                    }
                    qf[0][s] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                    qf[1][s] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < VT; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        m = kNegBig;
        l = 0.0f;
    }

    // Online-softmax update with CH blocks; valid[cb][i] masks token 4 i + j.
    template <int CH>
    __device__ __forceinline__ void accumulate(const Mx4Chunk<D, CH>& ck, const bool (&valid)[CH][4]) {
        float sc[CH][4];
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            const float ksc = mx_operand(ck.ks[cb]);
            floatx4 st = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                uint32_t kd[4];
                e2m1x8_to_bf16(ck.k[cb][s], ksc, kd);
                const uint4 ka = make_uint4(kd[0], kd[1], kd[2], kd[3]);
                st = mma_bf16(ka, qf[0][s], st);
                if constexpr (NQ == 2) st = mma_bf16(ka, qf[1][s], st);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[cb][i] = mul_rn(st[i], scale_log2);
        }
        float mloc = kNegBig;
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mloc = valid[cb][i] ? fmaxf(mloc, sc[cb][i]) : mloc;
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        // the reference max moves only when some head's running max grows by more
        // than kSlack (a rare, wave-uniform branch)
        if (__builtin_amdgcn_ballot_w64(mloc > m + kSlack) != 0) {
            const float m_new = fmaxf(m, mloc);
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int t = 0; t < VT; ++t) acc[t] *= alpha;
        }
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = valid[cb][i] ? __builtin_amdgcn_exp2f(sc[cb][i] - m) : 0.0f;
                l += p[i];
            }
            uint4 pk;
            split_bf16(p[0], p[1], pk.x, pk.z);
            split_bf16(p[2], p[3], pk.y, pk.w);
            // V rows of the lane's four tokens, decoded with their scales: word x of
            // row i holds elements (2x, 2x + 1) of the lane's piece
            uint32_t vd[4][VT / 2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float vsc = mx_operand(ck.vs[cb][i]);
                if constexpr (D == 128) {
                    uint32_t o[4];
                    e2m1x8_to_bf16(ck.v[cb][i], vsc, o);
#pragma unroll
                    for (int x = 0; x < 4; ++x) vd[i][x] = o[x];
                } else {
                    uint32_t o[2];
                    e2m1x4_to_bf16(ck.v[cb][i], vsc, o);
                    vd[i][0] = o[0];
                    vd[i][1] = o[1];
                }
            }
#pragma unroll
            for (int t = 0; t < VT; ++t) {
                const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
                const int x = t >> 1;
                const uint32_t v01 = __builtin_amdgcn_perm(vd[1][x], vd[0][x], sel);
                const uint32_t v23 = __builtin_amdgcn_perm(vd[3][x], vd[2][x], sel);
                acc[t] = mma_bf16(make_uint4(v01, v23, v01, v23), pk, acc[t]);
            }
        }
    }
};

}  // namespace

template <int QDT, int D, int NW, int CH>
__global__ __launch_bounds__(NW * 64) void decode_mxfp4_mfma_kernel(const AttnArgs a) {
    using Geo = Mx4Geo<D>;
    using L = Mx4Lane<QDT, D>;
    constexpr int RB = Geo::RB, SB = Geo::SB, VT = Geo::VT;
    __shared__ int32_t s_ids[kWin];
    __shared__ int s_bad;
    __shared__ float s_m[NW][16];
    __shared__ float s_l[NW][16];
    __shared__ float s_o[NW][16][D + 4];

    const int BG = a.B * a.H_kv;
    const int unit = xcd_pair_unit(blockIdx.x, a.n_parts * BG);
    const int part = unit / BG;
    const int bg = unit - part * BG;
    const int b = bg / a.H_kv;
    const int g = bg - b * a.H_kv;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    L st;
    st.init(a, lane, b, g);
    const int32_t* table = a.block_tables + (int64_t)b * a.bt_stride;
    const int first_blk = part * (a.part_tokens / kBlockSize);
    constexpr int PRE = (kWin + NW * 64 - 1) / (NW * 64);
    int pre[PRE];
    {
        const int spec = min(min(a.part_tokens / kBlockSize, kWin), a.bt_stride - first_blk);
#pragma unroll
        for (int k = 0; k < PRE; ++k) {
            const int t = threadIdx.x + k * NW * 64;
            pre[k] = t < spec ? table[first_blk + t] : 0;
        }
    }
    const bool from_pos = a.context_lens == nullptr;
    const int n = from_pos ? a.positions[b] + 1 : a.context_lens[b];
    const bool bad_len = from_pos ? (n < 1 || n > a.max_context_len) : (n < 0 || n > a.max_context_len);
    if (bad_len || n == 0) {
        if (a.n_parts == 1 && part == 0)
            for (int x = threadIdx.x; x < a.G * D; x += NW * 64)
                a.out[((size_t)b * a.H_q + (size_t)g * a.G) * D + x] = bad_len ? __builtin_nanf("") : 0.0f;
        return;
    }
    const int start = part * a.part_tokens;
    if (start >= n) return;
    const int lim = min(start + a.part_tokens, n);
    const int nblk = (lim - start + kBlockSize - 1) / kBlockSize;

    // per-lane byte offsets inside one (block, KV head) tile of codes / of scales
    const int tau = 4 * (st.c & 3) + (st.c >> 2);
    const int koff = tau * RB + (D / 8) * st.j;
    const int ksoff = tau * SB + (Geo::KS * st.j) / 4;
    int voff[4], vsoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        voff[i] = (4 * i + st.j) * RB + st.c * Geo::VB;
        vsoff[i] = (4 * i + st.j) * SB + (st.c * VT) / 32;
    }
    const size_t blk_codes = (size_t)a.H_kv * kBlockSize * RB;
    const size_t blk_sc = (size_t)a.H_kv * kBlockSize * SB;
    const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.k_pool) + (size_t)g * kBlockSize * RB;
    const uint8_t* vp = reinterpret_cast<const uint8_t*>(a.v_pool) + (size_t)g * kBlockSize * RB;
    const uint8_t* ksp = a.k_mx_scale + (size_t)g * kBlockSize * SB;
    const uint8_t* vsp = a.v_mx_scale + (size_t)g * kBlockSize * SB;

    using Chunk = Mx4Chunk<D, CH>;
    auto load_chunk = [&](Chunk& ck, int cb0) {
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            const size_t id = (size_t)__builtin_amdgcn_readfirstlane(s_ids[cb0 + cb]);
            ld_kcodes<D>(kp + id * blk_codes + koff, ck.k[cb]);
            ck.ks[cb] = ksp[id * blk_sc + ksoff];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ck.v[cb][i] = ld_vcodes<D>(vp + id * blk_codes + voff[i]);
                ck.vs[cb][i] = vsp[id * blk_sc + vsoff[i]];
            }
        }
    };
    bool all_valid[CH][4];
#pragma unroll
    for (int cb = 0; cb < CH; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) all_valid[cb][i] = true;

    if (threadIdx.x == 0) s_bad = 0;
    for (int r0 = 0; r0 < nblk; r0 += kWin) {
        const int nr = min(kWin, nblk - r0);
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
        Chunk buf[2];
        int i = 0;
        if (nf >= 3) {
            load_chunk(buf[0], chunk_of(0));   // unconditional, so the loop's waits stay exact
            for (; i + 3 <= nf; i += 2) {
                load_chunk(buf[1], chunk_of(i + 1));
                st.template accumulate<CH>(buf[0], all_valid);
                load_chunk(buf[0], chunk_of(i + 2));
                st.template accumulate<CH>(buf[1], all_valid);
            }
        } else if (nf > 0) {
            load_chunk(buf[0], chunk_of(0));
        }
        for (; i < nf; i += 2) {   // at most two chunks left; chunk i is loaded
            if (i + 1 < nf) load_chunk(buf[1], chunk_of(i + 1));
            st.template accumulate<CH>(buf[0], all_valid);
            if (i + 1 < nf) {
                if (i + 2 < nf) load_chunk(buf[0], chunk_of(i + 2));
                st.template accumulate<CH>(buf[1], all_valid);
            }
        }
        // the partial chunk: rows at or past lim are never read and enter as zeros
        for (int k = nfull_all + ((w - nfull_all) % NW + NW) % NW; k < nch; k += NW) {
            const int cb0 = k * CH;
            Chunk ck;
            bool valid[CH][4];
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) {
                const bool in = cb0 + cb < nr;
                const size_t id = (size_t)__builtin_amdgcn_readfirstlane(in ? s_ids[cb0 + cb] : 0);
                const int tb = tok_r + (cb0 + cb) * kBlockSize;
#pragma unroll
                for (int x = 0; x < Geo::KW; ++x) ck.k[cb][x] = 0;
                ck.ks[cb] = 127;
                if (in && tb + tau < lim) {
                    ld_kcodes<D>(kp + id * blk_codes + koff, ck.k[cb]);
                    ck.ks[cb] = ksp[id * blk_sc + ksoff];
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    valid[cb][q] = in && tb + 4 * q + st.j < lim;
                    ck.v[cb][q] = 0;
                    ck.vs[cb][q] = 127;
                    if (valid[cb][q]) {
                        ck.v[cb][q] = ld_vcodes<D>(vp + id * blk_codes + voff[q]);
                        ck.vs[cb][q] = vsp[id * blk_sc + vsoff[q]];
                    }
                }
            }
            st.template accumulate<CH>(ck, valid);
        }
    }

    // merge the waves through LDS and write the partition's result
    float l = st.l;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (st.j == 0) {
        s_m[w][st.c] = st.m;
        s_l[w][st.c] = l;
    }
#pragma unroll
    for (int t = 0; t < VT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[w][st.c][(4 * st.j + i) * VT + t] = st.acc[t][i];
    __syncthreads();
    const bool bad = s_bad != 0;
    const int G = a.G;
    for (int x = threadIdx.x; x < G * D; x += NW * 64) {
        const int hh = x / D;
        const int d = x - hh * D;
        float M = s_m[0][hh];
#pragma unroll
        for (int q = 1; q < NW; ++q) M = fmaxf(M, s_m[q][hh]);
        float Ls = 0.0f, O = 0.0f;
#pragma unroll
        for (int q = 0; q < NW; ++q) {
            const float f = __builtin_amdgcn_exp2f(s_m[q][hh] - M);
            Ls += s_l[q][hh] * f;
            O += s_o[q][hh][d] * f;
        }
        const size_t row = (size_t)b * a.H_q + (size_t)g * G + hh;
        const float val = bad ? __builtin_nanf("") : O / Ls;
        if (a.n_parts == 1) {
            a.out[row * D + d] = val;
        } else {
            a.part_o[(row * a.n_parts + part) * D + d] = val;
            if (d == 0) a.part_lse[row * a.n_parts + part] = bad ? __builtin_nanf("") : M + __builtin_amdgcn_logf(Ls);
        }
    }
}

template <int QDT, int D, int NW, int CH>
static hipError_t launch_t(const AttnArgs& a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL((decode_mxfp4_mfma_kernel<QDT, D, NW, CH>), dim3(grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int QDT, int D>
static hipError_t launch_d(int nw, int ch, const AttnArgs& a, unsigned grid, hipStream_t s) {
    switch (nw * 10 + ch) {
    case 21: return launch_t<QDT, D, 2, 1>(a, grid, s);
    case 22: return launch_t<QDT, D, 2, 2>(a, grid, s);
    case 41: return launch_t<QDT, D, 4, 1>(a, grid, s);
    case 42: return launch_t<QDT, D, 4, 2>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_mxfp4_mfma(int q_dtype, int D, int nw, int ch, const AttnArgs& a, unsigned grid,
                                    hipStream_t stream) {
    switch (q_dtype * 1000 + D) {
    case DT_F16 * 1000 + 64: return launch_d<DT_F16, 64>(nw, ch, a, grid, stream);
    case DT_F16 * 1000 + 128: return launch_d<DT_F16, 128>(nw, ch, a, grid, stream);
    case DT_BF16 * 1000 + 64: return launch_d<DT_BF16, 64>(nw, ch, a, grid, stream);
    case DT_BF16 * 1000 + 128: return launch_d<DT_BF16, 128>(nw, ch, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

bool mxfp4_mfma_variant_exists(int nw, int ch) {
    const int v = nw * 10 + ch;
    return v == 21 || v == 22 || v == 41 || v == 42;
}

}  // namespace pkv
