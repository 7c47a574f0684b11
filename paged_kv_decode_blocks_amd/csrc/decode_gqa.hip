// decode_gqa.hip -- paged decode attention for grouped query heads on the
// gfx950 matrix cores.
//
// When G = H_q / H_kv query heads share one KV head, a workgroup that owns
// (request, KV head, partition) reads every K/V block once for all G heads, and
// the scores of a 16-token block form a real dense tile: S^T[16 tok][16 heads]
// = K[16 tok][D] * Q^T[D][16 heads] (heads >= G are zero padding).  Both
// products run as MFMA tiles, in f16 or bf16 with f32 accumulation:
//
//   scores  S^T = K Q^T   v_mfma_f32_16x16x32_{f16,bf16}, D/32 steps
//   output  O^T = V^T P^T v_mfma_f32_16x16x32_{f16,bf16}, D/16 tiles
//
// P is carried as hi + lo halves in the storage type (p = hi + lo to about
// 2^-17 relative for bf16), both in one K=32 product, so rounding P to bf16 does
// not cost output accuracy on short, peaked contexts.
//
// The tokens of a block are placed on the tile rows in the order
// rho = 4a + b <-> token 4b + a.  With that order the score tile that lane l
// holds (rows 4(l/16)+i, column l%16) is exactly the P^T operand that the
// second product needs (k index 4(l/16)+i, column l%16), and the V rows a lane
// needs for it (tokens 4i + l/16) are the ones a plain coalesced load of the
// block gives it.  The d index of the output tile is permuted the same way
// (row m of tile T is d = m*D/16 + T), so V is never transposed: the A operand
// of tile T is element T of the lane's four V loads, packed with v_perm.
//
// Softmax is online per query head in the log2 domain; the per-chunk max is
// shared by the four lane groups holding a head with two cross-row shuffles.
// Results merge across the waves of the workgroup through LDS, as in the
// per-head kernel, and the fused APPEND variant also writes the new token.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kWindowBlocksG = 256;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <int DT> struct Mfma;

template <> struct Mfma<DT_BF16> {
    static __device__ __forceinline__ floatx4 mma(const uint4& a, const uint4& b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
    }
    // p0, p1 -> packed (hi0, hi1) and packed (lo0, lo1) with p ~= hi + lo
    static __device__ __forceinline__ void split(float p0, float p1, uint32_t& hi, uint32_t& lo) {
        const bf162_t h = {(__bf16)p0, (__bf16)p1};
        const bf162_t r = {(__bf16)(p0 - (float)h.x), (__bf16)(p1 - (float)h.y)};
        hi = __builtin_bit_cast(uint32_t, h);
        lo = __builtin_bit_cast(uint32_t, r);
    }
};

template <> struct Mfma<DT_F16> {
    static __device__ __forceinline__ floatx4 mma(const uint4& a, const uint4& b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                      c, 0, 0, 0);
    }
    static __device__ __forceinline__ void split(float p0, float p1, uint32_t& hi, uint32_t& lo) {
        const half2_t h = {(_Float16)p0, (_Float16)p1};
        const half2_t r = {(_Float16)(p0 - (float)h.x), (_Float16)(p1 - (float)h.y)};
        hi = __builtin_bit_cast(uint32_t, h);
        lo = __builtin_bit_cast(uint32_t, r);
    }
};

// V load of VB bytes per lane (16 for D = 128, 8 for D = 64), as 32-bit words
template <int NWORD> struct VRow { uint32_t w[NWORD]; };

template <int NWORD>
__device__ __forceinline__ VRow<NWORD> ldv(const char* p) {
    VRow<NWORD> r;
    if constexpr (NWORD == 4) {
        uint4 v = ld16(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
        uint2 v = ld8(p);
        r.w[0] = v.x; r.w[1] = v.y;
    }
    return r;
}
template <int NWORD>
__device__ __forceinline__ VRow<NWORD> ldv_cached(const char* p) {
    VRow<NWORD> r;
    if constexpr (NWORD == 4) {
        uint4 v = ld16_cached(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
        uint2 v = *reinterpret_cast<const uint2*>(p);
        r.w[0] = v.x; r.w[1] = v.y;
    }
    return r;
}
template <int NWORD>
__device__ __forceinline__ void stv(char* p, const VRow<NWORD>& r) {
    if constexpr (NWORD == 4) st16(p, make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]));
    else st8(p, make_uint2(r.w[0], r.w[1]));
}

template <int DT, int D, int NW, int CH, bool APPEND>
__global__ __launch_bounds__(NW * 64) void decode_gqa_kernel(const AttnArgs a) {
    constexpr int ES = 2;
    constexpr int KS = D / 32;          // score MFMA steps
    constexpr int VT = D / 16;          // output tiles = V elements per lane per load
    constexpr int NWORD = VT / 2;       // 32-bit words per V load
    constexpr int DP = D + 4;           // padded LDS row
    static_assert(D == 64 || D == 128, "unsupported head dim");

    __shared__ int32_t s_ids[kWindowBlocksG];
    __shared__ int s_bad;
    __shared__ float s_m[NW][16];
    __shared__ float s_l[NW][16];
    __shared__ float s_o[NW][16][DP];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int j = lane >> 4;       // lane group: MFMA k-group / output row group
    const int col = lane & 15;     // MFMA column: query head within the group; also A-row

    const int BG = a.B * a.H_kv;
    const int part = blockIdx.x / BG;
    const int bg = blockIdx.x - part * BG;
    const int b = bg / a.H_kv;
    const int g = bg - b * a.H_kv;
    const int G = a.G;

    const int n = APPEND ? a.positions[b] + 1 : a.context_lens[b];
    const bool bad_len = APPEND ? (n < 1 || n > a.max_context_len) : (n < 0 || n > a.max_context_len);
    if (bad_len || n == 0) {
        if (a.n_parts == 1 && part == 0)
            for (int x = threadIdx.x; x < G * D; x += NW * 64)
                a.out[((size_t)b * a.H_q + (size_t)g * G) * D + x] = bad_len ? __builtin_nanf("") : 0.0f;
        return;
    }
    const int start = part * a.part_tokens;
    if (start >= n) return;
    const int end = min(start + a.part_tokens, n);
    const int n_hist = APPEND ? n - 1 : n;
    const int lim = min(end, n_hist);
    // only the partition that ends at n holds the new token; a chunk may run past
    // its partition's last block, so every other partition must never match it
    const int pos_new = (APPEND && end == n) ? n - 1 : -1;

    // Q^T fragments: column col = query head g*G + col, k = d = 32 s + 8 j .. +7
    uint4 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        qf[s] = make_uint4(0, 0, 0, 0);
        if (col < G)
            qf[s] = ld16_cached(a.q + ((int64_t)b * a.q_row_stride + (int64_t)(g * G + col) * D + 32 * s + 8 * j) * ES);
    }

    const int tau = 4 * (col & 3) + (col >> 2);          // token (within a block) on A-row `col`
    int koff[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) koff[s] = (tau * D + 32 * s + 8 * j) * ES;
    int voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[i] = ((4 * i + j) * D + col * VT) * ES;
    const size_t knew_off = ((size_t)b * a.new_row_stride + (size_t)g * D) * ES;

    floatx4 acc[VT];
#pragma unroll
    for (int t = 0; t < VT; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = kNegBig, l = 0.0f;

    const int32_t* table = a.block_tables + (int64_t)b * a.bt_stride;
    const int first_blk = start / kBlockSize;
    const int nblk = (end - start + kBlockSize - 1) / kBlockSize;
    const size_t blk_bytes = (size_t)a.H_kv * kBlockSize * D * ES;
    const size_t head_bytes = (size_t)g * kBlockSize * D * ES;

    if (threadIdx.x == 0) s_bad = 0;
    for (int r0 = 0; r0 < nblk; r0 += kWindowBlocksG) {
        const int nr = min(kWindowBlocksG, nblk - r0);
        __syncthreads();
        for (int t = threadIdx.x; t < nr; t += NW * 64) {
            int id = table[first_blk + r0 + t];
            if ((unsigned)id >= (unsigned)a.n_blocks) {
                s_bad = 1;
                id = 0;
            }
            s_ids[t] = id;
        }
        __syncthreads();
        const bool any_bad = s_bad != 0;
        const int nch = (nr + CH - 1) / CH;
        for (int k = w; k < nch; k += NW) {
            const int cb0 = k * CH;
            const int tok0 = start + (r0 + cb0) * kBlockSize;
            const char* kb[CH];
            const char* vb[CH];
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) {
                const int id = __builtin_amdgcn_readfirstlane(cb0 + cb < nr ? s_ids[cb0 + cb] : 0);
                kb[cb] = a.k_pool + (size_t)id * blk_bytes + head_bytes;
                vb[cb] = a.v_pool + (size_t)id * blk_bytes + head_bytes;
            }
            uint4 kf[CH][KS];
            VRow<NWORD> vf[CH][4];
            bool valid[CH][4];
            const bool fast = tok0 + CH * kBlockSize <= lim;
            if (fast) {
#pragma unroll
                for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                    for (int s = 0; s < KS; ++s) kf[cb][s] = ld16(kb[cb] + koff[s]);
#pragma unroll
                for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) vf[cb][i] = ldv<NWORD>(vb[cb] + voff[i]);
#pragma unroll
                for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) valid[cb][i] = true;
            } else {
#pragma unroll
                for (int cb = 0; cb < CH; ++cb) {
                    const int tb = tok0 + cb * kBlockSize;
                    const int tk = tb + tau;
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        kf[cb][s] = make_uint4(0, 0, 0, 0);
                        if (tk < lim) {
                            kf[cb][s] = ld16(kb[cb] + koff[s]);
                        } else if (APPEND && tk == pos_new) {
                            kf[cb][s] = ld16_cached(a.k_new + knew_off + (32 * s + 8 * j) * ES);
                            if (!any_bad) st16(a.k_pool_w + (kb[cb] - a.k_pool) + koff[s], kf[cb][s]);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tv = tb + 4 * i + j;
#pragma unroll
                        for (int x = 0; x < NWORD; ++x) vf[cb][i].w[x] = 0;
                        valid[cb][i] = false;
                        if (tv < lim) {
                            vf[cb][i] = ldv<NWORD>(vb[cb] + voff[i]);
                            valid[cb][i] = true;
                        } else if (APPEND && tv == pos_new) {
                            vf[cb][i] = ldv_cached<NWORD>(a.v_new + knew_off + col * VT * ES);
                            valid[cb][i] = true;
                            if (!any_bad) stv<NWORD>(a.v_pool_w + (vb[cb] - a.v_pool) + voff[i], vf[cb][i]);
                        }
                    }
                }
            }
            // scores: lane holds S[head col][token tb + 4 i + j], i = 0..3
            float sc[CH][4];
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) {
                floatx4 st = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < KS; ++s) st = Mfma<DT>::mma(kf[cb][s], qf[s], st);
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[cb][i] = mul_rn(st[i], a.scale_log2);
            }
            float mloc = kNegBig;
#pragma unroll
            for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) mloc = valid[cb][i] ? fmaxf(mloc, sc[cb][i]) : mloc;
            mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
            const float m_new = fmaxf(m, mloc);
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int t = 0; t < VT; ++t) acc[t] *= alpha;
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = valid[cb][i] ? __builtin_amdgcn_exp2f(sc[cb][i] - m) : 0.0f;
                    l += p[i];
                }
                // P^T operand: the k slots hold (hi of tokens 0..3, lo of tokens 0..3); the V^T
                // operand repeats its four tokens, so one K=32 product adds V*hi + V*lo
                uint4 pk;
                Mfma<DT>::split(p[0], p[1], pk.x, pk.z);
                Mfma<DT>::split(p[2], p[3], pk.y, pk.w);
#pragma unroll
                for (int t = 0; t < VT; ++t) {
                    const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
                    const int x = t >> 1;
                    const uint32_t v01 = __builtin_amdgcn_perm(vf[cb][1].w[x], vf[cb][0].w[x], sel);
                    const uint32_t v23 = __builtin_amdgcn_perm(vf[cb][3].w[x], vf[cb][2].w[x], sel);
                    acc[t] = Mfma<DT>::mma(make_uint4(v01, v23, v01, v23), pk, acc[t]);
                }
            }
        }
    }

    // per-head sum over the four lane groups (they share m)
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (j == 0) {
        s_m[w][col] = m;
        s_l[w][col] = l;
    }
#pragma unroll
    for (int t = 0; t < VT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[w][col][(4 * j + i) * VT + t] = acc[t][i];
    __syncthreads();
    const bool bad = s_bad != 0;
    for (int x = threadIdx.x; x < G * D; x += NW * 64) {
        const int hh = x / D;
        const int d = x - hh * D;
        float M = s_m[0][hh];
#pragma unroll
        for (int i = 1; i < NW; ++i) M = fmaxf(M, s_m[i][hh]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const float f = __builtin_amdgcn_exp2f(s_m[i][hh] - M);
            L += s_l[i][hh] * f;
            O += s_o[i][hh][d] * f;
        }
        const size_t row = (size_t)b * a.H_q + (size_t)g * G + hh;
        const float val = bad ? __builtin_nanf("") : O / L;
        if (a.n_parts == 1) {
            a.out[row * D + d] = val;
        } else {
            a.part_o[(row * a.n_parts + part) * D + d] = val;
            // v_log_f32 is log base 2, matching the log2-domain scores
            if (d == 0) a.part_lse[row * a.n_parts + part] = bad ? __builtin_nanf("") : M + __builtin_amdgcn_logf(L);
        }
    }
}

template <int DT, int D, int NW, int CH>
static hipError_t launch_gqa_t(bool append, const AttnArgs& a, unsigned grid, hipStream_t stream) {
    if (append)
        hipLaunchKernelGGL((decode_gqa_kernel<DT, D, NW, CH, true>), dim3(grid), dim3(NW * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_gqa_kernel<DT, D, NW, CH, false>), dim3(grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_gqa_d(int nw, int ch, bool append, const AttnArgs& a, unsigned grid, hipStream_t s) {
    switch (nw * 10 + ch) {
    case 21: return launch_gqa_t<DT, D, 2, 1>(append, a, grid, s);
    case 22: return launch_gqa_t<DT, D, 2, 2>(append, a, grid, s);
    case 41: return launch_gqa_t<DT, D, 4, 1>(append, a, grid, s);
    case 42: return launch_gqa_t<DT, D, 4, 2>(append, a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_gqa(int dtype, int D, int nw, int ch, bool append, const AttnArgs& a,
                             unsigned grid, hipStream_t stream) {
    switch (dtype * 1000 + D) {
    case DT_F16 * 1000 + 64: return launch_gqa_d<DT_F16, 64>(nw, ch, append, a, grid, stream);
    case DT_F16 * 1000 + 128: return launch_gqa_d<DT_F16, 128>(nw, ch, append, a, grid, stream);
    case DT_BF16 * 1000 + 64: return launch_gqa_d<DT_BF16, 64>(nw, ch, append, a, grid, stream);
    case DT_BF16 * 1000 + 128: return launch_gqa_d<DT_BF16, 128>(nw, ch, append, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

bool gqa_variant_exists(int nw, int ch) {
    return (nw == 2 || nw == 4) && (ch == 1 || ch == 2);
}

}  // namespace pkv
