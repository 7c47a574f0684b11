// decode_mxfp4_mfma.hip -- paged decode attention over an MXFP4 K/V cache on the
// gfx950 matrix cores, one workgroup per (partition, request, group of KV heads)
// -- or, for an even split of the batch, per (run of blocks, group of KV heads) --
// each KV head serving its G <= 16 query heads.
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
// the 16-bit grouped kernel; the waves of a head merge through LDS; the result
// goes to the output or, when split, to the log-sum-exp merge.  In the fused
// step the new token is quantized inside the kernel, in the wave whose ring slot
// holds its block (see APPEND below), so the step is one launch plus the merge.
#include "pkv_mxfp4.h"
#include "pkv_launch.h"

namespace pkv {

namespace {

constexpr int kWin = 256;                 // block ids staged per window
constexpr float kSlack = 8.0f;            // log2 units: weights stay below 256

template <bool B>
struct Flag { static constexpr bool value = B; };

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx4 mma_bf16(const uint4& a, const uint4& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// (p0, p1) -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float p0, float p1) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){p0, p1}, bf162_t));
}

// p0, p1 -> packed bf16 (hi0, hi1) and (lo0, lo1) with p ~= hi + lo (to ~2^-17)
__device__ __forceinline__ void split_bf16(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16(p0, p1);
    lo = pack_bf16(p0 - __uint_as_float(hi << 16), p1 - __uint_as_float(hi & 0xffff0000u));
}

// One half of split_bf16 per lane: the hi pair when lo_mul = 0, the lo pair when
// lo_mul = 1 (p - 1 * hi is exact, p - 0 * hi is p).
__device__ __forceinline__ uint32_t split_half_bf16(float p0, float p1, float lo_mul) {
    const uint32_t hi = pack_bf16(p0, p1);
    return pack_bf16(fmaf(-lo_mul, __uint_as_float(hi << 16), p0),
                     fmaf(-lo_mul, __uint_as_float(hi & 0xffff0000u), p1));
}

// Max / sum over the four lane groups (lanes 16 apart) with the gfx950 lane swaps:
// v_permlane16_swap pairs rows 0-1 and 2-3, v_permlane32_swap pairs the halves.
__device__ __forceinline__ float max_groups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_groups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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
// byte X of a word of codes -> one packed bf16 pair (elements 2X, 2X + 1), scaled
template <int X>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16(uint32_t w, float sc) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, X));
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

// CH blocks as read from LDS: K codes of the lane's row, its scale byte, and the
// codes and scale bytes of its four V rows.
template <int D, int CH>
struct Mx4Chunk {
    uint32_t k[CH][Mx4Geo<D>::KW];
    uint32_t ks[CH];
    uint32_t v[CH][4];                         // VB bytes used (4 for D = 128, 2 for D = 64)
    uint32_t vs[CH][4];
};

// LO: G <= 8, and columns [G, 2G) of both products repeat heads [0, G): their
// scores, maxima and weights are the same numbers, and they carry the lo half of
// P while columns [0, G) carry the hi half, so one K=32 output product takes 32
// distinct tokens (two blocks) and the halves are added once at the end.
// Otherwise (G <= 16) hi and lo share a product's k-slots, one block at a time.
template <int QDT, int D, bool LO>
struct Mx4Lane {
    using Geo = Mx4Geo<D>;
    static constexpr int KS = Geo::KS, VT = Geo::VT, NQ = QDT == DT_F16 ? 2 : 1;
    int j, c;
    float lo_mul;              // 1 if this lane's column carries the lo half of P, else 0
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
        lo_mul = (LO && c >= a.G) ? 1.0f : 0.0f;
        if (c < (LO ? 2 : 1) * a.G) {
            const int h = c < a.G ? c : c - a.G;
            const char* qp = a.q + ((int64_t)b * a.q_row_stride + (int64_t)(g * a.G + h) * D + 8 * KS * j) * 2;
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

    // Score tile of block cb (lane holds tokens 4 i + j of its column), log2 domain.
    template <int CH>
    __device__ __forceinline__ void scores(const Mx4Chunk<D, CH>& ck, int cb, float (&sc)[4]) {
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
        for (int i = 0; i < 4; ++i) sc[i] = mul_rn(st[i], scale_log2);
    }

    // V rows of the lane's four tokens of block cb, decoded with their scales: word
    // x of row i holds elements (2x, 2x + 1) of the lane's piece.
    template <int CH>
    __device__ __forceinline__ void vrows(const Mx4Chunk<D, CH>& ck, int cb, uint32_t (&vd)[4][VT / 2]) {
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
    }

    // Shared max of the chunk and the lazy rescale; returns nothing, updates m, l, acc.
    template <int CH, bool MASK>
    __device__ __forceinline__ void rescale(const float (&sc)[CH][4], const bool (&valid)[CH][4]) {
        float mloc = kNegBig;
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mloc = (!MASK || valid[cb][i]) ? fmaxf(mloc, sc[cb][i]) : mloc;
        mloc = max_groups(mloc);
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
    }

    // LO: two blocks, 32 tokens in one K=32 output product per tile, in two stages
    // so that a wave overlaps one chunk's score products with the previous
    // chunk's softmax and output products (the caller runs scores(i) and
    // finish(i - 1) back to back, in one basic block).
    struct PairStage {
        uint32_t v[2][4];      // V code words of the lane's four tokens, per block
        uint32_t vs[2][4];     // their scale bytes; 0 (2^-127, finite) for masked tokens
        float sc[2][4];        // scores, log2 domain; -inf for masked tokens
    };

    __device__ __forceinline__ void pair_scores(const Mx4Chunk<D, 2>& ck, PairStage& ps) {
        scores<2>(ck, 0, ps.sc[0]);
        scores<2>(ck, 1, ps.sc[1]);
    }

    // Softmax update and output products of a chunk whose scores are in ps.  Masked
    // tokens carry a score of -inf, so they take no part in the max and get weight
    // exp2(-inf) = 0 (m is always finite), and their V rows decode to finite values
    // (scale byte 0), so their K and V bytes (unwritten slots hold NaN scale bytes)
    // never reach the accumulators.
    __device__ __forceinline__ void pair_finish(const PairStage& ps) {
        const bool unused[2][4] = {};   // no mask: masked scores are -inf
        rescale<2, false>(ps.sc, unused);
        uint32_t pw[2][2];     // per block: packed weights of tokens (0, 1) and (2, 3), hi or lo half
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = __builtin_amdgcn_exp2f(ps.sc[cb][i] - m);
                l += p[i];
            }
            pw[cb][0] = split_half_bf16(p[0], p[1], lo_mul);
            pw[cb][1] = split_half_bf16(p[2], p[3], lo_mul);
        }
        const uint4 pk = make_uint4(pw[0][0], pw[0][1], pw[1][0], pw[1][1]);
        float vsc[2][4];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) vsc[cb][i] = mx_operand(ps.vs[cb][i]);
        pv_pair<0>(ps, vsc, pk);
        if constexpr (VT / 2 > 1) pv_pair<1>(ps, vsc, pk);
        if constexpr (VT / 2 > 2) pv_pair<2>(ps, vsc, pk);
        if constexpr (VT / 2 > 3) pv_pair<3>(ps, vsc, pk);
    }

    // Output tiles 2X and 2X + 1 of a two-block chunk: byte X of each V piece.
    template <int X>
    __device__ __forceinline__ void pv_pair(const PairStage& ps, const float (&vsc)[2][4], const uint4& pk) {
        uint32_t d0[4], d1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d0[i] = e2m1x2_to_bf16<X>(ps.v[0][i], vsc[0][i]);
            d1[i] = e2m1x2_to_bf16<X>(ps.v[1][i], vsc[1][i]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t sel = h ? 0x07060302u : 0x05040100u;
            const uint32_t a01 = __builtin_amdgcn_perm(d0[1], d0[0], sel);
            const uint32_t a23 = __builtin_amdgcn_perm(d0[3], d0[2], sel);
            const uint32_t b01 = __builtin_amdgcn_perm(d1[1], d1[0], sel);
            const uint32_t b23 = __builtin_amdgcn_perm(d1[3], d1[2], sel);
            acc[2 * X + h] = mma_bf16(make_uint4(a01, a23, b01, b23), pk, acc[2 * X + h]);
        }
    }

    // Not LO: one block at a time, hi and lo halves of P in the k-slots of one product.
    template <bool MASK>
    __device__ __forceinline__ void accumulate(const Mx4Chunk<D, 1>& ck, const bool (&valid)[1][4]) {
        float sc[1][4];
        scores<1>(ck, 0, sc[0]);
        rescale<1, MASK>(sc, valid);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = (!MASK || valid[0][i]) ? __builtin_amdgcn_exp2f(sc[0][i] - m) : 0.0f;
            l += p[i];
        }
        uint4 pk;
        split_bf16(p[0], p[1], pk.x, pk.z);
        split_bf16(p[2], p[3], pk.y, pk.w);
        uint32_t vd[4][VT / 2];
        vrows<1>(ck, 0, vd);
#pragma unroll
        for (int t = 0; t < VT; ++t) {
            const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
            const int x = t >> 1;
            const uint32_t v01 = __builtin_amdgcn_perm(vd[1][x], vd[0][x], sel);
            const uint32_t v23 = __builtin_amdgcn_perm(vd[3][x], vd[2][x], sel);
            acc[t] = mma_bf16(make_uint4(v01, v23, v01, v23), pk, acc[t]);
        }
    }
};

}  // namespace

// global -> LDS, 4 or 16 bytes per active lane: lane l writes lds_base + 4 l or
// 16 l (lds_base wave-uniform).  The LDS address-space cast only means something
// in the device pass; in the host pass it would drop the kernel's launch stub.
__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
#else
    (void)src;
    (void)lds_base;
#endif
}
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
#else
    (void)src;
    (void)lds_base;
#endif
}

// s_waitcnt vmcnt(N), other counters unconstrained (gfx9: vmcnt in bits [3:0] and [15:14])
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Wait until at most n chunks' DMAs (LPC instructions each) are outstanding, for a
// runtime n in [0, MAXN]: DMAs complete in issue order, so this is the exact wait
// for the oldest chunk when n later chunks have been issued after it.
template <int LPC, int MAXN>
__device__ __forceinline__ void wait_chunks(int n) {
    if constexpr (MAXN >= 3) {
        if (n >= 3) { wait_vm<3 * LPC>(); return; }
    }
    if constexpr (MAXN >= 2) {
        if (n == 2) { wait_vm<2 * LPC>(); return; }
    }
    if constexpr (MAXN >= 1) {
        if (n == 1) { wait_vm<LPC>(); return; }
    }
    wait_vm<0>();
}

template <int N>
struct SlotTag {
    static constexpr int value = N;
};
// f(SlotTag<s>{}) for a wave-uniform ring slot s < R: a chain of uniform branches
// that folds away where s is a constant, so that per-slot registers are never
// indexed at run time
template <int R, int N = R - 1, typename F>
__device__ __forceinline__ void on_slot(int s, F&& f) {
    static_assert(N >= 0 && N < R, "ring slot");
    if constexpr (N == 0) {
        f(SlotTag<0>{});
    } else {
        if (s == N) {
            f(SlotTag<N>{});
            return;
        }
        on_slot<R, N - 1>(s, f);
    }
}

// One block's loads in flight through registers (register staging): K codes (16
// bytes per lane, 8 for D = 64), V codes (16, or two words), the lane's scale word.
struct Mx4Stage {
    uint32_t k[4], v[4], s;
};
// Up to ten stages as named members: reached through at<I>() with a constant I,
// never through an index, so that they stay in registers.
struct Mx4StageRing {
    Mx4Stage x0, x1, x2, x3, x4, x5, x6, x7, x8, x9;
    template <int I>
    __device__ __forceinline__ Mx4Stage& at() {
        static_assert(I >= 0 && I < 10, "stage");
        if constexpr (I == 0) return x0;
        else if constexpr (I == 1) return x1;
        else if constexpr (I == 2) return x2;
        else if constexpr (I == 3) return x3;
        else if constexpr (I == 4) return x4;
        else if constexpr (I == 5) return x5;
        else if constexpr (I == 6) return x6;
        else if constexpr (I == 7) return x7;
        else if constexpr (I == 8) return x8;
        else return x9;
    }
};

// Register staging: a block's codes and scales are loaded into registers and written
// into its ring slot by the wave itself, at the places a DMA would have filled, once
// the chunk's loads have landed.  At two waves per SIMD a wave stream that moves
// every piece by global_load_lds reads markedly slower than one that loads into
// registers (the tile-read probe), so the loads go through registers -- for one chunk
// in flight (PF = 1); two or more do not fit beside the kernel's other registers and
// keep the DMA.  Every load of a chunk is issued by every lane, none behind a branch:
// the compiler counts outstanding loads exactly only then, and otherwise waits for
// some of the next chunk's loads before writing this one (which undid the gain).
constexpr bool kMx4RegisterStaging = true;

// One block of the ring -> registers in the MFMA layout, completed before return.
// Issued as inline asm: the compiler cannot tell this slot from the DMAs still in
// flight into the other slots and would drain every load before a plain LDS read;
// the caller's vmcnt wait orders these reads after the DMAs that filled the slot.
// The outputs are early-clobber: a read's destination must not share a register
// with an address that a later read of the same statement still uses.
// Offsets: K codes at ka (16 bytes; for D = 64 two words at ka and ka + 256), K scale byte at ksa, V pieces at va +
// i * VSTEP (4 or 2 bytes), V scale bytes at vsa + i * SSTEP.
template <int D>
__device__ __forceinline__ void lds_block(uint32_t ka, uint32_t ksa, uint32_t va, uint32_t vsa,
                                          uint32_t (&k)[Mx4Geo<D>::KW], uint32_t& ks, uint32_t (&v)[4],
                                          uint32_t (&vs)[4]) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int VSTEP = 4 * Mx4Geo<D>::RB, SSTEP = 4 * Mx4Geo<D>::SB;
    if constexpr (D == 128) {
        u32x4_t kk;
        asm volatile(
            "ds_read_b128 %0, %10\n\t"
            "ds_read_u8 %1, %11\n\t"
            "ds_read_b32 %2, %12\n\t"
            "ds_read_b32 %3, %12 offset:%14\n\t"
            "ds_read_b32 %4, %12 offset:%15\n\t"
            "ds_read_b32 %5, %12 offset:%16\n\t"
            "ds_read_u8 %6, %13\n\t"
            "ds_read_u8 %7, %13 offset:%17\n\t"
            "ds_read_u8 %8, %13 offset:%18\n\t"
            "ds_read_u8 %9, %13 offset:%19\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(kk), "=&v"(ks), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(vs[0]), "=&v"(vs[1]),
              "=&v"(vs[2]), "=&v"(vs[3])
            : "v"(ka), "v"(ksa), "v"(va), "v"(vsa), "i"(VSTEP), "i"(2 * VSTEP), "i"(3 * VSTEP), "i"(SSTEP),
              "i"(2 * SSTEP), "i"(3 * SSTEP)
            : "memory");
        k[0] = kk.x; k[1] = kk.y; k[2] = kk.z; k[3] = kk.w;
    } else {   // the lane's two K words are at ka and ka + 256 (two dword DMAs)
        asm volatile(
            "ds_read_b32 %0, %11\n\t"
            "ds_read_b32 %1, %11 offset:256\n\t"
            "ds_read_u8 %2, %12\n\t"
            "ds_read_u16 %3, %13\n\t"
            "ds_read_u16 %4, %13 offset:%15\n\t"
            "ds_read_u16 %5, %13 offset:%16\n\t"
            "ds_read_u16 %6, %13 offset:%17\n\t"
            "ds_read_u8 %7, %14\n\t"
            "ds_read_u8 %8, %14 offset:%18\n\t"
            "ds_read_u8 %9, %14 offset:%19\n\t"
            "ds_read_u8 %10, %14 offset:%20\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(k[0]), "=&v"(k[1]), "=&v"(ks), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(vs[0]),
              "=&v"(vs[1]), "=&v"(vs[2]), "=&v"(vs[3])
            : "v"(ka), "v"(ksa), "v"(va), "v"(vsa), "i"(VSTEP), "i"(2 * VSTEP), "i"(3 * VSTEP), "i"(SSTEP),
              "i"(2 * SSTEP), "i"(3 * SSTEP)
            : "memory");
    }
#else
    (void)ka; (void)ksa; (void)va; (void)vsa;
    for (int x = 0; x < Mx4Geo<D>::KW; ++x) k[x] = 0;
    ks = 0;
    for (int i = 0; i < 4; ++i) v[i] = vs[i] = 0;
#endif
}

// Each wave streams its blocks through a ring of R = PF + 1 LDS chunk slots, PF
// chunks ahead of the one it computes (for PF = 1 the loads go through registers
// and the wave writes them into the slot, kMx4RegisterStaging; deeper rings load by
// DMA).  A slot holds one block of the KV head: K codes placed so that lane l's 16
// bytes sit at 16 l (for D = 64 its two words at 4 l and 256 + 4 l) -- the lane that
// fetches them is lane l, so the read is conflict-free -- then V codes, K scales and
// V scales in pool order.  Every load stays inside the block's rows of this KV head;
// rows at or past the length are masked after the read, so the last, partial block
// needs no other path.
//
// HG: KV heads per workgroup.  Wave w streams head g0 + w % HG over blocks w / HG,
// w / HG + NW / HG, ... of the partition, so the HG heads' 1 KiB code tiles of a
// block -- neighbours in the pool -- are read together as one HG KiB piece; HG = 1 is
// one head per workgroup, its blocks round-robin over the waves.  The waves of a head
// then merge through LDS.
//
// EVEN (HG = NW): the even split of the batch.  The requests' blocks, end to end in
// request order, are cut into `runs` equal runs of tw blocks; workgroup (S, hg) takes
// run S for KV heads hg NW .. hg NW + NW - 1, wave w head hg NW + w.  Every wave
// streams the same number of blocks whatever the length mix, the grid is one resident
// round, and a block's NW head tiles are read together.  The waves walk the run's
// pieces (its overlap with each request) in step, each with a fresh softmax state per
// piece; a piece that is a whole request is written as the output, any other as piece
// (S + b) H_kv + g of request b -- rows part_o[(((S + b) H_kv + g) G + h) D ...] and
// part_lse[((S + b) H_kv + g) G + h] -- which the merge kernel combines in run order (a
// run and a request meet in one interval, and along the end-to-end order S and b only
// grow, so S + b names each meeting once).  Every workgroup prefix-sums the requests'
// block counts in LDS (lengths out of range count as empty: the merge writes their
// rows); workgroup 0 stores tw, the runs used and the prefix for the merge.
template <int QDT, int D, int NW, int PF, bool LO, bool APPEND, int HG, bool EVEN>
__global__ __launch_bounds__(NW * 64, 2)
void decode_mxfp4_mfma_kernel(const AttnArgs a) {
    using Geo = Mx4Geo<D>;
    using L = Mx4Lane<QDT, D, LO>;
    constexpr int RB = Geo::RB, SB = Geo::SB, VT = Geo::VT;
    constexpr int CH = LO ? 2 : 1;                         // blocks per chunk (one output product)
    constexpr int R = PF + 1;                              // chunk slots per wave
    constexpr int CODES = kBlockSize * RB;                 // bytes of one tile of codes
    constexpr int SLOT = 2 * CODES + 2 * kBlockSize * SB;  // K codes, V codes, K scales, V scales
    constexpr bool RS = kMx4RegisterStaging && PF == 1;   // deeper rings do not fit the registers
    constexpr int LPB = D == 128 ? 3 : RS ? 4 : 5;         // load instructions per block
    constexpr int LPC = CH * LPB;
    static_assert(PF * LPC < 64, "vmcnt range");
    static_assert(NW % HG == 0, "a workgroup's waves split evenly over its heads");
    static_assert(!EVEN || HG == NW, "the even split streams one head per wave");
    static_assert(kEvenMaxWaveBlocks <= kWin, "a run's block ids fit one window");
    constexpr int BW = NW / HG;                            // waves per head
    constexpr int T = NW * 64;
    constexpr int RING = NW * R * CH * SLOT;
    constexpr int MERGE = EVEN ? 0 : NW * 16 * (D + 4) * 4;
    constexpr int PER = EVEN ? kEvenMaxBatch / T + 1 : 1;  // requests per thread in the prefix sum (covers index B)
    __shared__ __attribute__((aligned(16))) char s_ring[RING > MERGE ? RING : MERGE];
    __shared__ uint32_t s_ids[kWin];   // block offsets in 256-byte units of the code pools
    __shared__ int s_bad;
    __shared__ float s_m[EVEN ? 1 : NW][16];
    __shared__ float s_l[EVEN ? 1 : NW][16];
    __shared__ uint8_t s_new[HG][2][APPEND ? D / 2 : 1];    // APPEND: per head, the new K and V rows' codes ...
    __shared__ uint8_t s_nsc[HG][2][APPEND ? D / 32 : 1];   // ... and scale bytes
    __shared__ int32_t s_pre[EVEN ? PER * T : 1];           // EVEN: blocks before each request
    __shared__ int32_t s_scan[EVEN ? T : 1];
    __shared__ int s_badw[EVEN ? NW : 1];                   // EVEN: a wave's lanes saw a bad id

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hs = w % HG;                      // the wave's head slot
    const int wi = w / HG;                      // ... and its place among that head's waves
    const int HGS = a.H_kv / HG;                // head groups per request
    // the workgroup's unit: (partition, request, head group), or EVEN (run, head group)
    int part = 0, b = 0, S = 0, g0;
    if constexpr (EVEN) {
        S = blockIdx.x / HGS;
        g0 = (blockIdx.x - S * HGS) * HG;
    } else {
        const int BG = a.B * HGS;
        const int unit = xcd_pair_unit(blockIdx.x, a.n_parts * BG);
        const int pg = unit / BG;
        part = unit_part(a, pg);
        const int bg = unit - pg * BG;
        b = bg / HGS;
        g0 = (bg - b * HGS) * HG;
    }
    const int g = g0 + hs;                      // the wave's KV head

    L st;
    // The tokens being streamed: request length n, bound lim (tokens at or past it
    // are masked), blocks nblk.  APPEND: when they end at n, the new token (position
    // n - 1, row t_new of the last block) is quantized here from k_new / v_new by the
    // wave of each head that owns that block (a head's blocks go round-robin over its
    // BW waves and a window holds a multiple of BW blocks), exactly as the append
    // kernel would: it writes the codes into the block's ring slot before the slot is
    // read, and to the pools (this workgroup is the only one holding that position of
    // its KV heads).
    int n = 0, lim = 0, nblk = 0, t_new = 0;
    bool new_wave = false;

    const int j = lane >> 4, c = lane & 15;     // the lane's row group and column (as st.init sets them)
    const int tau = 4 * (c & 3) + (c >> 2);
    // DMA sources inside one (block, KV head) tile
    const int kdma = D == 128 ? tau * RB + 16 * j : tau * RB + 8 * j;   // + 4 h for D = 64
    const bool sc_lane = lane < 8 * SB;                                  // 4 SB lanes per scale tile
    const int sdma = lane < 4 * SB ? 4 * lane : 4 * (lane - 4 * SB);
    // A block of a code pool is H_kv * 16 * D / 2 bytes, a multiple of 256, and its
    // scales 1/16 of that: the window stages id * blk_units (exact; below 2^32 for
    // pools under 1 TiB), and a DMA address is one shift-add of it.
    const uint32_t blk_units = (uint32_t)a.H_kv * kBlockSize * RB / 256;
    const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.k_pool) + (size_t)g * kBlockSize * RB;
    const uint8_t* vp = reinterpret_cast<const uint8_t*>(a.v_pool) + (size_t)g * kBlockSize * RB;
    const uint8_t* sp = (lane < 4 * SB ? a.k_mx_scale : a.v_mx_scale) + (size_t)g * kBlockSize * SB + sdma;
    // LDS read offsets inside a slot
    const uint32_t ring0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)s_ring;
    const uint32_t k_rd = (D == 128 ? 16 : 4) * lane;
    const uint32_t ks_rd = 2 * CODES + tau * SB + (Geo::KS * j) / 4;
    const uint32_t v_rd = CODES + j * RB + c * Geo::VB;
    const uint32_t vs_rd = 2 * CODES + kBlockSize * SB + j * SB + (c * VT) / 32;
    char* my_ring = s_ring + w * R * CH * SLOT;
    const uint32_t my_ring_a = ring0 + w * R * CH * SLOT;

    // APPEND: the new K and V rows of (b, g), quantized into the wave's small LDS area
    // (lane l: elements 2l and 2l + 1, one row per pass); copied into the ring slot once
    // the block's DMAs have landed there
    auto quantize_new = [&]() {
        const bool on = lane < D / 2;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            float x0 = 0.0f, x1 = 0.0f;
            if (on) {
                const uint32_t u = *reinterpret_cast<const uint32_t*>(
                    (which ? a.v_new : a.k_new) + ((size_t)b * a.new_row_stride + (size_t)g * D + 2 * lane) * 2);
                if constexpr (QDT == DT_F16) {
                    const half2_t h = __builtin_bit_cast(half2_t, u);
                    x0 = (float)h.x;
                    x1 = (float)h.y;
                } else {
                    x0 = __uint_as_float(u << 16);
                    x1 = __uint_as_float(u & 0xffff0000u);
                }
            }
            int E;
            const uint32_t code = mx4_quantize_pair(x0, x1, E);
            if (on) {
                s_new[hs][which][lane] = (uint8_t)code;
                if ((lane & 15) == 0) s_nsc[hs][which][lane / 16] = (uint8_t)(E + 127);
            }
        }
    };

    // APPEND: put the new rows in row t_new of ring slot sl, at the places the
    // block's DMAs fill (after they have landed there); the pools get them after
    // the loop
    auto put_new = [&](int sl) {
        if (lane < D / 2) {
            char* dst = my_ring + sl * SLOT;
            const int cn = 4 * (t_new & 3) + (t_new >> 2);   // the lane column whose K row is t_new
            const int kpos = D == 128 ? 256 * (lane / 16) + 16 * cn + (lane % 16)
                                      : 256 * ((lane % 8) / 4) + 4 * (16 * (lane / 8) + cn) + (lane % 4);
            dst[kpos] = (char)s_new[hs][0][lane];
            dst[CODES + t_new * RB + lane] = (char)s_new[hs][1][lane];
            if ((lane & 15) == 0) {
                dst[2 * CODES + t_new * SB + lane / 16] = (char)s_nsc[hs][0][lane / 16];
                dst[2 * CODES + kBlockSize * SB + t_new * SB + lane / 16] = (char)s_nsc[hs][1][lane / 16];
            }
        }
        // this wave's LDS writes land before its reads of the slot (in order per wave)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // APPEND: the new rows to the pools, from each head's owner wave (s_ids still holds
    // the window with the new token's block)
    auto write_new = [&]() {
        if (lane < D / 2) {
            const size_t u = s_ids[(nblk - 1) % kWin];
            const size_t row = (size_t)g * kBlockSize * RB + (u << 8) + (size_t)t_new * RB + lane;
            reinterpret_cast<uint8_t*>(a.k_pool_w)[row] = s_new[hs][0][lane];
            reinterpret_cast<uint8_t*>(a.v_pool_w)[row] = s_new[hs][1][lane];
            if ((lane & 15) == 0) {
                const size_t srow = (size_t)g * kBlockSize * SB + (u << 4) + (size_t)t_new * SB + lane / 16;
                a.k_mx_scale_w[srow] = s_nsc[hs][0][lane / 16];
                a.v_mx_scale_w[srow] = s_nsc[hs][1][lane / 16];
            }
        }
    };

    // RS: R slots of CH blocks in flight through registers
    static_assert(!RS || R * CH <= 10, "stage ring");
    static_assert((8 * SB & (8 * SB - 1)) == 0, "scale lanes a power of two");
    const int l_sc = lane & (8 * SB - 1);   // the scale lane this lane repeats
    const uint8_t* sp_all = (l_sc < 4 * SB ? a.k_mx_scale : a.v_mx_scale) + (size_t)g * kBlockSize * SB +
                            4 * (l_sc & (4 * SB - 1));
    Mx4StageRing stg;
    auto load_block = [&](Mx4Stage& sg, int blk) __attribute__((always_inline)) {
        const uint64_t u = (uint32_t)__builtin_amdgcn_readfirstlane(s_ids[blk]);
        const uint64_t co = u << 8, so = u << 4;
        if constexpr (D == 128) {
            const u32x4_t kk = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + co + kdma));
            const u32x4_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vp + co + 16 * lane));
            sg.k[0] = kk.x; sg.k[1] = kk.y; sg.k[2] = kk.z; sg.k[3] = kk.w;
            sg.v[0] = vv.x; sg.v[1] = vv.y; sg.v[2] = vv.z; sg.v[3] = vv.w;
        } else {   // the lane's two K words are adjacent (kdma is a multiple of 8)
            const u32x2_t kk = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(kp + co + kdma));
            sg.k[0] = kk.x; sg.k[1] = kk.y;
            sg.v[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vp + co + 4 * lane));
            sg.v[1] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vp + co + 256 + 4 * lane));
        }
        // every lane loads a scale word (lanes past the first 8 SB repeat theirs), so that no
        // load sits behind a branch the compiler's wait counting must allow for
        sg.s = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sp_all + so));
    };
    auto land_block = [&](const Mx4Stage& sg, int flat) __attribute__((always_inline)) {
        char* dst = my_ring + flat * SLOT;
        if constexpr (D == 128) {
            *reinterpret_cast<u32x4_t*>(dst + 16 * lane) = u32x4_t{sg.k[0], sg.k[1], sg.k[2], sg.k[3]};
            *reinterpret_cast<u32x4_t*>(dst + CODES + 16 * lane) = u32x4_t{sg.v[0], sg.v[1], sg.v[2], sg.v[3]};
        } else {
            *reinterpret_cast<uint32_t*>(dst + 4 * lane) = sg.k[0];
            *reinterpret_cast<uint32_t*>(dst + 256 + 4 * lane) = sg.k[1];
            *reinterpret_cast<uint32_t*>(dst + CODES + 4 * lane) = sg.v[0];
            *reinterpret_cast<uint32_t*>(dst + CODES + 256 + 4 * lane) = sg.v[1];
        }
        *reinterpret_cast<uint32_t*>(dst + 2 * CODES + 4 * (lane & (8 * SB - 1))) = sg.s;   // repeats: same value
    };
    // RS: chunk slot `slot`'s registers into its LDS blocks (the caller has waited for
    // its loads); this wave's writes land before its reads of the slot
    auto land = [&](int slot) __attribute__((always_inline)) {
        on_slot<R>(slot, [&](auto tag) __attribute__((always_inline)) {
            constexpr int s0 = decltype(tag)::value;
            land_block(stg.template at<CH * s0>(), CH * s0);
            if constexpr (CH == 2) land_block(stg.template at<CH * s0 + 1>(), CH * s0 + 1);
        });
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    auto issue_block = [&](int slot, int blk) {
        const uint64_t u = (uint32_t)__builtin_amdgcn_readfirstlane(s_ids[blk]);
        const uint64_t co = u << 8, so = u << 4;
        char* dst = my_ring + slot * SLOT;
        if constexpr (D == 128) {
            dma16(kp + co + kdma, dst);
            dma16(vp + co + 16 * lane, dst + CODES);
        } else {
            dma4(kp + co + kdma, dst);
            dma4(kp + co + kdma + 4, dst + 256);
            dma4(vp + co + 4 * lane, dst + CODES);
            dma4(vp + co + 256 + 4 * lane, dst + CODES + 256);
        }
        if (sc_lane) dma4(sp + so, dst + 2 * CODES);
    };
    // chunk i of the wave: blocks wi + BW (CH i + cb); a block past the window's
    // end (the last chunk's second block) is fetched as a copy of the first and
    // masked, so every chunk issues the same number of DMAs
    int nr = 0, r0_cur = 0;   // the current window: its block count and first block
    auto blk_of = [&](int i, int cb) { return wi + BW * (CH * i + cb); };
    auto issue = [&](int slot, int i) __attribute__((always_inline)) {
        if constexpr (RS) {
            on_slot<R>(slot, [&](auto tag) __attribute__((always_inline)) {
                constexpr int s0 = decltype(tag)::value;
                load_block(stg.template at<CH * s0>(), blk_of(i, 0));
                if constexpr (CH == 2) {
                    const int blk = blk_of(i, 1);
                    load_block(stg.template at<CH * s0 + 1>(), blk < nr ? blk : blk_of(i, 0));
                }
            });
        } else {
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) {
                const int blk = blk_of(i, cb);
                issue_block(CH * slot + cb, blk < nr ? blk : blk_of(i, 0));
            }
        }
    };
    // one chunk from its slots: read, mask rows at or past lim, accumulate
    auto consume = [&](int slot, int i, int tok_r) {
        Mx4Chunk<D, CH> ck;
        bool valid[CH][4];
        int tbs[CH];
        int nfull = 0;
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            const int blk = blk_of(i, cb);
            tbs[cb] = blk < nr ? tok_r + blk * kBlockSize : lim;   // a copied block is wholly masked
            nfull += tbs[cb] + kBlockSize <= lim;
        }
        const bool full = __builtin_amdgcn_readfirstlane(nfull) == CH;   // wave-uniform
        if constexpr (RS) land(slot);
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            const uint32_t base = my_ring_a + (CH * slot + cb) * SLOT;
            if constexpr (APPEND) {
                if (new_wave && r0_cur + blk_of(i, cb) == nblk - 1) put_new(CH * slot + cb);   // full or not
            }
            lds_block<D>(base + k_rd, base + ks_rd, base + v_rd, base + vs_rd, ck.k[cb], ck.ks[cb], ck.v[cb],
                         ck.vs[cb]);
        }
        if (!full) {   // only a window's last chunk
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) {
                if (tbs[cb] + tau >= lim) {
#pragma unroll
                    for (int x = 0; x < Geo::KW; ++x) ck.k[cb][x] = 0;
                    ck.ks[cb] = 127;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    valid[cb][q] = tbs[cb] + 4 * q + j < lim;
                    if (!valid[cb][q]) {
                        ck.v[cb][q] = 0;
                        ck.vs[cb][q] = 127;
                    }
                }
            }
        } else {
#pragma unroll
            for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                for (int q = 0; q < 4; ++q) valid[cb][q] = true;
        }
        if constexpr (!LO) {
            if (full) st.template accumulate<false>(ck, valid);
            else st.template accumulate<true>(ck, valid);
        }
    };
    // LO, stage A of chunk i from its slots: read, scores, and (MASK) mark the tokens
    // at or past lim.  Branch-free, so that it shares a basic block with the previous
    // chunk's stage B.  Only a wave's last chunk of a window can hold such tokens (the
    // partition's ragged last block, or a copied block past the window's end), and
    // the steady loop never stages it, so the steady loop stages without the mask.
    auto stage_scores = [&](int slot, int i, int tok_r, typename L::PairStage& ps, auto mask) {
        constexpr bool MASK = decltype(mask)::value;
        Mx4Chunk<D, 2> ck;
        if constexpr (RS) land(slot);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const uint32_t base = my_ring_a + (2 * slot + cb) * SLOT;
            if constexpr (APPEND && MASK) {
                if (new_wave && r0_cur + blk_of(i, cb) == nblk - 1) put_new(2 * slot + cb);
            }
            lds_block<D>(base + k_rd, base + ks_rd, base + v_rd, base + vs_rd, ck.k[cb], ck.ks[cb], ck.v[cb],
                         ck.vs[cb]);
#pragma unroll
            for (int q = 0; q < 4; ++q) ps.v[cb][q] = ck.v[cb][q];
        }
        st.pair_scores(ck, ps);
        if constexpr (!MASK) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int q = 0; q < 4; ++q) ps.vs[cb][q] = ck.vs[cb][q];
            return;
        }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int blk = blk_of(i, cb);
            // token 4 q + j of the block is valid iff 4 q < rem (a copied block is wholly masked)
            const int rem = blk < nr ? lim - (tok_r + blk * kBlockSize) - j : 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool valid = 4 * q < rem;
                ps.sc[cb][q] = valid ? ps.sc[cb][q] : -__builtin_inff();
                ps.vs[cb][q] = valid ? ck.vs[cb][q] : 0u;
            }
        }
    };

    // the current window's nr blocks (ids in s_ids), the first at token tok_r
    auto stream = [&](int tok_r) {
        const int nbw = wi < nr ? (nr - wi + BW - 1) / BW : 0;   // this wave's blocks: wi + BW i
        const int nb = (nbw + CH - 1) / CH;                      // ... in chunks of CH
        if constexpr (LO) {
            // chunk i is read from slot i % R; the DMAs of chunk i + PF go into the slot
            // chunk i - 1 was read from.  Iteration i runs scores(i), then finish(i - 1).
            // ps[0] holds the staged chunk awaiting stage B between iterations; with an
            // even R the unrolled steady loop alternates the two buffers instead of copying
            typename L::PairStage ps[2];
            int i = 1;
            if (nb >= R + PF + 1) {
                // unconditional prologue (keeps the loop's waits exact): chunks 0 .. PF
#pragma unroll
                for (int v = 0; v <= PF; ++v) issue(v, v);
                wait_vm<PF * LPC>();
                stage_scores(0, 0, tok_r, ps[0], Flag<false>{});
                for (; i + R + PF <= nb; i += R) {   // i = 1 mod R: read slot (1 + v) % R, refill slot v
#pragma unroll
                    for (int v = 0; v < R; ++v) {
                        issue(v, i + v + PF);
                        wait_vm<PF * LPC>();
                        if constexpr (R % 2 == 0) {
                            stage_scores((1 + v) % R, i + v, tok_r, ps[(v + 1) & 1], Flag<false>{});
                            st.pair_finish(ps[v & 1]);
                        } else {
                            stage_scores((1 + v) % R, i + v, tok_r, ps[1], Flag<false>{});
                            st.pair_finish(ps[0]);
                            ps[0] = ps[1];
                        }
                    }
                }
            } else if (nb > 0) {
#pragma unroll
                for (int v = 0; v <= PF; ++v)
                    if (v < nb) issue(v, v);
                wait_chunks<LPC, PF>(min(nb - 1, PF));
                stage_scores(0, 0, tok_r, ps[0], Flag<true>{});
            }
            // the last chunks, waiting for chunk i + v only; i = 1 mod R here (either branch
            // above), so chunk i + v sits in slot (1 + v) % R and chunk i + v + PF goes to slot v
            for (; i < nb; i += R) {
#pragma unroll
                for (int v = 0; v < R; ++v) {
                    if (i + v < nb) {
                        if (i + v + PF < nb) issue(v, i + v + PF);
                        wait_chunks<LPC, PF>(min(nb - 1 - (i + v), PF));
                        stage_scores((1 + v) % R, i + v, tok_r, ps[1], Flag<true>{});
                        st.pair_finish(ps[0]);
                        ps[0] = ps[1];
                    }
                }
            }
            if (nb > 0) st.pair_finish(ps[0]);
            return;
        }
        int i = 0;
        if (nb >= R + PF) {
            // unconditional prologue, so the loop is entered with the same DMAs in
            // flight as it loops back with (keeps the waits exact)
#pragma unroll
            for (int v = 0; v < PF; ++v) issue(v, v);
            for (; i + R + PF <= nb; i += R) {
#pragma unroll
                for (int v = 0; v < R; ++v) {
                    issue((v + PF) % R, i + v + PF);
                    wait_vm<PF * LPC>();
                    consume(v, i + v, tok_r);
                }
            }
        } else {
#pragma unroll
            for (int v = 0; v < PF; ++v)
                if (v < nb) issue(v, v);
        }
        for (; i < nb; i += R) {   // at most two rounds left
#pragma unroll
            for (int v = 0; v < R; ++v) {
                if (i + v < nb) {
                    if (i + v + PF < nb) issue((v + PF) % R, i + v + PF);
                    wait_vm<0>();
                    consume(v, i + v, tok_r);
                }
            }
        }
    };

    if constexpr (!EVEN) {
        st.init(a, lane, b, g);
        const int32_t* table = a.block_tables + (int64_t)b * a.bt_stride;
        const int first_blk = part * (a.part_tokens / kBlockSize);
        constexpr int PRE = (kWin + T - 1) / T;
        int pre[PRE];
        {
            const int spec = min(min(a.part_tokens / kBlockSize, kWin), a.bt_stride - first_blk);
#pragma unroll
            for (int k = 0; k < PRE; ++k) {
                const int t = threadIdx.x + k * T;
                pre[k] = t < spec ? table[first_blk + t] : 0;
            }
        }
        n = APPEND ? a.positions[b] + 1 : a.context_lens[b];
        const bool bad_len = APPEND ? (n < 1 || n > a.max_context_len) : (n < 0 || n > a.max_context_len);
        if (bad_len || n == 0) {
            if (a.n_parts == 1 && part == 0)   // the rows of all HG heads
                for (int x = threadIdx.x; x < HG * a.G * D; x += T)
                    a.out[((size_t)b * a.H_q + (size_t)g0 * a.G) * D + x] = bad_len ? __builtin_nanf("") : 0.0f;
            return;
        }
        const int start = part * a.part_tokens;
        if (start >= n) return;
        lim = min(start + a.part_tokens, n);
        nblk = (lim - start + kBlockSize - 1) / kBlockSize;
        t_new = (n - 1) % kBlockSize;
        new_wave = APPEND && lim == n && wi == (nblk - 1) % BW;
        if constexpr (APPEND) {
            if (new_wave) quantize_new();
        }

        if (threadIdx.x == 0) s_bad = 0;
        for (int r0 = 0; r0 < nblk; r0 += kWin) {
            nr = min(kWin, nblk - r0);
            r0_cur = r0;
            __syncthreads();
            if (r0 == 0) {
#pragma unroll
                for (int k = 0; k < PRE; ++k) {
                    const int t = threadIdx.x + k * T;
                    if (t < nr) {
                        int id = pre[k];
                        if ((unsigned)id >= (unsigned)a.n_blocks) {
                            s_bad = 1;
                            id = 0;
                        }
                        s_ids[t] = (uint32_t)id * blk_units;
                    }
                }
            } else {
                for (int t = threadIdx.x; t < nr; t += T) {
                    int id = table[first_blk + r0 + t];
                    if ((unsigned)id >= (unsigned)a.n_blocks) {
                        s_bad = 1;
                        id = 0;
                    }
                    s_ids[t] = (uint32_t)id * blk_units;
                }
            }
            __syncthreads();
            stream(start + r0 * kBlockSize);
        }
        // an out-of-range id writes nothing
        if constexpr (APPEND) {
            if (new_wave && s_bad == 0) write_new();
        }

        // merge each head's waves through LDS (the ring is free once every wave is past here)
        const float l = sum_groups(st.l);
        __syncthreads();
        float (*s_o)[16][D + 4] = reinterpret_cast<float (*)[16][D + 4]>(s_ring);
        if (j == 0) {
            s_m[w][c] = st.m;
            s_l[w][c] = l;
        }
#pragma unroll
        for (int t = 0; t < VT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) s_o[w][c][(4 * j + q) * VT + t] = st.acc[t][q];
        __syncthreads();
        const bool bad = s_bad != 0;
        const int G = a.G;
        for (int x = threadIdx.x; x < HG * G * D; x += T) {
            const int hr = x / D;         // head slot hr / G, query row hh of that head
            const int d = x - hr * D;
            const int h0 = hr / G;
            const int hh = hr - h0 * G;
            float M = s_m[h0][hh];
#pragma unroll
            for (int k = 1; k < BW; ++k) M = fmaxf(M, s_m[h0 + HG * k][hh]);
            float Ls = 0.0f, O = 0.0f;
#pragma unroll
            for (int k = 0; k < BW; ++k) {
                const int q = h0 + HG * k;   // the head's k-th wave
                const float f = __builtin_amdgcn_exp2f(s_m[q][hh] - M);
                Ls += s_l[q][hh] * f;
                O += (LO ? s_o[q][hh][d] + s_o[q][hh + G][d] : s_o[q][hh][d]) * f;   // hi + lo columns
            }
            const size_t row = (size_t)b * a.H_q + (size_t)g0 * G + hr;
            const float val = bad ? __builtin_nanf("") : O / Ls;
            if (a.n_parts == 1) {
                a.out[row * D + d] = val;
            } else {
                a.part_o[(row * a.n_parts + part) * D + d] = val;
                if (d == 0)
                    a.part_lse[row * a.n_parts + part] = bad ? __builtin_nanf("") : M + __builtin_amdgcn_logf(Ls);
            }
        }
    } else {
        // block counts of requests tid * PER ..., prefix-summed over the workgroup
        const int tid = threadIdx.x;
        int loc[PER];
        int sum = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int bb = tid * PER + k;
            int nbk = 0;
            if (bb < a.B) {
                const int nn = APPEND ? a.positions[bb] + 1 : a.context_lens[bb];
                const bool bad = APPEND ? (nn < 1 || nn > a.max_context_len) : (nn < 0 || nn > a.max_context_len);
                nbk = bad ? 0 : (nn + kBlockSize - 1) / kBlockSize;
            }
            loc[k] = sum;
            sum += nbk;
        }
        s_scan[tid] = sum;
        __syncthreads();
#pragma unroll
        for (int off = 1; off < T; off <<= 1) {
            const int x = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += x;
            __syncthreads();
        }
        const int excl = s_scan[tid] - sum;
#pragma unroll
        for (int k = 0; k < PER; ++k) s_pre[tid * PER + k] = excl + loc[k];
        __syncthreads();

        const int total = s_pre[a.B];   // blocks per KV head over the batch (the host keeps it below 2^30)
        const int min_run = min(max(kEvenMinWaveBlocks, a.even_min_run), kEvenMaxWaveBlocks);
        const int runs = max(1, min(a.even_waves / a.H_kv, (total + min_run - 1) / min_run));
        const int tw = max(1, (total + runs - 1) / runs);   // <= kEvenMaxWaveBlocks (host sizing)
        if (blockIdx.x == 0) {
            for (int bb = tid; bb <= a.B; bb += T) a.even_meta[2 + bb] = s_pre[bb];
            if (tid == 0) {
                a.even_meta[0] = tw;
                a.even_meta[1] = runs;
            }
        }
        int x0 = S * tw;
        const int x1 = min(x0 + tw, total);
        if (S >= runs || x0 >= x1) return;   // workgroup-uniform: nothing to stream
        // the request holding block x0: the last one whose blocks start at or before it
        {
            int lo = 0, hi = a.B - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_pre[mid] <= x0) lo = mid;
                else hi = mid - 1;
            }
            b = __builtin_amdgcn_readfirstlane(lo);
        }
        // the waves walk the same pieces: the workgroup's barriers below are uniform
        while (x0 < x1) {
            const int seg0 = __builtin_amdgcn_readfirstlane(s_pre[b]);
            const int nbb = __builtin_amdgcn_readfirstlane(s_pre[b + 1]) - seg0;
            const int pend = min(x1, seg0 + nbb);
            const int blk0 = x0 - seg0, np = pend - x0;   // the piece: blocks [blk0, blk0 + np) of request b
            const bool whole = blk0 == 0 && np == nbb;
            n = APPEND ? a.positions[b] + 1 : a.context_lens[b];
            lim = n;
            nblk = np;
            nr = np;
            r0_cur = 0;
            t_new = (n - 1) % kBlockSize;
            new_wave = APPEND && blk0 + np == nbb;
            st.init(a, lane, b, g);   // q of the row's G heads; fresh softmax state
            if constexpr (APPEND) {
                if (new_wave) quantize_new();
            }
            // the piece's block ids, range-checked, staged for the workgroup
            __syncthreads();   // every wave is past the previous piece's ids
            const int32_t* table = a.block_tables + (int64_t)b * a.bt_stride + blk0;
            bool bad_lane = false;
            for (int t = tid; t < np; t += T) {
                int id = table[t];
                if ((unsigned)id >= (unsigned)a.n_blocks) {
                    bad_lane = true;
                    id = 0;
                }
                s_ids[t] = (uint32_t)id * blk_units;
            }
            const bool wave_bad = __builtin_amdgcn_ballot_w64(bad_lane) != 0;
            if (lane == 0) s_badw[w] = wave_bad ? 1 : 0;
            __syncthreads();
            bool bad = false;
#pragma unroll
            for (int q = 0; q < NW; ++q) bad = bad || s_badw[q] != 0;
            stream(blk0 * kBlockSize);
            if constexpr (APPEND) {
                if (new_wave && !bad) write_new();   // an out-of-range id writes nothing
            }

            // the piece's result for its G heads: lane (j, col) holds head col, elements
            // d = (4 j + q) VT + t; LO: column col + G holds the lo half of head col
            const float l = sum_groups(st.l);
            const int G = a.G;
            float o[VT][4];
#pragma unroll
            for (int t = 0; t < VT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v = st.acc[t][q];
                    if constexpr (LO) v += __shfl(v, lane + G, 64);
                    o[t][q] = v;
                }
            if (c < G) {
                const size_t pid = (((size_t)S + b) * a.H_kv + g) * G + c;
                float* o0 = whole ? a.out + ((size_t)b * a.H_q + (size_t)g * G + c) * D : a.part_o + pid * D;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float* op = o0 + (4 * j + q) * VT;
#pragma unroll
                    for (int t = 0; t < VT; t += 4) {
                        floatx4 val;
#pragma unroll
                        for (int e = 0; e < 4; ++e) val[e] = bad ? __builtin_nanf("") : o[t + e][q] / l;
                        *reinterpret_cast<floatx4*>(op + t) = val;
                    }
                }
                // v_log_f32 is log base 2, matching the log2-domain scores
                if (!whole && j == 0) a.part_lse[pid] = bad ? __builtin_nanf("") : st.m + __builtin_amdgcn_logf(l);
            }

            x0 = pend;
            if (x0 < x1) {   // the next request with blocks
                do {
                    ++b;
                } while (s_pre[b + 1] == s_pre[b]);
                b = __builtin_amdgcn_readfirstlane(b);
            }
        }
    }
}

template <int QDT, int D, int NW, int PF, int HG, bool EVEN>
static const void* kernel_ptr(bool lo, bool append) {
    if (lo)
        return append ? reinterpret_cast<const void*>(&decode_mxfp4_mfma_kernel<QDT, D, NW, PF, true, true, HG, EVEN>)
                      : reinterpret_cast<const void*>(&decode_mxfp4_mfma_kernel<QDT, D, NW, PF, true, false, HG, EVEN>);
    return append ? reinterpret_cast<const void*>(&decode_mxfp4_mfma_kernel<QDT, D, NW, PF, false, true, HG, EVEN>)
                  : reinterpret_cast<const void*>(&decode_mxfp4_mfma_kernel<QDT, D, NW, PF, false, false, HG, EVEN>);
}

// the fused step passes positions instead of context_lens; two blocks per output
// product (LO) when G <= 8
static hipError_t launch_fn(const void* fn, int nw, const AttnArgs& a, unsigned grid, hipStream_t stream) {
    AttnArgs args = a;
    void* params[] = {&args};
    const hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(nw * 64), params, 0, stream);
    return e != hipSuccess ? e : hipGetLastError();
}

// (waves, chunks in flight per wave, KV heads per workgroup; a chunk is two blocks when
// G <= 8, else one)
#define PKV_MX4_MFMA_VARIANTS(X) \
    X(4, 1, 1) X(4, 2, 1) X(4, 3, 1) X(2, 2, 1) X(2, 4, 1) X(4, 1, 2) X(4, 2, 2) X(4, 1, 4) X(4, 2, 4) X(8, 1, 4) \
    X(8, 2, 4) X(8, 2, 8) X(8, 3, 8) X(8, 1, 8)
// even split: (waves = KV heads per workgroup, chunks in flight per wave)
#define PKV_MX4_EVEN_VARIANTS(X) X(8, 1) X(4, 1) X(4, 2) X(2, 2)

template <int QDT, int D>
static const void* find_kernel(bool even, int nw, int pf, int hg, bool lo, bool append) {
    if (even) {
#define X(NW_, PF_) \
    if (nw == NW_ && pf == PF_) return kernel_ptr<QDT, D, NW_, PF_, NW_, true>(lo, append);
        PKV_MX4_EVEN_VARIANTS(X)
#undef X
        return nullptr;
    }
#define X(NW_, PF_, HG_) \
    if (nw == NW_ && pf == PF_ && hg == HG_) return kernel_ptr<QDT, D, NW_, PF_, HG_, false>(lo, append);
    PKV_MX4_MFMA_VARIANTS(X)
#undef X
    return nullptr;
}

static const void* find_kernel(int q_dtype, int D, bool even, int nw, int pf, int hg, bool lo, bool append) {
    switch (q_dtype * 1000 + D) {
    case DT_F16 * 1000 + 64: return find_kernel<DT_F16, 64>(even, nw, pf, hg, lo, append);
    case DT_F16 * 1000 + 128: return find_kernel<DT_F16, 128>(even, nw, pf, hg, lo, append);
    case DT_BF16 * 1000 + 64: return find_kernel<DT_BF16, 64>(even, nw, pf, hg, lo, append);
    case DT_BF16 * 1000 + 128: return find_kernel<DT_BF16, 128>(even, nw, pf, hg, lo, append);
    default: return nullptr;
    }
}

hipError_t launch_decode_mxfp4_mfma(int q_dtype, int D, int nw, int pf, int hg, const AttnArgs& a, unsigned grid,
                                    hipStream_t stream) {
    if (hg <= 0 || a.H_kv % hg) return hipErrorInvalidValue;
    const void* fn = find_kernel(q_dtype, D, false, nw, pf, hg, a.G <= 8, a.context_lens == nullptr);
    return fn ? launch_fn(fn, nw, a, grid, stream) : hipErrorInvalidValue;
}

bool mxfp4_mfma_variant_exists(int nw, int pf, int hg) {
#define X(NW_, PF_, HG_) \
    if (nw == NW_ && pf == PF_ && hg == HG_) return true;
    PKV_MX4_MFMA_VARIANTS(X)
#undef X
    return false;
}

hipError_t launch_decode_mxfp4_even(int q_dtype, int D, int nw, int pf, const AttnArgs& a, unsigned grid,
                                    hipStream_t stream) {
    if (a.H_kv % nw || !a.even_meta || a.B > kEvenMaxBatch) return hipErrorInvalidValue;
    const void* fn = find_kernel(q_dtype, D, true, nw, pf, nw, a.G <= 8, a.context_lens == nullptr);
    return fn ? launch_fn(fn, nw, a, grid, stream) : hipErrorInvalidValue;
}

bool mxfp4_even_variant_exists(int nw, int pf) {
#define X(NW_, PF_) \
    if (nw == NW_ && pf == PF_) return true;
    PKV_MX4_EVEN_VARIANTS(X)
#undef X
    return false;
}

int mxfp4_even_wgs_per_cu(int q_dtype, int D, int nw, int pf, int G, bool fused) {
    const void* fn = find_kernel(q_dtype, D, true, nw, pf, nw, G <= 8, fused);
    int n = 0;
    if (!fn || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, nw * 64, 0) != hipSuccess) return 0;
    return n;
}

}  // namespace pkv
