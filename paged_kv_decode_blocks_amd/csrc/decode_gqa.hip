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
// shared by the four lane groups holding a head with two cross-row shuffles,
// and the accumulators are rescaled lazily (only when a head's running max
// grows by more than 2^8), so the VALU rarely touches the MFMA accumulators.
//
// Three kernels:
//  * decode_gqa_kernel      V global -> registers; K global -> registers
//    (KDMA = false) or global -> LDS with global_load_lds_dwordx4 (KDMA = true,
//    the default: a register load in the MFMA layout takes half cache lines,
//    a DMA takes 1 KiB contiguous); the loads of the chunk PF ahead go out
//    before the current chunk is computed;
//  * decode_gqa_lds_kernel  K and V both go global -> LDS into a per-wave ring
//    of S block slots, then LDS -> registers in the MFMA layout;
//  * decode_gqa_fp8_kernel  the same tiles over an FP8 (E4M3) cache, codes
//    widened to q's type, row scales on scores and weights; in the fused step it
//    quantizes the new token itself (after its loop) as the append kernel would.
// K rows in LDS are stored with their 16-byte chunks XOR-swizzled by row, so the
// column-wise MFMA reads hit different banks.  All merge across the waves of the
// workgroup through LDS, and the fused APPEND variants also write the new token.
#include "pkv_fp8.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kWindowBlocksG = kGqaWindowTokens / kBlockSize;
constexpr float kRescaleSlack = 8.0f;   // log2 units: weights stay below 256

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

// V row piece of VB bytes per lane (16 for D = 128, 8 for D = 64), as 32-bit words
template <int NWORD> struct VRow { uint32_t w[NWORD]; };

template <int NWORD>
__device__ __forceinline__ VRow<NWORD> ldv(const char* p) {   // global, streaming
    VRow<NWORD> r;
    if constexpr (NWORD == 4) {
        const uint4 v = ld16(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
        const uint2 v = ld8(p);
        r.w[0] = v.x; r.w[1] = v.y;
    }
    return r;
}
template <int NWORD>
__device__ __forceinline__ VRow<NWORD> ldv_plain(const char* p) {   // global (cached) or LDS
    VRow<NWORD> r;
    if constexpr (NWORD == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        r.w[0] = v.x; r.w[1] = v.y;
    }
    return r;
}
template <int NWORD>
__device__ __forceinline__ void stv(char* p, const VRow<NWORD>& r) {
    if constexpr (NWORD == 4) st16(p, make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]));
    else st8(p, make_uint2(r.w[0], r.w[1]));
}

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes lds_base + 16 l (global_load_lds_dwordx4; lds_base wave-uniform).  The
// LDS address-space cast is only meaningful in the device pass; in the host pass
// it would silently drop the kernel's launch stub, so it is compiled there only.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
#else
    (void)src;
    (void)lds_base;
#endif
}

// KL 16-byte reads from LDS, completed before return.  Issued as inline asm: the
// compiler cannot tell a ring slot from the LDS DMAs still in flight into the
// other slots and would drain every load before a plain LDS read; the caller's
// own vmcnt wait orders the read after the DMA that filled the slot.  The outputs
// are early-clobber: a read's destination must not share a register with an
// address that a later read of the same statement still uses.
template <int KL>
__device__ __forceinline__ void lds_read16x(const char* base, const int (&off)[KL], uint4 (&r)[KL]) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t a0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)base;
    if constexpr (KL == 1) {
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r[0]) : "v"(a0 + off[0]) : "memory");
    } else if constexpr (KL == 2) {
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(r[0]), "=&v"(r[1])
                     : "v"(a0 + off[0]), "v"(a0 + off[1])
                     : "memory");
    } else {
        static_assert(KL == 4, "one, two or four reads");
        asm volatile(
            "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
            : "v"(a0 + off[0]), "v"(a0 + off[1]), "v"(a0 + off[2]), "v"(a0 + off[3])
            : "memory");
    }
#else
    (void)base;
    (void)off;
    for (int q = 0; q < KL; ++q) r[q] = make_uint4(0, 0, 0, 0);
#endif
}

// s_waitcnt vmcnt(N) leaving the other counters unconstrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// ---------------------------------------------------------------------------
// Per-lane state and arithmetic shared by both kernels.
// ---------------------------------------------------------------------------
template <int DT, int D, bool APPEND>
struct GqaLane {
    static constexpr int ES = 2;
    static constexpr int KS = D / 32;      // score MFMA steps
    static constexpr int VT = D / 16;      // output tiles = V elements per lane per row piece
    static constexpr int NWORD = VT / 2;   // 32-bit words per V row piece
    static_assert(D == 64 || D == 128, "unsupported head dim");

    int j, col, tau;
    uint4 qf[KS];
    int koff[KS];      // byte offset of this lane's K piece of step s inside a (block, head) tile
    int voff[4];       // byte offset of this lane's V piece of row-load i inside a tile
    floatx4 acc[VT];
    float m, l;
    float scale_log2;

    __device__ __forceinline__ void init(const AttnArgs& a, int lane, int b, int g) {
        j = lane >> 4;
        col = lane & 15;
        tau = 4 * (col & 3) + (col >> 2);   // token (within a block) on A-row `col`
        scale_log2 = a.scale_log2;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qf[s] = make_uint4(0, 0, 0, 0);
            if (col < a.G)
                qf[s] = ld16_cached(a.q + ((int64_t)b * a.q_row_stride + (int64_t)(g * a.G + col) * D + 32 * s + 8 * j) * ES);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) koff[s] = (tau * D + 32 * s + 8 * j) * ES;
#pragma unroll
        for (int i = 0; i < 4; ++i) voff[i] = ((4 * i + j) * D + col * VT) * ES;
#pragma unroll
        for (int t = 0; t < VT; ++t) acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        m = kNegBig;
        l = 0.0f;
    }

    // Online-softmax update with CH blocks: score tiles on MFMA, shared per-head
    // max with lazy rescaling, PV tiles on MFMA.
    template <int CH>
    __device__ __forceinline__ void accumulate(const uint4 (&kf)[CH][KS], const VRow<NWORD> (&vf)[CH][4],
                                               const bool (&valid)[CH][4]) {
        // scores: lane holds S[head col][token 4 i + j of block cb], i = 0..3
        float sc[CH][4];
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            floatx4 st = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < KS; ++s) st = Mfma<DT>::mma(kf[cb][s], qf[s], st);
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
        // The reference max m only moves when some head's running max grows by
        // more than kRescaleSlack (a rare, wave-uniform branch); with a stale m the
        // weights exp2(s - m) stay <= 2^kRescaleSlack.
        if (__builtin_amdgcn_ballot_w64(mloc > m + kRescaleSlack) != 0) {
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

    // One block that is not wholly below `lim`: masked loads straight from global
    // memory and, in the fused call, the new token from k_new/v_new (also written
    // to its pool slot).
    __device__ __forceinline__ void partial_block(const AttnArgs& a, const char* kb, const char* vb, int tb, int lim,
                                                  int pos_new, size_t new_off, bool may_write) {
        uint4 kf[1][KS];
        VRow<NWORD> vf[1][4];
        bool valid[1][4];
        const int tk = tb + tau;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            kf[0][s] = make_uint4(0, 0, 0, 0);
            if (tk < lim) {
                kf[0][s] = ld16(kb + koff[s]);
            } else if (APPEND && tk == pos_new) {
                kf[0][s] = ld16_cached(a.k_new + new_off + (32 * s + 8 * j) * ES);
                if (may_write) st16(a.k_pool_w + (kb - a.k_pool) + koff[s], kf[0][s]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tv = tb + 4 * i + j;
#pragma unroll
            for (int x = 0; x < NWORD; ++x) vf[0][i].w[x] = 0;
            valid[0][i] = false;
            if (tv < lim) {
                vf[0][i] = ldv<NWORD>(vb + voff[i]);
                valid[0][i] = true;
            } else if (APPEND && tv == pos_new) {
                vf[0][i] = ldv_plain<NWORD>(a.v_new + new_off + col * VT * ES);
                valid[0][i] = true;
                if (may_write) stv<NWORD>(a.v_pool_w + (vb - a.v_pool) + voff[i], vf[0][i]);
            }
        }
        accumulate<1>(kf, vf, valid);
    }

    // Merge the waves' states through LDS and write the normalised output, or this
    // partition's (o / l, lse) for the merge kernel.  Wave w's [16][DP] floats (DP >= D)
    // are at s_o_lo + w * 16 DP for the first (NW + 1) / 2 waves and at s_o_hi + (w -
    // (NW + 1) / 2) * 16 DP for the others, so the area may be two separate LDS objects.
    template <int NW, int DP>
    __device__ __forceinline__ void finish(const AttnArgs& a, float (*s_m)[16], float (*s_l)[16], float* s_o_lo,
                                           float* s_o_hi, int w, int b, int g, int part, bool bad) {
        static_assert(DP >= D, "merge row");
        constexpr int HALF = (NW + 1) / 2;
        auto s_o = [&](int wv) -> float (*)[DP] {
            return reinterpret_cast<float (*)[DP]>((wv < HALF ? s_o_lo : s_o_hi) + (wv % HALF) * 16 * DP);
        };
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
            for (int i = 0; i < 4; ++i) s_o(w)[col][(4 * j + i) * VT + t] = acc[t][i];
        __syncthreads();
        const int G = a.G;
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
                O += s_o(i)[hh][d] * f;
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
};

// Work unit of a workgroup: (partition, request, KV head) from the block index,
// KV head fastest.  PAIR deals neighbouring KV heads to one XCD (xcd_pair_unit),
// for the FP8 kernel whose per-(block, head) scale pieces share lines in pairs.
struct GqaUnit {
    int part, b, g, n, start, end, lim, pos_new, first_blk;
};

template <bool PAIR = false>
__device__ __forceinline__ void gqa_indices(const AttnArgs& a, GqaUnit& u) {
    const int BG = a.B * a.H_kv;
    const int x = PAIR ? xcd_pair_unit(blockIdx.x, a.n_parts * BG) : (int)blockIdx.x;
    const int pg = x / BG;
    u.part = unit_part(a, pg);
    const int bg = x - pg * BG;
    u.b = bg / a.H_kv;
    u.g = bg - u.b * a.H_kv;
    u.first_blk = u.part * (a.part_tokens / kBlockSize);
}

// The partition's first window of block ids, loaded before the length is known
// (clamped to the table row; only entries below the real block count are used).
template <int NW, int PRE, int WIN = kWindowBlocksG>
__device__ __forceinline__ void gqa_preload_ids(const AttnArgs& a, const GqaUnit& u, int (&pre)[PRE]) {
    const int32_t* table = a.block_tables + (int64_t)u.b * a.bt_stride;
    const int spec = min(min(a.part_tokens / kBlockSize, WIN), a.bt_stride - u.first_blk);
#pragma unroll
    for (int k = 0; k < PRE; ++k) {
        const int t = threadIdx.x + k * NW * 64;
        pre[k] = t < spec ? table[u.first_blk + t] : 0;
    }
}

// Length checks; returns false when the workgroup has nothing to stream (it has
// already written what it owns).
template <int D, int NW, bool APPEND>
__device__ __forceinline__ bool gqa_unit(const AttnArgs& a, GqaUnit& u) {
    u.n = APPEND ? a.positions[u.b] + 1 : a.context_lens[u.b];
    const bool bad_len = APPEND ? (u.n < 1 || u.n > a.max_context_len) : (u.n < 0 || u.n > a.max_context_len);
    if (bad_len || u.n == 0) {
        if (a.n_parts == 1 && u.part == 0)
            for (int x = threadIdx.x; x < a.G * D; x += NW * 64)
                a.out[((size_t)u.b * a.H_q + (size_t)u.g * a.G) * D + x] = bad_len ? __builtin_nanf("") : 0.0f;
        return false;
    }
    u.start = u.part * a.part_tokens;
    if (u.start >= u.n) return false;
    u.end = min(u.start + a.part_tokens, u.n);
    u.lim = min(u.end, APPEND ? u.n - 1 : u.n);
    // only the partition that ends at n holds the new token; a chunk may run past
    // its partition's last block, so every other partition must never match it
    u.pos_new = (APPEND && u.end == u.n) ? u.n - 1 : -1;
    return true;
}

// Stage one window of the partition's block ids in LDS, range-checked; the first
// window comes from the preloaded registers.
template <int NW, int PRE>
__device__ __forceinline__ void stage_ids(const AttnArgs& a, const int32_t* table, int first, int r0, int nr,
                                          const int (&pre)[PRE], int32_t* s_ids, int* s_bad) {
    if (r0 == 0) {
#pragma unroll
        for (int k = 0; k < PRE; ++k) {
            const int t = threadIdx.x + k * NW * 64;
            if (t < nr) {
                int id = pre[k];
                if ((unsigned)id >= (unsigned)a.n_blocks) {
                    *s_bad = 1;
                    id = 0;
                }
                s_ids[t] = id;
            }
        }
        return;
    }
    // the thread index is re-read here so that the staging addresses of a later window are
    // formed where they are used instead of being hoisted out of the caller's loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    for (int t = tid; t < nr; t += NW * 64) {
        int id = table[first + r0 + t];
        if ((unsigned)id >= (unsigned)a.n_blocks) {
            *s_bad = 1;
            id = 0;
        }
        s_ids[t] = id;
    }
}

// ---------------------------------------------------------------------------
// Kernel 1: V through registers; K through registers (KDMA = false) or staged
// in LDS (KDMA = true).  Each wave keeps the loads of PF chunks in flight while
// it computes one: the loads of chunk i + PF go out before chunk i is used.
// A register load in the MFMA layout takes 64 bytes of each of 16 K rows (half
// cache lines); with KDMA the K tile instead goes global -> LDS with
// global_load_lds_dwordx4 (1 KiB contiguous per instruction) into a per-wave
// ring of R = PF + 1 chunk slots, rows stored with an XOR chunk swizzle so the
// MFMA-layout reads are conflict-free.  V rows are whole lines either way.
// ---------------------------------------------------------------------------
template <int DT, int D, int NW, int CH, int PF, bool KDMA, bool APPEND>
__global__ __launch_bounds__(NW * 64) void decode_gqa_kernel(const AttnArgs a) {
    using L = GqaLane<DT, D, APPEND>;
    constexpr int KS = L::KS, NWORD = L::NWORD, ES = L::ES;
    constexpr int R = PF + 1;                  // chunk buffers
    constexpr int TILE = kBlockSize * D * ES;  // bytes of one (block, head) K tile
    constexpr int CPR = D * ES / 16;           // 16-byte chunks per K row
    constexpr int NDMA = TILE / 1024;          // DMA instructions per tile
    constexpr int SLOT = CH * TILE;            // one chunk's K tiles
    constexpr int LPC = CH * (NDMA + 4);       // vmcnt units per chunk: K DMAs, then 4 V rows
    static_assert(R <= 4, "ring depth");
    static_assert(!KDMA || PF * LPC < 64, "vmcnt range");
    // With KDMA the waves' merge rows ([16][D + 4] floats each, half of the waves in
    // each of the first two ring slots) reuse the ring once every wave is past its loop.
    constexpr int OROWS = 16 * (D + 4) * 4;                 // one wave's merge rows, bytes
    constexpr int RING = KDMA ? (NW * SLOT > (NW + 1) / 2 * OROWS ? NW * SLOT : (NW + 1) / 2 * OROWS) : 16;
    __shared__ __attribute__((aligned(16))) char s_k0[RING];
    __shared__ __attribute__((aligned(16))) char s_k1[RING];
    __shared__ __attribute__((aligned(16))) char s_k2[KDMA && R > 2 ? NW * SLOT : 16];
    __shared__ __attribute__((aligned(16))) char s_k3[KDMA && R > 3 ? NW * SLOT : 16];
    constexpr int WIN = kGqaSpanTokens / kBlockSize;   // block ids staged in LDS at a time
    __shared__ int32_t s_ids[WIN];
    __shared__ int s_bad;
    __shared__ float s_m[NW][16];
    __shared__ float s_l[NW][16];
    __shared__ float s_o[KDMA ? 4 : NW * 16 * (D + 4)];

    GqaUnit u;
    gqa_indices(a, u);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
    L st;
    st.init(a, lane, u.b, u.g);   // q loads, issued before the length is known
    constexpr int PRE = (WIN + NW * 64 - 1) / (NW * 64);
    int pre[PRE];
    gqa_preload_ids<NW, PRE, WIN>(a, u, pre);
    if (!gqa_unit<D, NW, APPEND>(a, u)) return;

    const int32_t* table = a.block_tables + (int64_t)u.b * a.bt_stride;
    const int first_blk = u.first_blk;
    const int nblk = (u.end - u.start + kBlockSize - 1) / kBlockSize;
    const size_t blk_bytes = (size_t)a.H_kv * kBlockSize * D * ES;
    const size_t head_bytes = (size_t)u.g * kBlockSize * D * ES;
    const size_t new_off = ((size_t)u.b * a.new_row_stride + (size_t)u.g * D) * ES;
    const char* kpool = a.k_pool + head_bytes;
    const char* vpool = a.v_pool + head_bytes;

    // DMA sources: lane l of instruction i fills LDS byte 16 (64 i + l) of the tile,
    // i.e. row r = (64 i + l) / CPR, position p = (64 i + l) % CPR, with global chunk
    // p ^ (r % CPR) of row r; the lane's piece of step s (chunk 4 s + j of row tau)
    // is then at position (4 s + j) ^ (tau % CPR).
    int kdma[NDMA], kread[KS];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int slot16 = i * 64 + lane;
        const int row = slot16 / CPR, p = slot16 % CPR;
        kdma[i] = row * D * ES + ((p ^ (row % CPR)) * 16);
    }
#pragma unroll
    for (int q = 0; q < KS; ++q) kread[q] = st.tau * D * ES + (((4 * q + st.j) ^ (st.tau % CPR)) * 16);
    auto slot_of = [&](int v) -> char* {
        char* base = v == 0 ? s_k0 : v == 1 ? s_k1 : v == 2 ? s_k2 : s_k3;
        return base + w * SLOT;
    };

    struct Buf {
        uint4 k[CH][KS];
        VRow<NWORD> v[CH][4];
    };
    auto load_chunk = [&](int v, Buf& bf, int cb0) {
        size_t id[CH];
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) id[cb] = (size_t)__builtin_amdgcn_readfirstlane(s_ids[cb0 + cb]);
        if constexpr (KDMA) {   // the chunk's DMAs first: a wait that leaves later loads pending covers them
#pragma unroll
            for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                for (int i = 0; i < NDMA; ++i)
                    dma16(kpool + id[cb] * blk_bytes + kdma[i], slot_of(v) + cb * TILE + i * 1024);
        } else {
#pragma unroll
            for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                for (int s = 0; s < KS; ++s) bf.k[cb][s] = ld16(kpool + id[cb] * blk_bytes + st.koff[s]);
        }
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) bf.v[cb][i] = ldv<NWORD>(vpool + id[cb] * blk_bytes + st.voff[i]);
    };
    bool all_valid[CH][4];
#pragma unroll
    for (int cb = 0; cb < CH; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) all_valid[cb][i] = true;
    // steady: exactly PF later chunks' loads were issued after this chunk's
    auto consume = [&](int v, Buf& bf, bool steady) {
        if constexpr (KDMA) {
            if (steady) wait_vmcnt<KDMA ? PF * LPC : 0>();
            else wait_vmcnt<0>();
            const char* sl = slot_of(v);
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) lds_read16x<KS>(sl + cb * TILE, kread, bf.k[cb]);
        }
        st.template accumulate<CH>(bf.k, bf.v, all_valid);
    };

    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    // the first window from the preloaded ids, before the loop: their live range ends here
    stage_ids<NW>(a, table, first_blk, 0, min(WIN, nblk), pre, s_ids, &s_bad);
    for (int r0 = 0; r0 < nblk; r0 += WIN) {
        const int nr = min(WIN, nblk - r0);
        if (r0 > 0) {
            __syncthreads();   // every wave is done with the previous window
            stage_ids<NW>(a, table, first_blk, r0, nr, pre, s_ids, &s_bad);
        }
        __syncthreads();
        const bool any_bad = s_bad != 0;
        const int nch = (nr + CH - 1) / CH;

        // Chunks wholly below `lim` need no masking.  Round-robin: wave w takes chunks w,
        // w + NW, ... of the window.  Partition per wave (a.wave_tokens > 0; the span is
        // one window): wave w takes the chunks of its own partition, blocks [wb0, wb1).
        const int tok_r = u.start + r0 * kBlockSize;
        const bool blocked = a.wave_tokens > 0;
        const int wb0 = blocked ? w * (a.wave_tokens / kBlockSize) : 0;
        const int wb1 = blocked ? min(wb0 + a.wave_tokens / kBlockSize, nr) : nr;
        const int nch_w = blocked ? max(0, (wb1 - wb0 + CH - 1) / CH) : nch;
        const int nfull_all = blocked ? max(0, min(nch_w, (u.lim - tok_r - wb0 * kBlockSize) / (CH * kBlockSize)))
                                      : max(0, min(nch, (u.lim - tok_r) / (CH * kBlockSize)));
        const int nf = blocked ? nfull_all : (w < nfull_all ? (nfull_all - w + NW - 1) / NW : 0);
        auto chunk_of = [&](int i) { return blocked ? wb0 + i * CH : (w + NW * i) * CH; };
        // chunk i lives in buffer (and ring slot) i % R
        Buf buf[R];
        int i = 0;
        if (nf >= R + PF) {
            // unconditional prologue, so the loop is entered with the same loads in
            // flight as it loops back with (keeps the compiler's waits exact)
#pragma unroll
            for (int v = 0; v < PF; ++v) load_chunk(v, buf[v], chunk_of(v));
            for (; i + R + PF <= nf; i += R) {   // steady state: every load in range
#pragma unroll
                for (int v = 0; v < R; ++v) {
                    load_chunk((v + PF) % R, buf[(v + PF) % R], chunk_of(i + v + PF));
                    consume(v, buf[v], true);
                }
            }
        } else {
#pragma unroll
            for (int v = 0; v < PF; ++v)
                if (v < nf) load_chunk(v, buf[v], chunk_of(v));
        }
        for (; i < nf; i += R) {   // at most two rounds left
#pragma unroll
            for (int v = 0; v < R; ++v) {
                if (i + v < nf) {
                    if (i + v + PF < nf) load_chunk((v + PF) % R, buf[(v + PF) % R], chunk_of(i + v + PF));
                    consume(v, buf[v], false);
                }
            }
        }
        // the partial chunk (at most one per round, or per partition), block by block
        const int k0 = blocked ? nfull_all : nfull_all + ((w - nfull_all) % NW + NW) % NW;
        for (int k = k0; k < nch_w; k += blocked ? 1 : NW) {
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) {
                const int blk = (blocked ? wb0 : 0) + k * CH + cb;
                const int id = __builtin_amdgcn_readfirstlane(blk < wb1 ? s_ids[blk] : 0);
                const char* kb = a.k_pool + (size_t)id * blk_bytes + head_bytes;
                const char* vb = a.v_pool + (size_t)id * blk_bytes + head_bytes;
                st.partial_block(a, kb, vb, tok_r + blk * kBlockSize, u.lim, u.pos_new, new_off, !any_bad);
            }
        }
    }
    if constexpr (KDMA) {
        __syncthreads();   // every wave is done with its ring slots: the merge reuses them
        st.template finish<NW, D + 4>(a, s_m, s_l, reinterpret_cast<float*>(s_k0), reinterpret_cast<float*>(s_k1),
                                      w, u.b, u.g, u.part, s_bad != 0);
    } else {
        st.template finish<NW, D + 4>(a, s_m, s_l, s_o, s_o + (NW + 1) / 2 * 16 * (D + 4), w, u.b, u.g, u.part,
                                      s_bad != 0);
    }
}

// ---------------------------------------------------------------------------
// Kernel 1e: kernel 1's per-wave pipeline (K staged in LDS by DMA, V in
// registers, one block per chunk) over an even split of the whole batch.
//
// The requests' blocks are laid end to end (request order) and cut into `runs`
// equal runs of tw blocks.  Workgroup (S, g) takes super-run S -- runs S NW ..
// S NW + NW - 1 -- for KV head g, wave w streaming run S NW + w: every wave gets
// the same number of blocks whatever the length mix, so no workgroup is left
// running alone at the end, and the H_kv workgroups of a super-run (neighbours in
// the grid, started together) read the same blocks at the same time, their tiles
// neighbours in each pool block.  A wave walks the pieces of its run (its overlap
// with each request) with a fresh softmax state each; a piece that is a whole
// request is written as the output at once.  The others -- a run's first piece,
// if it starts inside a request, and its last, if it ends inside one -- are kept
// in LDS, and at the end wave 0 merges them in token order: the pieces of one
// request within the super-run become one (the log-sum-exp regrouping of the
// softmax sum, as for split partitions), written as the output if they cover the
// request, else as the super-run's piece (o / l, log2 l + m) for the merge kernel.
//
// Piece of super-run S in request b for KV head g: id (S + b) H_kv + g (a
// super-run and a request meet in one interval, and along the end-to-end order S
// and b only grow, so S + b names each meeting once); its rows are
// part_o[(((S + b) H_kv + g) G + h) D ...] and part_lse[((S + b) H_kv + g) G + h].
//
// Every workgroup prefix-sums the requests' block counts in LDS (lengths out of
// range count as empty: the merge writes their NaN rows, and empty rows' zeros);
// workgroup 0 also stores NW tw (the super-run length), the runs used and the
// prefix for the merge.
// ---------------------------------------------------------------------------
template <int DT, int D, int NW, int PF, bool APPEND>
__global__ __launch_bounds__(NW * 64) void decode_gqa_even_kernel(const AttnArgs a) {
    using L = GqaLane<DT, D, APPEND>;
    constexpr int KS = L::KS, NWORD = L::NWORD, ES = L::ES, VT = L::VT;
    constexpr int R = PF + 1;                  // ring slots per wave
    constexpr int TILE = kBlockSize * D * ES;  // bytes of one (block, head) K tile
    constexpr int CPR = D * ES / 16;           // 16-byte chunks per K row
    constexpr int NDMA = TILE / 1024;          // DMA instructions per tile
    constexpr int LPC = NDMA + 4;              // vmcnt units per block: K DMAs, then 4 V rows
    constexpr int T = NW * 64;
    constexpr int PER = kEvenMaxBatch / T + 1; // requests per thread in the prefix sum (covers index B)
    static_assert(R <= 4 && PF * LPC < 64, "ring depth / vmcnt range");
    __shared__ __attribute__((aligned(16))) char s_ring[NW * R * TILE];
    __shared__ int32_t s_pre[PER * T];
    __shared__ int32_t s_scan[T];
    __shared__ int32_t s_wid[NW][kEvenMaxWaveBlocks];
    // a run's first piece, when it starts inside a request: its state ([VT * 4][64], lane-minor);
    // its last piece, when it ends inside one, goes to the wave's ring once the wave is done
    constexpr int STATE = VT * 4 * 64;                      // floats of one piece's state
    static_assert(R * TILE >= STATE * 4, "a piece's state fits the wave's ring");
    __shared__ float s_first[NW][STATE];
    __shared__ float s_ml[NW][2][2][16];                    // [wave][first, last][m, l][head]
    __shared__ int s_req[NW][2];                            // request of each kept piece, -1 = none
    __shared__ int s_flags[NW][2];                          // 1 starts the request, 2 ends it, 4 bad id

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (lane == 0) {
        s_req[w][0] = -1;
        s_req[w][1] = -1;
    }

    // block counts of requests tid * PER ..., prefix-summed over the workgroup
    int loc[PER];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int b = tid * PER + k;
        int nb = 0;
        if (b < a.B) {
            const int n = APPEND ? a.positions[b] + 1 : a.context_lens[b];
            const bool bad = APPEND ? (n < 1 || n > a.max_context_len) : (n < 0 || n > a.max_context_len);
            nb = bad ? 0 : (n + kBlockSize - 1) / kBlockSize;
        }
        loc[k] = sum;
        sum += nb;
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
        for (int b = tid; b <= a.B; b += T) a.even_meta[2 + b] = s_pre[b];
        if (tid == 0) {
            a.even_meta[0] = NW * tw;
            a.even_meta[1] = runs;
        }
    }
    const int S = blockIdx.x / a.H_kv, g = blockIdx.x - S * a.H_kv;
    const int run = S * NW + w;
    const int run0 = run * tw;
    int x0 = run0;
    const int x1 = min(x0 + tw, total);
    const size_t head_bytes = (size_t)g * kBlockSize * D * ES;
    char* ring = s_ring + w * R * TILE;
    L st;
    if (run < runs && x0 < x1) {   // else nothing to stream (the workgroup's closing merge follows)
        // the request holding block x0: the last one whose blocks start at or before it
        int b;
        {
            int lo = 0, hi = a.B - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_pre[mid] <= x0) lo = mid;
                else hi = mid - 1;
            }
            b = __builtin_amdgcn_readfirstlane(lo);
        }

        const size_t blk_bytes = (size_t)a.H_kv * kBlockSize * D * ES;
        const char* kpool = a.k_pool + head_bytes;
        const char* vpool = a.v_pool + head_bytes;
        int32_t* wid = s_wid[w];
        int kdma[NDMA], kread[KS];
        while (x0 < x1) {
            const int seg0 = __builtin_amdgcn_readfirstlane(s_pre[b]);
            const int nbb = __builtin_amdgcn_readfirstlane(s_pre[b + 1]) - seg0;
            const int pend = min(x1, seg0 + nbb);
            const int blk0 = x0 - seg0, np = pend - x0;   // the piece: blocks [blk0, blk0 + np) of request b
            const bool whole = blk0 == 0 && np == nbb;
            const int n = APPEND ? a.positions[b] + 1 : a.context_lens[b];
            const int lim = APPEND ? n - 1 : n;   // tokens below lim come from the pools
            const int pos_new = (APPEND && blk0 + np == nbb) ? n - 1 : -1;

            st.init(a, lane, b, g);   // q of the row's G heads; fresh softmax state
#pragma unroll
            for (int i = 0; i < NDMA; ++i) {
                const int slot16 = i * 64 + lane;
                const int row = slot16 / CPR, p = slot16 % CPR;
                kdma[i] = row * D * ES + ((p ^ (row % CPR)) * 16);
            }
#pragma unroll
            for (int q = 0; q < KS; ++q) kread[q] = st.tau * D * ES + (((4 * q + st.j) ^ (st.tau % CPR)) * 16);

            // the piece's block ids, range-checked, into the wave's LDS list
            const int32_t* table = a.block_tables + (int64_t)b * a.bt_stride + blk0;
            bool bad_lane = false;
            for (int t = lane; t < np; t += 64) {
                int id = table[t];
                if ((unsigned)id >= (unsigned)a.n_blocks) {
                    bad_lane = true;
                    id = 0;
                }
                wid[t] = id;
            }
            const bool bad = __builtin_amdgcn_ballot_w64(bad_lane) != 0;
            // the wave's LDS operations complete in order; the fence keeps the compiler from
            // moving the list's reads above its writes
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();

            const size_t new_off = ((size_t)b * a.new_row_stride + (size_t)g * D) * ES;
            struct Buf {
                uint4 k[1][KS];
                VRow<NWORD> v[1][4];
            };
            auto load_blk = [&](int slot, Buf& bf, int i) {
                const size_t id = (size_t)__builtin_amdgcn_readfirstlane(wid[i]);
#pragma unroll
                for (int q = 0; q < NDMA; ++q) dma16(kpool + id * blk_bytes + kdma[q], ring + slot * TILE + q * 1024);
#pragma unroll
                for (int r = 0; r < 4; ++r) bf.v[0][r] = ldv<NWORD>(vpool + id * blk_bytes + st.voff[r]);
            };
            bool all_valid[1][4] = {{true, true, true, true}};
            // steady: exactly PF later blocks' loads were issued after this block's
            auto consume = [&](int slot, Buf& bf, bool steady) {
                if (steady) wait_vmcnt<PF * LPC>();
                else wait_vmcnt<0>();
                lds_read16x<KS>(ring + slot * TILE, kread, bf.k[0]);
                st.template accumulate<1>(bf.k, bf.v, all_valid);
            };

            // blocks wholly below lim, pipelined; block i lives in buffer and ring slot i % R
            const int nf = max(0, min(blk0 + np, lim / kBlockSize) - blk0);
            Buf buf[R];
            int i = 0;
            if (nf >= R + PF) {
#pragma unroll
                for (int u = 0; u < PF; ++u) load_blk(u, buf[u], u);
                for (; i + R + PF <= nf; i += R) {
#pragma unroll
                    for (int u = 0; u < R; ++u) {
                        load_blk((u + PF) % R, buf[(u + PF) % R], i + u + PF);
                        consume(u, buf[u], true);
                    }
                }
            } else {
#pragma unroll
                for (int u = 0; u < PF; ++u)
                    if (u < nf) load_blk(u, buf[u], u);
            }
            for (; i < nf; i += R) {
#pragma unroll
                for (int u = 0; u < R; ++u) {
                    if (i + u < nf) {
                        if (i + u + PF < nf) load_blk((u + PF) % R, buf[(u + PF) % R], i + u + PF);
                        consume(u, buf[u], false);
                    }
                }
            }
            // the rest (the row's last block, holding the length boundary and the new token)
            for (int k = nf; k < np; ++k) {
                const int id = __builtin_amdgcn_readfirstlane(wid[k]);
                const char* kb = a.k_pool + (size_t)id * blk_bytes + head_bytes;
                const char* vb = a.v_pool + (size_t)id * blk_bytes + head_bytes;
                st.partial_block(a, kb, vb, (blk0 + k) * kBlockSize, lim, pos_new, new_off, !bad);
            }

            // the piece's result for its G heads (lane (j, col): head col, d = (4 j + i) VT + t)
            float l = st.l;
            l += __shfl_xor(l, 16, 64);
            l += __shfl_xor(l, 32, 64);
            if (whole) {
                if (st.col < a.G) {
                    float* o0 = a.out + ((size_t)b * a.H_q + (size_t)g * a.G + st.col) * D;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float* o = o0 + (4 * st.j + r) * VT;
#pragma unroll
                        for (int t = 0; t < VT; t += 4) {
                            floatx4 val;
#pragma unroll
                            for (int e = 0; e < 4; ++e) val[e] = bad ? __builtin_nanf("") : st.acc[t + e][r] / l;
                            *reinterpret_cast<floatx4*>(o + t) = val;
                        }
                    }
                }
            } else {
                // the run's first piece (starts the run), or its last (the run ends inside the
                // request; nothing streams through the ring after it)
                const int k = x0 == run0 ? 0 : 1;
                float* dst = k == 0 ? s_first[w] : reinterpret_cast<float*>(ring);
#pragma unroll
                for (int t = 0; t < VT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[(t * 4 + r) * 64 + lane] = st.acc[t][r];
                if (st.j == 0) {
                    s_ml[w][k][0][st.col] = st.m;
                    s_ml[w][k][1][st.col] = l;
                }
                if (lane == 0) {
                    s_req[w][k] = b;
                    s_flags[w][k] = (blk0 == 0 ? 1 : 0) | (blk0 + np == nbb ? 2 : 0) | (bad ? 4 : 0);
                }
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

    // Wave 0 merges the kept pieces in token order (wave by wave, first piece before
    // last); consecutive pieces of one request combine by the log-sum-exp regrouping.
    __syncthreads();
    if (w != 0) return;
    const int col = lane & 15, j = lane >> 4;
    floatx4 O[VT];
    float M = 0.0f, Lsum = 0.0f;
    int cur = -1, flags = 0;
    auto flush = [&]() {
        if (col >= a.G) return;
        const bool covers = (flags & 3) == 3;     // the pieces start and end the request
        const bool badr = (flags & 4) != 0;
        const size_t pid = ((size_t)(S + cur) * a.H_kv + g) * a.G + col;
        float* o0 = covers ? a.out + ((size_t)cur * a.H_q + (size_t)g * a.G + col) * D : a.part_o + pid * D;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float* o = o0 + (4 * j + r) * VT;
#pragma unroll
            for (int t = 0; t < VT; t += 4) {
                floatx4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = badr ? __builtin_nanf("") : O[t + e][r] / Lsum;
                *reinterpret_cast<floatx4*>(o + t) = val;
            }
        }
        // v_log_f32 is log base 2, matching the log2-domain scores
        if (!covers && j == 0) a.part_lse[pid] = badr ? __builtin_nanf("") : M + __builtin_amdgcn_logf(Lsum);
    };
    for (int ww = 0; ww < NW; ++ww) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int rq = s_req[ww][k];
            if (rq < 0) continue;
            const float* src = k == 0 ? s_first[ww] : reinterpret_cast<const float*>(s_ring + ww * R * TILE);
            const float mi = s_ml[ww][k][0][col], li = s_ml[ww][k][1][col];
            const int fi = s_flags[ww][k];
            if (rq != cur) {
                if (cur >= 0) flush();
                cur = rq;
                flags = fi;
                M = mi;
                Lsum = li;
#pragma unroll
                for (int t = 0; t < VT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) O[t][r] = src[(t * 4 + r) * 64 + lane];
            } else {
                flags = (flags & 1) | (fi & 2) | ((flags | fi) & 4);
                const float Mn = fmaxf(M, mi);
                const float c0 = __builtin_amdgcn_exp2f(M - Mn), c1 = __builtin_amdgcn_exp2f(mi - Mn);
                M = Mn;
                Lsum = Lsum * c0 + li * c1;
#pragma unroll
                for (int t = 0; t < VT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) O[t][r] = O[t][r] * c0 + src[(t * 4 + r) * 64 + lane] * c1;
            }
        }
    }
    if (cur >= 0) flush();
}

// ---------------------------------------------------------------------------
// Kernel 2: loads through LDS.  Each wave owns a ring of S slots; a slot holds
// one block's K tile (chunk-swizzled rows) followed by its V tile.
// ---------------------------------------------------------------------------
template <int D>
constexpr int gqa_tile_bytes() { return kBlockSize * D * 2; }


template <int DT, int D, int NW, int S, bool APPEND>
__global__ __launch_bounds__(NW * 64) void decode_gqa_lds_kernel(const AttnArgs a) {
    using L = GqaLane<DT, D, APPEND>;
    constexpr int KS = L::KS, NWORD = L::NWORD, ES = L::ES;
    constexpr int TILE = gqa_tile_bytes<D>();
    constexpr int SLOT = 2 * TILE;
    constexpr int CPR = D * ES / 16;          // 16-byte chunks per token row
    constexpr int NDMA = TILE / 1024;         // 1 KiB DMA instructions per tile
    constexpr int PER_BLOCK = 2 * NDMA;       // vmcnt units per block (K + V)
    static_assert(S >= 2 && S <= 4 && (S - 1) * PER_BLOCK < 64, "ring depth");

    // one LDS object per ring slot, so that the compiler's alias analysis can tell
    // a read of slot v from the DMAs still in flight into the other slots
    __shared__ __attribute__((aligned(16))) char s_ring0[NW * SLOT];
    __shared__ __attribute__((aligned(16))) char s_ring1[NW * SLOT];
    __shared__ __attribute__((aligned(16))) char s_ring2[S > 2 ? NW * SLOT : 16];
    __shared__ __attribute__((aligned(16))) char s_ring3[S > 3 ? NW * SLOT : 16];
    __shared__ int32_t s_ids[kWindowBlocksG];
    __shared__ int s_bad;
    __shared__ float s_m[NW][16];
    __shared__ float s_l[NW][16];

    GqaUnit u;
    gqa_indices(a, u);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    L st;
    st.init(a, lane, u.b, u.g);   // q loads, issued before the length is known
    constexpr int PRE = (kWindowBlocksG + NW * 64 - 1) / (NW * 64);
    int pre[PRE];
    gqa_preload_ids<NW>(a, u, pre);
    if (!gqa_unit<D, NW, APPEND>(a, u)) return;

    // DMA source offsets (lane l of instruction i fills LDS byte i*1024 + 16 l):
    // K rows are chunk-swizzled (LDS chunk p of row r holds global chunk p ^ (r % CPR)),
    // V is copied as it lies.
    int kdma[NDMA], vdma[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int slot16 = i * 64 + lane;
        const int row = slot16 / CPR;
        const int p = slot16 % CPR;
        kdma[i] = row * D * ES + ((p ^ (row % CPR)) * 16);
        vdma[i] = slot16 * 16;
    }
    // LDS read offsets of this lane's K pieces, in the MFMA layout
    int kread[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int c = 4 * s + st.j;
        kread[s] = st.tau * D * ES + ((c ^ (st.tau % CPR)) * 16);
    }

    const int32_t* table = a.block_tables + (int64_t)u.b * a.bt_stride;
    const int first_blk = u.first_blk;
    const int nblk = (u.end - u.start + kBlockSize - 1) / kBlockSize;
    const size_t blk_bytes = (size_t)a.H_kv * kBlockSize * D * ES;
    const size_t head_bytes = (size_t)u.g * kBlockSize * D * ES;
    const size_t new_off = ((size_t)u.b * a.new_row_stride + (size_t)u.g * D) * ES;
    auto slot_of = [&](int v) -> char* {
        char* base = v == 0 ? s_ring0 : v == 1 ? s_ring1 : v == 2 ? s_ring2 : s_ring3;
        return base + w * SLOT;
    };

    auto issue = [&](int v, int blk) {   // DMA round-local block `blk` into ring slot v
        const int id = __builtin_amdgcn_readfirstlane(s_ids[blk]);
        const char* kt = a.k_pool + (size_t)id * blk_bytes + head_bytes;
        const char* vt = a.v_pool + (size_t)id * blk_bytes + head_bytes;
        char* slot = slot_of(v);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) dma16(kt + kdma[i], slot + i * 1024);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) dma16(vt + vdma[i], slot + TILE + i * 1024);
    };
    bool all_valid[1][4] = {{true, true, true, true}};
    auto consume = [&](int v) {   // ring slot v -> registers -> softmax / MFMA update
        const char* slot = slot_of(v);
        uint4 kf[1][KS];
        VRow<NWORD> vf[1][4];
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[0][s] = *reinterpret_cast<const uint4*>(slot + kread[s]);
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[0][i] = ldv_plain<NWORD>(slot + TILE + st.voff[i]);
        st.template accumulate<1>(kf, vf, all_valid);
    };
    // wait until at most `after` blocks' DMAs issued after the wanted block are pending
    auto wait_blocks = [&](int after) {
        if (after <= 0) wait_vmcnt<0>();
        else if (after == 1) wait_vmcnt<PER_BLOCK>();
        else if (after == 2) wait_vmcnt<(S > 2 ? 2 : 1) * PER_BLOCK>();
        else wait_vmcnt<(S - 1) * PER_BLOCK>();
    };

    if (threadIdx.x == 0) s_bad = 0;
    for (int r0 = 0; r0 < nblk; r0 += kWindowBlocksG) {
        const int nr = min(kWindowBlocksG, nblk - r0);
        __syncthreads();
        stage_ids<NW>(a, table, first_blk, r0, nr, pre, s_ids, &s_bad);
        __syncthreads();
        const bool any_bad = s_bad != 0;

        // blocks wholly below `lim`; wave w takes blk = w, w + NW, ...
        const int tok_r = u.start + r0 * kBlockSize;
        const int nfull_all = max(0, min(nr, (u.lim - tok_r) / kBlockSize));
        const int nf = w < nfull_all ? (nfull_all - w + NW - 1) / NW : 0;
        auto blk_of = [&](int i) { return w + NW * i; };
        if (nf >= S) {
#pragma unroll
            for (int v = 0; v < S; ++v) issue(v, blk_of(v));
            int i = 0;
            for (; i + 2 * S <= nf; i += S) {
#pragma unroll
                for (int v = 0; v < S; ++v) {
                    wait_vmcnt<(S - 1) * PER_BLOCK>();
                    consume(v);
                    issue(v, blk_of(i + S + v));
                }
            }
            const int rem = nf - i - S;   // in [0, S)
#pragma unroll
            for (int v = 0; v < S; ++v) {
                wait_blocks(S - 1 - v + min(v, rem));
                consume(v);
                if (v < rem) issue(v, blk_of(i + S + v));
            }
#pragma unroll
            for (int v = 0; v < S; ++v)
                if (v < rem) {
                    wait_blocks(rem - 1 - v);
                    consume(v);
                }
        } else {
            for (int i = 0; i < nf; ++i) {
                issue(0, blk_of(i));
                wait_vmcnt<0>();
                consume(0);
            }
        }
        // remaining (partial) blocks of the round, straight from global memory
        for (int blk = nfull_all + ((w - nfull_all) % NW + NW) % NW; blk < nr; blk += NW) {
            const int id = __builtin_amdgcn_readfirstlane(s_ids[blk]);
            const char* kb = a.k_pool + (size_t)id * blk_bytes + head_bytes;
            const char* vb = a.v_pool + (size_t)id * blk_bytes + head_bytes;
            st.partial_block(a, kb, vb, tok_r + blk * kBlockSize, u.lim, u.pos_new, new_off, !any_bad);
        }
    }
    __syncthreads();   // every wave is done with its ring: the merge reuses that LDS
    // unpadded [NW][16][D] floats are exactly NW * SLOT bytes: the merge fits in slot 0's object
    static_assert(NW * 16 * D * 4 <= NW * SLOT, "merge area");
    st.template finish<NW, D>(a, s_m, s_l, reinterpret_cast<float*>(s_ring0),
                              reinterpret_cast<float*>(s_ring0) + (NW + 1) / 2 * 16 * D, w, u.b, u.g, u.part,
                              s_bad != 0);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <int DT, int D, int NW, int CH, int PF, bool KDMA>
static hipError_t launch_gqa_t(bool append, const AttnArgs& a, unsigned grid, hipStream_t stream) {
    if (append)
        hipLaunchKernelGGL((decode_gqa_kernel<DT, D, NW, CH, PF, KDMA, true>), dim3(grid), dim3(NW * 64), 0, stream,
                           a);
    else
        hipLaunchKernelGGL((decode_gqa_kernel<DT, D, NW, CH, PF, KDMA, false>), dim3(grid), dim3(NW * 64), 0, stream,
                           a);
    return hipGetLastError();
}

template <int DT, int D, int NW, int S>
static hipError_t launch_gqa_lds_t(bool append, const AttnArgs& a, unsigned grid, hipStream_t stream) {
    if (append)
        hipLaunchKernelGGL((decode_gqa_lds_kernel<DT, D, NW, S, true>), dim3(grid), dim3(NW * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_gqa_lds_kernel<DT, D, NW, S, false>), dim3(grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

// (waves, blocks per chunk, chunks in flight) of kernel 1 with K in registers (kind 0) and with
// K staged in LDS (kind 2); (waves, ring slots) of the LDS kernel (kind 1)
#define PKV_GQA_VARIANTS(X) X(4, 1, 1) X(4, 1, 2) X(2, 1, 1) X(2, 1, 2) X(4, 2, 1)
#define PKV_GQA_KDMA_VARIANTS(X) X(2, 1, 1) X(2, 1, 2) X(4, 1, 1) X(2, 2, 1) X(4, 1, 2) X(8, 1, 1)
#define PKV_GQA_LDS_VARIANTS(X) X(2, 2) X(2, 3) X(2, 4) X(4, 2) X(4, 3) X(8, 2)

template <int DT, int D>
static hipError_t launch_gqa_d(int kind, int nw, int ch, int pf, bool append, const AttnArgs& a, unsigned grid,
                               hipStream_t s) {
    if (kind == 0) {
        switch (nw * 100 + ch * 10 + pf) {
#define PKV_CASE(NW_, CH_, PF_) \
    case NW_ * 100 + CH_ * 10 + PF_: return launch_gqa_t<DT, D, NW_, CH_, PF_, false>(append, a, grid, s);
            PKV_GQA_VARIANTS(PKV_CASE)
#undef PKV_CASE
        default: return hipErrorInvalidValue;
        }
    }
    if (kind == 2) {
        switch (nw * 100 + ch * 10 + pf) {
#define PKV_CASE(NW_, CH_, PF_) \
    case NW_ * 100 + CH_ * 10 + PF_: return launch_gqa_t<DT, D, NW_, CH_, PF_, true>(append, a, grid, s);
            PKV_GQA_KDMA_VARIANTS(PKV_CASE)
#undef PKV_CASE
        default: return hipErrorInvalidValue;
        }
    }
    switch (nw * 10 + pf) {
#define PKV_CASE(NW_, S_) \
    case NW_ * 10 + S_: return launch_gqa_lds_t<DT, D, NW_, S_>(append, a, grid, s);
        PKV_GQA_LDS_VARIANTS(PKV_CASE)
#undef PKV_CASE
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_gqa(int dtype, int D, int kind, int nw, int ch, int pf, bool append, const AttnArgs& a,
                             unsigned grid, hipStream_t stream) {
    switch (dtype * 1000 + D) {
    case DT_F16 * 1000 + 64: return launch_gqa_d<DT_F16, 64>(kind, nw, ch, pf, append, a, grid, stream);
    case DT_F16 * 1000 + 128: return launch_gqa_d<DT_F16, 128>(kind, nw, ch, pf, append, a, grid, stream);
    case DT_BF16 * 1000 + 64: return launch_gqa_d<DT_BF16, 64>(kind, nw, ch, pf, append, a, grid, stream);
    case DT_BF16 * 1000 + 128: return launch_gqa_d<DT_BF16, 128>(kind, nw, ch, pf, append, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

// (waves, blocks ahead) of the even-split kernel
#define PKV_GQA_EVEN_VARIANTS(X) X(4, 1) X(2, 1) X(8, 1)

template <int DT, int D, int NW, int PF>
static const void* gqa_even_fn(bool append) {
    return append ? reinterpret_cast<const void*>(&decode_gqa_even_kernel<DT, D, NW, PF, true>)
                  : reinterpret_cast<const void*>(&decode_gqa_even_kernel<DT, D, NW, PF, false>);
}

template <int DT, int D>
static const void* gqa_even_fn_d(int nw, int pf, bool append) {
    switch (nw * 10 + pf) {
#define PKV_CASE(NW_, PF_) \
    case NW_ * 10 + PF_: return gqa_even_fn<DT, D, NW_, PF_>(append);
        PKV_GQA_EVEN_VARIANTS(PKV_CASE)
#undef PKV_CASE
    default: return nullptr;
    }
}

static const void* gqa_even_kernel_fn(int dtype, int D, int nw, int pf, bool append) {
    switch (dtype * 1000 + D) {
    case DT_F16 * 1000 + 64: return gqa_even_fn_d<DT_F16, 64>(nw, pf, append);
    case DT_F16 * 1000 + 128: return gqa_even_fn_d<DT_F16, 128>(nw, pf, append);
    case DT_BF16 * 1000 + 64: return gqa_even_fn_d<DT_BF16, 64>(nw, pf, append);
    case DT_BF16 * 1000 + 128: return gqa_even_fn_d<DT_BF16, 128>(nw, pf, append);
    default: return nullptr;
    }
}

hipError_t launch_decode_gqa_even(int dtype, int D, int nw, int pf, bool append, const AttnArgs& a, unsigned grid,
                                  hipStream_t stream) {
    const void* fn = gqa_even_kernel_fn(dtype, D, nw, pf, append);
    if (!fn || !a.even_meta || a.even_waves <= 0 || a.B > kEvenMaxBatch) return hipErrorInvalidValue;
    void* args[] = {const_cast<AttnArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(grid), dim3(nw * 64), args, 0, stream);
}

bool gqa_even_variant_exists(int nw, int pf) {
    switch (nw * 10 + pf) {
#define PKV_CASE(NW_, PF_) case NW_ * 10 + PF_:
        PKV_GQA_EVEN_VARIANTS(PKV_CASE)
#undef PKV_CASE
        return true;
    default: return false;
    }
}

int gqa_even_wgs_per_cu(int dtype, int D, int nw, int pf, bool append) {
    const void* fn = gqa_even_kernel_fn(dtype, D, nw, pf, append);
    if (!fn) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, nw * 64, 0) != hipSuccess) return 0;
    return n;
}

bool gqa_variant_exists(int kind, int nw, int ch, int pf) {
    if (kind == 0) {
        switch (nw * 100 + ch * 10 + pf) {
#define PKV_CASE(NW_, CH_, PF_) case NW_ * 100 + CH_ * 10 + PF_:
            PKV_GQA_VARIANTS(PKV_CASE)
#undef PKV_CASE
            return true;
        default: return false;
        }
    }
    if (kind == 2) {
        switch (nw * 100 + ch * 10 + pf) {
#define PKV_CASE(NW_, CH_, PF_) case NW_ * 100 + CH_ * 10 + PF_:
            PKV_GQA_KDMA_VARIANTS(PKV_CASE)
#undef PKV_CASE
            return true;
        default: return false;
        }
    }
    if (kind != 1) return false;
    if (ch != 1) return false;
    switch (nw * 10 + pf) {
#define PKV_CASE(NW_, S_) case NW_ * 10 + S_:
        PKV_GQA_LDS_VARIANTS(PKV_CASE)
#undef PKV_CASE
        return true;
    default: return false;
    }
}

// ---------------------------------------------------------------------------
// Kernel 3: grouped heads over an FP8 (OCP E4M3) K/V cache.
//
// The same MFMA tiles in q's type (f16 or bf16), with the codes widened by
// v_cvt_scalef32_pk_{bf16,f16}_fp8 at scale 1 (every E4M3 value is exact in
// both types), so the products see code values.  The row scales (one power of
// two per token row and KV head) enter where the tokens are separate: the
// score of token t is multiplied by k_scale[t] before the softmax, and its
// weight by v_scale[t] before the P V product -- exact multiplications.
//
// Layout differences from the 16-bit kernels, all to cut load instructions per
// block (a code block is half as many bytes, so the per-block instruction and
// latency cost, not the bytes, sets the rate):
//  * tile row r is token r of the block, so the lane holding head `col` in
//    lane group j gets the scores of tokens 4 j .. 4 j + 3; its V rows and its
//    eight scales are those four tokens (one 16-byte load per scale pool);
//  * the head dimension is renumbered inside each 64-wide slice: MFMA step
//    2 u + e, k slot kk of lane group j is d = 64 u + 16 j + 8 e + kk, applied to
//    q and K alike (the dot product does not depend on the order of d), so one
//    16-byte K load feeds two steps;
//  * loads of the chunk PF ahead are issued before the current chunk's
//    arithmetic, and a lane's offsets are 32-bit from a per-block scalar base.
//
// Lengths are context_lens[b], or positions[b] + 1 when context_lens is NULL:
// the fused FP8 step appends with the quantizing append kernel first and then
// runs this kernel over the updated pools.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ uint32_t fp8x2_widen(uint32_t w, bool hi) {
    if constexpr (DT == DT_BF16) {
        return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true))
                  : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false));
    } else {
        return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true))
                  : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false));
    }
}

__device__ __forceinline__ uint32_t ld4(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// One block's loads for one lane.
template <int D>
struct F8Codes {
    static constexpr int KL = D / 64;   // 16-byte K loads (two MFMA steps each)
    static constexpr int VW = D / 64;   // 32-bit words of V codes per row piece
    uint4 k[KL];
    uint32_t v[4][VW];
    float4 ks, vs;                      // scales of tokens 4 j .. 4 j + 3
};

template <int DT, int D>
struct GqaLaneF8 : GqaLane<DT, D, false> {
    using Base = GqaLane<DT, D, false>;
    using Codes = F8Codes<D>;
    static constexpr int KS = Base::KS, VT = Base::VT, NWORD = Base::NWORD, ES = Base::ES;
    static constexpr int KL = Codes::KL, VW = Codes::VW;
    uint32_t kofs;   // byte offset of this lane's first K piece in a (block, head) tile
    uint32_t vofs;   // byte offset of this lane's V piece of token 4 j
    uint32_t sofs;   // byte offset of this lane's four scales in a (block, head) scale row

    __device__ __forceinline__ void init8(const AttnArgs& a, int lane, int b, int g) {
        this->j = lane >> 4;
        this->col = lane & 15;
        this->tau = this->col;
        this->scale_log2 = a.scale_log2;
        const int j = this->j, col = this->col;
#pragma unroll
        for (int u = 0; u < KL; ++u)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                this->qf[2 * u + e] = make_uint4(0, 0, 0, 0);
                if (col < a.G)
                    this->qf[2 * u + e] = ld16_cached(
                        a.q + ((int64_t)b * a.q_row_stride + (int64_t)(g * a.G + col) * D + 64 * u + 16 * j + 8 * e) * ES);
            }
        kofs = (uint32_t)(col * D + 16 * j);
        vofs = (uint32_t)(4 * j * D + col * VT);
        sofs = (uint32_t)(16 * j);
#pragma unroll
        for (int t = 0; t < VT; ++t) this->acc[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        this->m = kNegBig;
        this->l = 0.0f;
    }

    __device__ __forceinline__ void load_v(const uint8_t* vb, int i, uint32_t (&vc)[VW]) const {
        if constexpr (VW == 2) {
            const uint2 v = ld8(vb + vofs + i * D);
            vc[0] = v.x;
            vc[1] = v.y;
        } else {
            vc[0] = ld4(vb + vofs + i * D);
        }
    }

    // kb, vb: the (block, head) code tiles; ksb, vsb: its scale rows
    __device__ __forceinline__ void load_k(const uint8_t* kb, Codes& c) const {
#pragma unroll
        for (int u = 0; u < KL; ++u) c.k[u] = ld16(kb + kofs + 64 * u);
    }
    __device__ __forceinline__ void load_vs(const uint8_t* vb, const uint8_t* ksb, const uint8_t* vsb,
                                            Codes& c) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) load_v(vb, i, c.v[i]);
        c.ks = *reinterpret_cast<const float4*>(ksb + sofs);
        c.vs = *reinterpret_cast<const float4*>(vsb + sofs);
    }

    // Online-softmax update with CH blocks of codes.
    template <int CH>
    __device__ __forceinline__ void accumulate8(const uint4 (&kc)[CH][KL], const Codes (&c)[CH],
                                                const bool (&valid)[CH][4]) {
        float sc[CH][4];
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            floatx4 st = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int u = 0; u < KL; ++u) {
                const uint4 kw = kc[cb][u];
                const uint4 k0 = make_uint4(fp8x2_widen<DT>(kw.x, false), fp8x2_widen<DT>(kw.x, true),
                                            fp8x2_widen<DT>(kw.y, false), fp8x2_widen<DT>(kw.y, true));
                const uint4 k1 = make_uint4(fp8x2_widen<DT>(kw.z, false), fp8x2_widen<DT>(kw.z, true),
                                            fp8x2_widen<DT>(kw.w, false), fp8x2_widen<DT>(kw.w, true));
                st = Mfma<DT>::mma(k0, this->qf[2 * u], st);
                st = Mfma<DT>::mma(k1, this->qf[2 * u + 1], st);
            }
            const float ks[4] = {c[cb].ks.x, c[cb].ks.y, c[cb].ks.z, c[cb].ks.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[cb][i] = mul_rn(st[i] * ks[i], this->scale_log2);
        }
        float mloc = kNegBig;
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mloc = valid[cb][i] ? fmaxf(mloc, sc[cb][i]) : mloc;
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        if (__builtin_amdgcn_ballot_w64(mloc > this->m + kRescaleSlack) != 0) {   // lazy rescale, as in GqaLane
            const float m_new = fmaxf(this->m, mloc);
            const float alpha = __builtin_amdgcn_exp2f(this->m - m_new);
            this->m = m_new;
            this->l *= alpha;
#pragma unroll
            for (int t = 0; t < VT; ++t) this->acc[t] *= alpha;
        }
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            const float vs[4] = {c[cb].vs.x, c[cb].vs.y, c[cb].vs.z, c[cb].vs.w};
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = valid[cb][i] ? __builtin_amdgcn_exp2f(sc[cb][i] - this->m) : 0.0f;
                this->l += e;
                p[i] = e * vs[i];
            }
            uint4 pk;
            Mfma<DT>::split(p[0], p[1], pk.x, pk.z);
            Mfma<DT>::split(p[2], p[3], pk.y, pk.w);
            // widen the four V rows: word x of row i holds elements 2x, 2x+1 of the lane's piece
            uint32_t vw[4][NWORD];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int x = 0; x < NWORD; ++x) vw[i][x] = fp8x2_widen<DT>(c[cb].v[i][x >> 1], (x & 1) != 0);
#pragma unroll
            for (int t = 0; t < VT; ++t) {
                const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
                const int x = t >> 1;
                const uint32_t v01 = __builtin_amdgcn_perm(vw[1][x], vw[0][x], sel);
                const uint32_t v23 = __builtin_amdgcn_perm(vw[3][x], vw[2][x], sel);
                this->acc[t] = Mfma<DT>::mma(make_uint4(v01, v23, v01, v23), pk, this->acc[t]);
            }
        }
    }

    // One block not wholly below `lim`: masked loads; the scales of tokens at or
    // past `lim` are taken as zero (their slots may hold anything).
    __device__ __forceinline__ void partial_block8(const uint8_t* kb, const uint8_t* vb, const uint8_t* ksb,
                                                   const uint8_t* vsb, int tb, int lim) {
        Codes c[1];
        bool valid[1][4];
        const int tk = tb + this->col;
#pragma unroll
        for (int u = 0; u < KL; ++u) c[0].k[u] = tk < lim ? ld16(kb + kofs + 64 * u) : make_uint4(0, 0, 0, 0);
        const int t0 = tb + 4 * this->j;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            valid[0][i] = t0 + i < lim;
#pragma unroll
            for (int x = 0; x < VW; ++x) c[0].v[i][x] = 0;
            if (valid[0][i]) load_v(vb, i, c[0].v[i]);
        }
        float4 ks = make_float4(0.0f, 0.0f, 0.0f, 0.0f), vs = ks;
        if (t0 < lim) {
            ks = *reinterpret_cast<const float4*>(ksb + sofs);
            vs = *reinterpret_cast<const float4*>(vsb + sofs);
        }
        c[0].ks = make_float4(valid[0][0] ? ks.x : 0.0f, valid[0][1] ? ks.y : 0.0f, valid[0][2] ? ks.z : 0.0f,
                              valid[0][3] ? ks.w : 0.0f);
        c[0].vs = make_float4(valid[0][0] ? vs.x : 0.0f, valid[0][1] ? vs.y : 0.0f, valid[0][2] ? vs.z : 0.0f,
                              valid[0][3] ? vs.w : 0.0f);
        uint4 kc[1][KL];
#pragma unroll
        for (int u = 0; u < KL; ++u) kc[0][u] = c[0].k[u];
        accumulate8<1>(kc, c, valid);
    }
};

// WPE: waves per SIMD the register allocation must leave room for (2 = as many
// registers as the code wants; 3 trades a few spills for occupancy).  PF: chunks
// whose loads are in flight while a chunk is being computed.  KDMA: K tiles go
// global -> LDS with global_load_lds_dwordx4 (1 KiB contiguous per instruction,
// whole cache lines; a register load of the MFMA layout takes 64 bytes of each
// of 16 rows) into a per-wave ring of R chunk slots, rows stored with an XOR
// chunk swizzle so the MFMA-layout reads (16 rows, one chunk each) are
// conflict-free; V and the scales stay register loads (already whole lines).
// KDMA with register staging: each K piece is loaded into a register from the address
// its DMA would read and written by the wave into the LDS place that DMA would fill,
// just before the slot's MFMA-layout reads (all V, scale and K loads then go through
// registers, which a wave streams faster than global_load_lds pieces).
constexpr bool kFp8RegisterStaging = true;

template <int DT, int D, int NW, int CH, int PF, int WPE, bool KDMA>
__global__ __launch_bounds__(NW * 64, WPE) void decode_gqa_fp8_kernel(const AttnArgs a) {
    using L = GqaLaneF8<DT, D>;
    using Codes = typename L::Codes;
    constexpr int KL = L::KL;
    constexpr int R = PF + 1;                 // chunk buffers
    constexpr int TILE = kBlockSize * D;      // bytes of one (block, head) code tile
    constexpr int CPR = D / 16;               // 16-byte chunks per code row
    constexpr int NDMA = TILE / 1024;         // DMA instructions per tile
    constexpr int SLOT = CH * TILE;           // one chunk's K tiles
    constexpr int LPC = CH * (NDMA + 6);      // vmcnt units per chunk: K DMAs, 4 V rows, 2 scale loads
    constexpr bool RS = KDMA && kFp8RegisterStaging && PF == 1;   // deeper rings do not fit the registers
    static_assert(NDMA == KL, "a K piece per register of the chunk's codes");
    static_assert(R <= 4, "ring depth");
    static_assert(!KDMA || PF * LPC < 64, "vmcnt range");
    // one LDS object per ring slot, so that alias analysis can tell a read of one
    // slot from the DMAs still in flight into the others; with KDMA the closing merge
    // of the waves reuses the first two, sized for half of it each
    constexpr int MERGE_HALF = (NW + 1) / 2 * 16 * (D + 4) * 4;
    constexpr int S01 = !KDMA ? 16 : NW * SLOT > MERGE_HALF ? NW * SLOT : MERGE_HALF;
    __shared__ __attribute__((aligned(16))) char s_k0[S01];
    __shared__ __attribute__((aligned(16))) char s_k1[S01];
    __shared__ __attribute__((aligned(16))) char s_k2[KDMA && R > 2 ? NW * SLOT : 16];
    __shared__ __attribute__((aligned(16))) char s_k3[KDMA && R > 3 ? NW * SLOT : 16];
    __shared__ int32_t s_ids[kWindowBlocksG];
    __shared__ int s_bad;
    __shared__ float s_m[NW][16];
    __shared__ float s_l[NW][16];
    __shared__ float s_o[KDMA ? 4 : NW * 16 * (D + 4)];

    GqaUnit u;
    gqa_indices<true>(a, u);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    L st;
    st.init8(a, lane, u.b, u.g);
    constexpr int PRE = (kWindowBlocksG + NW * 64 - 1) / (NW * 64);
    int pre[PRE];
    gqa_preload_ids<NW>(a, u, pre);
    // lengths: context_lens, or positions + 1 in the fused step
    {
        const bool from_pos = a.context_lens == nullptr;
        u.n = from_pos ? a.positions[u.b] + 1 : a.context_lens[u.b];
        const bool bad_len = from_pos ? (u.n < 1 || u.n > a.max_context_len) : (u.n < 0 || u.n > a.max_context_len);
        if (bad_len || u.n == 0) {
            if (a.n_parts == 1 && u.part == 0)
                for (int x = threadIdx.x; x < a.G * D; x += NW * 64)
                    a.out[((size_t)u.b * a.H_q + (size_t)u.g * a.G) * D + x] = bad_len ? __builtin_nanf("") : 0.0f;
            return;
        }
        u.start = u.part * a.part_tokens;
        if (u.start >= u.n) return;
        u.end = min(u.start + a.part_tokens, u.n);
        // the fused step: the pools hold the rows below n - 1; the new token is
        // quantized here, by wave 0 of the partition that ends at n (below)
        u.lim = from_pos ? min(u.end, u.n - 1) : u.end;
    }
    const bool holds_new = a.context_lens == nullptr && u.end == u.n;
    const int t_new = (u.n - 1) % kBlockSize;
    constexpr int PER = D / 64;   // elements of a new row per lane
    float xnew[2][PER];           // wave 0 of that partition: the new K and V rows, loaded now
#pragma unroll
    for (int which = 0; which < 2; ++which)
#pragma unroll
        for (int i = 0; i < PER; ++i) xnew[which][i] = 0.0f;
    if (holds_new && w == 0) {
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const char* src = (which ? a.v_new : a.k_new) + ((size_t)u.b * a.new_row_stride + (size_t)u.g * D + lane * PER) * L::ES;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const uint16_t v16 = reinterpret_cast<const uint16_t*>(src)[i];
                xnew[which][i] = DT == DT_F16 ? (float)__builtin_bit_cast(_Float16, v16) : __uint_as_float((uint32_t)v16 << 16);
            }
        }
    }

    const int32_t* table = a.block_tables + (int64_t)u.b * a.bt_stride;
    const int nblk = (u.end - u.start + kBlockSize - 1) / kBlockSize;
    const size_t blk_codes = (size_t)a.H_kv * kBlockSize * D;
    const size_t head_codes = (size_t)u.g * kBlockSize * D;
    const size_t blk_sbytes = (size_t)a.H_kv * kBlockSize * 4;
    const size_t head_sbytes = (size_t)u.g * kBlockSize * 4;
    const uint8_t* kpool = reinterpret_cast<const uint8_t*>(a.k_pool) + head_codes;
    const uint8_t* vpool = reinterpret_cast<const uint8_t*>(a.v_pool) + head_codes;
    const uint8_t* kspool = reinterpret_cast<const uint8_t*>(a.k_scale) + head_sbytes;
    const uint8_t* vspool = reinterpret_cast<const uint8_t*>(a.v_scale) + head_sbytes;

    // DMA sources: lane l of instruction i fills LDS byte 16 (64 i + l) of the tile,
    // i.e. row r = (64 i + l) / CPR, position p = (64 i + l) % CPR, with global chunk
    // p ^ (r % CPR) of row r; the lane's MFMA piece (chunk 4 u + j of row col) is
    // then at position (4 u + j) ^ (col % CPR).
    int kdma[NDMA], kread[KL];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int slot16 = i * 64 + lane;
        const int row = slot16 / CPR, p = slot16 % CPR;
        kdma[i] = row * D + ((p ^ (row % CPR)) * 16);
    }
#pragma unroll
    for (int q = 0; q < KL; ++q) kread[q] = st.col * D + (((4 * q + st.j) ^ (st.col % CPR)) * 16);
    auto slot_of = [&](int v) -> char* {
        char* base = v == 0 ? s_k0 : v == 1 ? s_k1 : v == 2 ? s_k2 : s_k3;
        return base + w * SLOT;
    };

    auto load_chunk = [&](int v, Codes (&c)[CH], int cb0) {
        size_t id[CH];
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) id[cb] = (size_t)__builtin_amdgcn_readfirstlane(s_ids[cb0 + cb]);
        if constexpr (RS) {   // K pieces into registers, written into the slot when the chunk is used
#pragma unroll
            for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                for (int i = 0; i < NDMA; ++i) c[cb].k[i] = ld16(kpool + id[cb] * blk_codes + kdma[i]);
        } else if constexpr (KDMA) {   // the chunk's DMAs first: a wait that leaves later loads pending covers them
#pragma unroll
            for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                for (int i = 0; i < NDMA; ++i)
                    dma16(kpool + id[cb] * blk_codes + kdma[i], slot_of(v) + cb * TILE + i * 1024);
        } else {
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) st.load_k(kpool + id[cb] * blk_codes, c[cb]);
        }
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
            st.load_vs(vpool + id[cb] * blk_codes, kspool + id[cb] * blk_sbytes, vspool + id[cb] * blk_sbytes, c[cb]);
    };
    // steady: exactly PF later chunks' loads were issued after this chunk's
    auto consume = [&](int v, const Codes (&c)[CH], bool steady) {
        uint4 kc[CH][KL];
        if constexpr (KDMA) {
            if (steady) wait_vmcnt<KDMA ? PF * LPC : 0>();
            else wait_vmcnt<0>();
            const char* sl = slot_of(v);
            if constexpr (RS) {   // lane l's piece i goes where DMA lane l of instruction i would put it
                char* slw = slot_of(v);
#pragma unroll
                for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                    for (int i = 0; i < NDMA; ++i)
                        *reinterpret_cast<uint4*>(slw + cb * TILE + i * 1024 + 16 * lane) = c[cb].k[i];
                // this wave's LDS writes land before its reads of the slot (in order per wave)
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) lds_read16x<KL>(sl + cb * TILE, kread, kc[cb]);
        } else {
#pragma unroll
            for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                for (int q = 0; q < KL; ++q) kc[cb][q] = c[cb].k[q];
        }
        bool all_valid[CH][4];
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) all_valid[cb][i] = true;
        st.template accumulate8<CH>(kc, c, all_valid);
    };

    if (threadIdx.x == 0) s_bad = 0;
    for (int r0 = 0; r0 < nblk; r0 += kWindowBlocksG) {
        const int nr = min(kWindowBlocksG, nblk - r0);
        __syncthreads();
        stage_ids<NW>(a, table, u.first_blk, r0, nr, pre, s_ids, &s_bad);
        __syncthreads();
        const int nch = (nr + CH - 1) / CH;
        const int tok_r = u.start + r0 * kBlockSize;
        const int nfull_all = max(0, min(nch, (u.lim - tok_r) / (CH * kBlockSize)));
        const int nf = w < nfull_all ? (nfull_all - w + NW - 1) / NW : 0;   // this wave's full chunks
        auto chunk_of = [&](int i) { return (w + NW * i) * CH; };
        // chunk i lives in buffer (and ring slot) i % R; the loads of chunk i + PF
        // go out before chunk i is used
        Codes buf[R][CH];
        int i = 0;
        if (nf >= R + PF) {
            // unconditional prologue, so the loop is entered with the same loads in
            // flight as it loops back with (keeps the compiler's waits exact)
#pragma unroll
            for (int v = 0; v < PF; ++v) load_chunk(v, buf[v], chunk_of(v));
            for (; i + R + PF <= nf; i += R) {   // steady state: every load in range
#pragma unroll
                for (int v = 0; v < R; ++v) {
                    load_chunk((v + PF) % R, buf[(v + PF) % R], chunk_of(i + v + PF));
                    consume(v, buf[v], true);
                }
            }
        } else {
#pragma unroll
            for (int v = 0; v < PF; ++v)
                if (v < nf) load_chunk(v, buf[v], chunk_of(v));
        }
        for (; i < nf; i += R) {   // at most two rounds left
#pragma unroll
            for (int v = 0; v < R; ++v) {
                if (i + v < nf) {
                    if (i + v + PF < nf) load_chunk((v + PF) % R, buf[(v + PF) % R], chunk_of(i + v + PF));
                    consume(v, buf[v], false);
                }
            }
        }
        for (int k = nfull_all + ((w - nfull_all) % NW + NW) % NW; k < nch; k += NW) {
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) {
                const int blk = k * CH + cb;
                const size_t id = (size_t)__builtin_amdgcn_readfirstlane(blk < nr ? s_ids[blk] : 0);
                st.partial_block8(kpool + id * blk_codes, vpool + id * blk_codes, kspool + id * blk_sbytes,
                                  vspool + id * blk_sbytes, tok_r + blk * kBlockSize, u.lim);
            }
        }
    }
    if (holds_new && w == 0) {
        // Quantize the new K and V rows as the append kernel does (lane l holds
        // elements PER l .. PER l + PER - 1; the row max from a wave reduction), write
        // them to the pools (this workgroup is the only one holding position n - 1 of
        // its KV head; an out-of-range block id writes nothing), and add the token
        // as one more masked row, its codes reaching the MFMA layout through LDS.
        __shared__ __attribute__((aligned(16))) uint8_t s_new[2][D];
        __shared__ float s_nsc[2];
        const int blk = (int)s_ids[(nblk - 1) % kWindowBlocksG];   // the last window is still staged
        const size_t row = ((size_t)blk * a.H_kv + u.g) * kBlockSize + t_new;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < PER; ++i) amax = fmaxf(amax, fabsf(xnew[which][i]));
            amax = group_max<64>(amax);
            const int E = fp8_row_exponent(amax);
            const float inv = pow2f(-E);
            uint8_t* pool = reinterpret_cast<uint8_t*>(which ? a.v_pool_w : a.k_pool_w);
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const uint8_t code = (uint8_t)fp8_encode(xnew[which][i] * inv);
                s_new[which][lane * PER + i] = code;
                if (s_bad == 0) pool[row * D + lane * PER + i] = code;
            }
            if (lane == 0) {
                s_nsc[which] = pow2f(E);
                if (s_bad == 0) (which ? a.v_scale_w : a.k_scale_w)[row] = pow2f(E);
            }
        }
        // this wave's LDS writes land before its reads (in order per wave)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        typename L::Codes c[1];
        bool valid[1][4];
        const int j = st.j, col = st.col;
#pragma unroll
        for (int q = 0; q < KL; ++q)
            c[0].k[q] = col == t_new ? *reinterpret_cast<const uint4*>(&s_new[0][64 * q + 16 * j]) : make_uint4(0, 0, 0, 0);
        float ks[4], vs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            valid[0][i] = 4 * j + i == t_new;
#pragma unroll
            for (int x = 0; x < L::VW; ++x)
                c[0].v[i][x] = valid[0][i] ? *reinterpret_cast<const uint32_t*>(&s_new[1][col * L::VT + 4 * x]) : 0u;
            ks[i] = valid[0][i] ? s_nsc[0] : 0.0f;
            vs[i] = valid[0][i] ? s_nsc[1] : 0.0f;
        }
        c[0].ks = make_float4(ks[0], ks[1], ks[2], ks[3]);
        c[0].vs = make_float4(vs[0], vs[1], vs[2], vs[3]);
        uint4 kc[1][KL];
#pragma unroll
        for (int q = 0; q < KL; ++q) kc[0][q] = c[0].k[q];
        st.template accumulate8<1>(kc, c, valid);
    }
    if constexpr (KDMA) {
        __syncthreads();   // every wave is done with its ring slots: the merge reuses them
        st.template finish<NW, D + 4>(a, s_m, s_l, reinterpret_cast<float*>(s_k0), reinterpret_cast<float*>(s_k1),
                                      w, u.b, u.g, u.part, s_bad != 0);
    } else {
        st.template finish<NW, D + 4>(a, s_m, s_l, s_o, s_o + (NW + 1) / 2 * 16 * (D + 4), w, u.b, u.g, u.part,
                                      s_bad != 0);
    }
}

#define PKV_GQA_FP8_VARIANTS(X)                                                                       \
    X(2, 1, 1, 2, 0) X(2, 1, 2, 2, 0) X(4, 1, 1, 2, 0) X(2, 2, 1, 2, 0) X(4, 2, 1, 2, 0) X(2, 1, 1, 3, 0) \
    X(4, 1, 1, 3, 0) X(2, 1, 1, 2, 1) X(2, 1, 2, 2, 1) X(2, 1, 3, 2, 1) X(4, 1, 1, 2, 1) X(4, 1, 2, 2, 1) \
    X(2, 2, 1, 2, 1) X(2, 1, 1, 3, 1) X(4, 1, 2, 3, 1)

#define PKV_GQA_FP8_KEY(NW_, CH_, PF_, W_, KD_) ((KD_) * 10000 + (W_) * 1000 + (NW_) * 100 + (CH_) * 10 + (PF_))

template <int DT, int D>
static hipError_t launch_gqa_fp8_d(int nw, int ch, int pf, int wpe, int kd, const AttnArgs& a, unsigned grid,
                                   hipStream_t s) {
    switch (PKV_GQA_FP8_KEY(nw, ch, pf, wpe, kd)) {
#define PKV_CASE(NW_, CH_, PF_, W_, KD_)                                                                     \
    case PKV_GQA_FP8_KEY(NW_, CH_, PF_, W_, KD_):                                                            \
        hipLaunchKernelGGL((decode_gqa_fp8_kernel<DT, D, NW_, CH_, PF_, W_, KD_ != 0>), dim3(grid),          \
                           dim3(NW_ * 64), 0, s, a);                                                         \
        return hipGetLastError();
        PKV_GQA_FP8_VARIANTS(PKV_CASE)
#undef PKV_CASE
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_gqa_fp8(int dtype, int D, int nw, int ch, int pf, int wpe, int kd, const AttnArgs& a,
                                 unsigned grid, hipStream_t stream) {
    switch (dtype * 1000 + D) {
    case DT_F16 * 1000 + 64: return launch_gqa_fp8_d<DT_F16, 64>(nw, ch, pf, wpe, kd, a, grid, stream);
    case DT_F16 * 1000 + 128: return launch_gqa_fp8_d<DT_F16, 128>(nw, ch, pf, wpe, kd, a, grid, stream);
    case DT_BF16 * 1000 + 64: return launch_gqa_fp8_d<DT_BF16, 64>(nw, ch, pf, wpe, kd, a, grid, stream);
    case DT_BF16 * 1000 + 128: return launch_gqa_fp8_d<DT_BF16, 128>(nw, ch, pf, wpe, kd, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

bool gqa_fp8_variant_exists(int nw, int ch, int pf, int wpe, int kd) {
    switch (PKV_GQA_FP8_KEY(nw, ch, pf, wpe, kd)) {
#define PKV_CASE(NW_, CH_, PF_, W_, KD_) case PKV_GQA_FP8_KEY(NW_, CH_, PF_, W_, KD_):
        PKV_GQA_FP8_VARIANTS(PKV_CASE)
#undef PKV_CASE
        return true;
    default: return false;
    }
}

}  // namespace pkv
