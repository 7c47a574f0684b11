// decode_mha.hip -- paged decode attention, one query head per workgroup.
//
// Decode attention reads each request's whole private K/V history once per
// step and does about one flop per byte, so it is bound by HBM bandwidth
// ("Injecting Adrenaline into LLM Serving" review, section 2.2: the decode
// attention kernel dominates decode time and consumes the HBM bandwidth).  The
// kernel is therefore built around the loads:
//
//  * K/V rows are read with 16-byte loads; the lanes of a wave cover whole
//    token rows, so each load instruction reads TPL consecutive rows of one
//    block (1 KiB contiguous for D = 128 f16).
//  * A workgroup owns one (request, query head, partition).  The physical block
//    ids of the partition are staged in LDS once (in windows of 256 blocks),
//    then read wave-uniformly; every block id is range-checked there.
//  * Each wave takes chunks of CH blocks round-robin, issues all K and V loads
//    of a chunk before using any of them, computes q.k with packed dot
//    instructions plus a DPP row reduction, and keeps an online softmax
//    (running max m, running sum l, output o) in the log2 domain.
//  * Lanes that share a row position keep separate softmax states, which are
//    merged once at the end, first across the wave with shuffles and then
//    across the waves through LDS.  With one partition the workgroup writes the
//    normalised output; otherwise it writes (o / l, m + log2 l) for the merge
//    kernel.
//
// The fused variant (APPEND) also performs the step's kv_append: the token at
// positions[b] is taken from k_new/v_new instead of the pool, and the lanes
// holding it write it to its pool slot.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kWindowBlocks = kMhaWindowTokens / kBlockSize;

// One work unit: (request, query head, partition) number `unit`, partition-major.
template <int DT, int D, int NW, int CH, int PF, bool APPEND>
__device__ __forceinline__ void mha_unit(const AttnArgs& a, const int unit) {
    constexpr int ES = Dt<DT>::bytes;
    constexpr int E = 16 / ES;                // elements per 16-byte lane vector
    constexpr int LPT = D / E;                // lanes per token row
    constexpr int TPL = 64 / LPT;             // tokens per wave-wide load
    constexpr int LPB = kBlockSize / TPL;     // loads per block
    constexpr int NL = CH * LPB;              // loads (and scores) per lane per chunk
    static_assert(TPL * LPT == 64 && LPB * TPL == kBlockSize, "unsupported shape");

    __shared__ int32_t s_ids[kWindowBlocks];
    __shared__ int s_bad;
    __shared__ float s_m[NW];
    __shared__ float s_l[NW];
    __shared__ float s_o[NW][D];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar)
    const int r = lane / LPT;
    const int c = lane % LPT;

    const int BH = a.B * a.H_q;
    const int pg = unit / BH;
    const int part = unit_part(a, pg);
    const int bh = unit - pg * BH;
    const int b = bh / a.H_q;
    const int h = bh - b * a.H_q;
    const int g = h / a.G;

    // Issued together, before the length is known: the length, this lane's q piece
    // and the partition's first window of block ids (clamped to the table row;
    // only the entries below the real block count are used).
    const int n = APPEND ? a.positions[b] + 1 : a.context_lens[b];
    const uint4 qv = ld16_cached(a.q + ((int64_t)b * a.q_row_stride + (int64_t)h * D + c * E) * ES);
    const int32_t* table = a.block_tables + (int64_t)b * a.bt_stride;
    const int first_blk = part * (a.part_tokens / kBlockSize);
    constexpr int PRE = (kWindowBlocks + NW * 64 - 1) / (NW * 64);
    int pre[PRE];
    {
        const int spec = min(min(a.part_tokens / kBlockSize, kWindowBlocks), a.bt_stride - first_blk);
#pragma unroll
        for (int k = 0; k < PRE; ++k) {
            const int t = threadIdx.x + k * NW * 64;
            pre[k] = t < spec ? table[first_blk + t] : 0;
        }
    }
    const bool bad_len = APPEND ? (n < 1 || n > a.max_context_len) : (n < 0 || n > a.max_context_len);
    float* out_row = a.out + (size_t)bh * D;
    if (bad_len || n == 0) {
        // unsplit: this workgroup owns the row; split: the merge kernel writes it
        if (a.n_parts == 1 && part == 0)
            for (int d = threadIdx.x; d < D; d += NW * 64) out_row[d] = bad_len ? __builtin_nanf("") : 0.0f;
        return;
    }
    const int start = part * a.part_tokens;
    if (start >= n) return;
    const int end = min(start + a.part_tokens, n);
    const int n_hist = APPEND ? n - 1 : n;   // tokens already in the pool
    const int lim = min(end, n_hist);
    // only the partition that ends at n holds the new token; a chunk may run past
    // its partition's last block, so every other partition must never match it
    const int pos_new = (APPEND && end == n) ? n - 1 : -1;

    float m = kNegBig, l = 0.0f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.0f;

    const int nblk = (end - start + kBlockSize - 1) / kBlockSize;
    const size_t blk_bytes = (size_t)a.H_kv * kBlockSize * D * ES;
    const size_t head_bytes = (size_t)g * kBlockSize * D * ES;
    // byte offset of this lane's 16 bytes for load i of a block
    int lane_off[LPB];
#pragma unroll
    for (int i = 0; i < LPB; ++i) lane_off[i] = ((i * TPL + r) * D + c * E) * ES;
    const size_t new_off = ((size_t)b * a.new_row_stride + (size_t)g * D + c * E) * ES;
    const bool writer = APPEND && (h % a.G) == 0;

    // Issue the K then V loads of the CH blocks starting at round-local block cb0.
    auto load_full = [&](uint4 (&kv)[NL], uint4 (&vv)[NL], int cb0) {
        const char* kb[CH];
        const char* vb[CH];
#pragma unroll
        for (int cb = 0; cb < CH; ++cb) {
            const int id = __builtin_amdgcn_readfirstlane(s_ids[cb0 + cb]);
            kb[cb] = a.k_pool + (size_t)id * blk_bytes + head_bytes;
            vb[cb] = a.v_pool + (size_t)id * blk_bytes + head_bytes;
        }
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
#pragma unroll
            for (int i = 0; i < LPB; ++i) kv[cb * LPB + i] = ld16(kb[cb] + lane_off[i]);
#pragma unroll
        for (int cb = 0; cb < CH; ++cb)
#pragma unroll
            for (int i = 0; i < LPB; ++i) vv[cb * LPB + i] = ld16(vb[cb] + lane_off[i]);
    };
    // Online-softmax update with one chunk: scores, running max, rescale, weighted V.
    auto accumulate = [&](const uint4 (&kv)[NL], const uint4 (&vv)[NL], const bool (&valid)[NL]) {
        float s[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) s[j] = mul_rn(group_sum<LPT>(dot16<DT>(qv, kv[j])), a.scale_log2);
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
            axpy16<DT>(o, p, vv[j]);
        }
    };
    bool all_valid[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) all_valid[j] = true;

    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    // The first window comes from the ids loaded up front; staging it before the
    // window loop ends their live range here, so nothing of it is held (or
    // spilled) across the loads of the loop.
#pragma unroll
    for (int k = 0; k < PRE; ++k) {
        const int t = threadIdx.x + k * NW * 64;
        if (t < min(kWindowBlocks, nblk)) {
            int id = pre[k];
            if ((unsigned)id >= (unsigned)a.n_blocks) {
                s_bad = 1;
                id = 0;
            }
            s_ids[t] = id;
        }
    }
    for (int r0 = 0; r0 < nblk; r0 += kWindowBlocks) {
        const int nr = min(kWindowBlocks, nblk - r0);
        if (r0 > 0) {
            __syncthreads();   // every wave is done with the previous window
            // the thread index is re-read here so that the per-thread staging
            // addresses are formed inside this rare branch instead of being
            // hoisted out of the loop and kept live across it
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            for (int t = tid; t < nr; t += NW * 64) {
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

        // Chunks that lie wholly below `lim` need no masking.  Each wave takes its
        // share of them through a PF-deep load pipeline: the loads of chunk i + PF are
        // issued as soon as chunk i has been consumed, so a wave keeps PF chunks of K/V
        // in flight while it computes.  Round-robin: wave w takes chunks w, w + NW, ...
        // of the window.  Partition per wave (a.wave_tokens > 0; the span is one
        // window): wave w takes the chunks of its own partition, blocks [wb0, wb1).
        const int tok_r = start + r0 * kBlockSize;
        const bool blocked = a.wave_tokens > 0;
        const int wb0 = blocked ? w * (a.wave_tokens / kBlockSize) : 0;
        const int wb1 = blocked ? min(wb0 + a.wave_tokens / kBlockSize, nr) : nr;
        const int nch_w = blocked ? max(0, (wb1 - wb0 + CH - 1) / CH) : nch;
        const int nfull_all = blocked ? max(0, min(nch_w, (lim - tok_r - wb0 * kBlockSize) / (CH * kBlockSize)))
                                      : max(0, min(nch, (lim - tok_r) / (CH * kBlockSize)));
        const int nf = blocked ? nfull_all : (w < nfull_all ? (nfull_all - w + NW - 1) / NW : 0);
        uint4 bk[PF][NL], bv[PF][NL];
        // round-local first block of the wave's chunk i
        auto chunk_of = [&](int i) { return blocked ? wb0 + i * CH : (w + NW * i) * CH; };
        if (nf >= PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) load_full(bk[u], bv[u], chunk_of(u));
            // steady state: every consumed buffer is refilled, no guards in the body
            int i = 0;
            for (; i + 2 * PF <= nf; i += PF) {
#pragma unroll
                for (int u = 0; u < PF; ++u) {
                    accumulate(bk[u], bv[u], all_valid);
                    load_full(bk[u], bv[u], chunk_of(i + PF + u));
                }
            }
            // drain: nf - i is in [PF, 2 PF)
            const int rem = nf - i - PF;
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                accumulate(bk[u], bv[u], all_valid);
                if (u < rem) load_full(bk[u], bv[u], chunk_of(i + PF + u));
            }
#pragma unroll
            for (int u = 0; u < PF; ++u)
                if (u < rem) accumulate(bk[u], bv[u], all_valid);
        } else {
            for (int i = 0; i < nf; ++i) {
                load_full(bk[0], bv[0], chunk_of(i));
                accumulate(bk[0], bv[0], all_valid);
            }
        }

        // The partial chunk (at most one per round, or per partition): masked loads,
        // and in the fused call the new token from k_new/v_new.
        const int k0 = blocked ? nfull_all : nfull_all + ((w - nfull_all) % NW + NW) % NW;
        for (int k = k0; k < nch_w; k += blocked ? 1 : NW) {
            const int cb0 = (blocked ? wb0 : 0) + k * CH;
            const int tok0 = start + (r0 + cb0) * kBlockSize;
            const char* kb[CH];
            const char* vb[CH];
#pragma unroll
            for (int cb = 0; cb < CH; ++cb) {
                const int id = __builtin_amdgcn_readfirstlane(cb0 + cb < wb1 ? s_ids[cb0 + cb] : 0);
                kb[cb] = a.k_pool + (size_t)id * blk_bytes + head_bytes;
                vb[cb] = a.v_pool + (size_t)id * blk_bytes + head_bytes;
            }
            uint4 kv[NL], vv[NL];
            bool valid[NL];
#pragma unroll
            for (int cb = 0; cb < CH; ++cb)
#pragma unroll
                for (int i = 0; i < LPB; ++i) {
                    const int j = cb * LPB + i;
                    const int t = tok0 + cb * kBlockSize + i * TPL + r;
                    kv[j] = make_uint4(0, 0, 0, 0);
                    vv[j] = make_uint4(0, 0, 0, 0);
                    valid[j] = false;
                    if (t < lim) {
                        kv[j] = ld16(kb[cb] + lane_off[i]);
                        vv[j] = ld16(vb[cb] + lane_off[i]);
                        valid[j] = true;
                    } else if (APPEND && t == pos_new) {
                        kv[j] = ld16_cached(a.k_new + new_off);
                        vv[j] = ld16_cached(a.v_new + new_off);
                        valid[j] = true;
                        if (writer && !any_bad) {
                            st16(a.k_pool_w + (kb[cb] - a.k_pool) + lane_off[i], kv[j]);
                            st16(a.v_pool_w + (vb[cb] - a.v_pool) + lane_off[i], vv[j]);
                        }
                    }
                }
            accumulate(kv, vv, valid);
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

// Two chunks of two blocks in flight need about 190 VGPRs; left unbounded the
// compiler takes all 256 of a lone wave plus one AGPR, and the kernel runs at one
// wave per SIMD.  That variant is held to two (four chunks of one block would
// spill there, so they keep the whole register file).
template <int DT, int D, int NW, int CH, int PF, bool APPEND>
__global__ __launch_bounds__(NW * 64, CH == 2 && PF == 2 ? 2 : 1) void decode_mha_kernel(const AttnArgs a) {
    mha_unit<DT, D, NW, CH, PF, APPEND>(a, blockIdx.x);
}

// Persistent form: gridDim.x workgroups walk the units round-robin.  With 16
// waves per workgroup and the register budget the body needs, a workgroup fills
// its CU's register file, so a grid of n workgroups runs on n CUs: the step on a
// bounded share of the GPU, next to whatever else runs on the other CUs ("Injecting
// Adrenaline into LLM Serving" review, section 3.3: a fraction of the GPU already
// draws most of the HBM bandwidth for decode attention).
template <int DT, int D, int CH, bool APPEND>
__global__ __launch_bounds__(1024) void decode_mha_persistent_kernel(const AttnArgs a) {
    const int units = a.n_parts * a.B * a.H_q;
    for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
        __syncthreads();   // the previous unit's readers of the shared arrays are done
        mha_unit<DT, D, 16, CH, 1, APPEND>(a, unit);
    }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <int DT, int D, int NW, int CH, int PF>
static hipError_t launch_mha_t(bool append, const AttnArgs& a, unsigned grid, hipStream_t stream) {
    if (append)
        hipLaunchKernelGGL((decode_mha_kernel<DT, D, NW, CH, PF, true>), dim3(grid), dim3(NW * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_mha_kernel<DT, D, NW, CH, PF, false>), dim3(grid), dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_mha_d(int nw, int ch, int pf, bool append, const AttnArgs& a, unsigned grid, hipStream_t s) {
    if constexpr (DT == DT_F32 && D == 128) {
        // f32 rows of 128 take 16 loads per 2-block chunk: the planner runs them with one
        // 2-block chunk in flight (deeper pipelines would spill), the only ones built
        if (ch != 2 || pf != 1) return hipErrorInvalidValue;
        if (nw == 4) return launch_mha_t<DT, D, 4, 2, 1>(append, a, grid, s);
        if (nw == 8) return launch_mha_t<DT, D, 8, 2, 1>(append, a, grid, s);
        return hipErrorInvalidValue;
    } else {
        switch (nw * 100 + ch * 10 + pf) {
        case 421: return launch_mha_t<DT, D, 4, 2, 1>(append, a, grid, s);
        case 422: return launch_mha_t<DT, D, 4, 2, 2>(append, a, grid, s);
        case 423: return launch_mha_t<DT, D, 4, 2, 3>(append, a, grid, s);
        case 412: return launch_mha_t<DT, D, 4, 1, 2>(append, a, grid, s);
        case 414: return launch_mha_t<DT, D, 4, 1, 4>(append, a, grid, s);
        case 822: return launch_mha_t<DT, D, 8, 2, 2>(append, a, grid, s);
        case 821: return launch_mha_t<DT, D, 8, 2, 1>(append, a, grid, s);
        default: return hipErrorInvalidValue;
        }
    }
}

hipError_t launch_decode_mha(int dtype, int D, int nw, int ch, int pf, bool append, const AttnArgs& a,
                             unsigned grid, hipStream_t stream) {
    switch (dtype * 1000 + D) {
    case DT_F32 * 1000 + 64: return launch_mha_d<DT_F32, 64>(nw, ch, pf, append, a, grid, stream);
    case DT_F32 * 1000 + 128: return launch_mha_d<DT_F32, 128>(nw, ch, pf, append, a, grid, stream);
    case DT_F16 * 1000 + 64: return launch_mha_d<DT_F16, 64>(nw, ch, pf, append, a, grid, stream);
    case DT_F16 * 1000 + 128: return launch_mha_d<DT_F16, 128>(nw, ch, pf, append, a, grid, stream);
    case DT_BF16 * 1000 + 64: return launch_mha_d<DT_BF16, 64>(nw, ch, pf, append, a, grid, stream);
    case DT_BF16 * 1000 + 128: return launch_mha_d<DT_BF16, 128>(nw, ch, pf, append, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int DT, int D, int CH>
static hipError_t launch_mha_p(bool append, const AttnArgs& a, unsigned grid, hipStream_t stream) {
    if (append)
        hipLaunchKernelGGL((decode_mha_persistent_kernel<DT, D, CH, true>), dim3(grid), dim3(1024), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_mha_persistent_kernel<DT, D, CH, false>), dim3(grid), dim3(1024), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_mha_persistent(int dtype, int D, bool append, const AttnArgs& a, unsigned grid,
                                        hipStream_t stream) {
    // 16 waves per workgroup leave 128 VGPRs per lane: bf16 D=128 takes one block per
    // chunk to stay inside them without spilling (f16 packs its PV products tighter)
    switch (dtype * 1000 + D) {
    case DT_F16 * 1000 + 64: return launch_mha_p<DT_F16, 64, 2>(append, a, grid, stream);
    case DT_F16 * 1000 + 128: return launch_mha_p<DT_F16, 128, 2>(append, a, grid, stream);
    case DT_BF16 * 1000 + 64: return launch_mha_p<DT_BF16, 64, 2>(append, a, grid, stream);
    case DT_BF16 * 1000 + 128: return launch_mha_p<DT_BF16, 128, 1>(append, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

bool mha_variant_exists(int nw, int ch, int pf) {
    switch (nw * 100 + ch * 10 + pf) {
    case 421: case 422: case 423: case 412: case 414: case 822: case 821: return true;
    default: return false;
    }
}

}  // namespace pkv
