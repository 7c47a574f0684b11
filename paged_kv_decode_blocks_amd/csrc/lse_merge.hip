// lse_merge.hip -- combine split-KV partitions of paged decode attention.
//
// Partition i of a (request, head) row holds o_i = its softmax-normalised
// output over tokens [i*P, min((i+1)*P, n)) and lse_i = log2 of its sum of
// exp2 scores.  The whole-context output is
//   out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M),   M = max_i lse_i,
// an exact regrouping of the softmax sum.  Partitions are added in a fixed
// order, so the result does not depend on scheduling.  A NaN lse (a partition
// that met an out-of-range block id) makes the row NaN.  The even split of the
// grouped kernel merges its pieces the same way.
#include "pkv_launch.h"

namespace pkv {

// The largest lse of np partial rows (lse at lse[p * ls]) and whether any is NaN,
// in every lane of the wave.
__device__ __forceinline__ float merge_max(const float* lse, int ls, int np, int lane, bool& nan) {
    float M = -__builtin_inff();
    bool bad = false;
    for (int p = lane; p < np; p += 64) {
        const float x = lse[(size_t)p * ls];
        bad |= (x != x);
        M = fmaxf(M, x);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    nan = __any(bad);
    return M;
}

// acc += sum_p 2^(lse_p - M) o_p and the sum of the weights (returned, in every lane) over
// np partial rows (o_p at po[p * os .. + D), lane l holding elements l, l + 64, ...), in
// index order.
template <int D>
__device__ __forceinline__ float merge_accumulate(const float* lse, int ls, const float* po, size_t os, int np,
                                                  float M, int lane, float (&acc)[D / 64]) {
    constexpr int PER = D / 64;
    constexpr int U = 8;   // partial rows in flight per lane
    float L = 0.0f;
    for (int p0 = 0; p0 < np; p0 += 64) {
        // lane p holds the weight of partition p0 + p; the partial rows are then read
        // U at a time, in partition order, each weight taken from its lane
        const int pl = p0 + lane;
        const float wl = pl < np ? __builtin_amdgcn_exp2f(lse[(size_t)pl * ls] - M) : 0.0f;
        L += wl;
        const int cnt = min(64, np - p0);
        for (int q0 = 0; q0 < cnt; q0 += U) {
            float v[U][PER];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < PER; ++k)
                    v[u][k] = q0 + u < cnt ? po[(size_t)(p0 + q0 + u) * os + lane + 64 * k] : 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float wu = __shfl(wl, min(q0 + u, 63), 64);
#pragma unroll
                for (int k = 0; k < PER; ++k) acc[k] = fmaf(q0 + u < cnt ? wu : 0.0f, v[u][k], acc[k]);
            }
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off, 64);
    return L;
}

// Rows of at most kFewPieces partial rows (the common case) are merged in one pass:
// every lse and every partial row is loaded at once -- one round trip to memory instead
// of one for the lse values and another for the rows -- and the rows are added in index
// order with the weights merge_accumulate would use.
constexpr int kFewPieces = 16;

// acc += sum_p 2^(lse_p - M) o_p over np <= kFewPieces partial rows (lse at lse[p * ls], o_p
// at po[p * os ..], lane l holding elements l, l + 64, ...); returns the sum of the weights,
// sets M's NaN test in nan.
template <int D>
__device__ __forceinline__ float merge_few(const float* lse, int ls, const float* po, size_t os, int np, int lane,
                                           float (&acc)[D / 64], bool& nan) {
    constexpr int PER = D / 64;
    float l[kFewPieces];
    float v[kFewPieces][PER];
#pragma unroll
    for (int u = 0; u < kFewPieces; ++u) {
        l[u] = u < np ? lse[(size_t)u * ls] : -__builtin_inff();
#pragma unroll
        for (int k = 0; k < PER; ++k) v[u][k] = u < np ? po[(size_t)u * os + lane + 64 * k] : 0.0f;
    }
    float M = l[0];
    bool bad = l[0] != l[0];
#pragma unroll
    for (int u = 1; u < kFewPieces; ++u) {
        M = fmaxf(M, l[u]);
        bad |= l[u] != l[u];
    }
    nan = bad;
    float L = 0.0f;
#pragma unroll
    for (int u = 0; u < kFewPieces; ++u) {
        const float w = u < np ? __builtin_amdgcn_exp2f(l[u] - M) : 0.0f;
        L += w;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = fmaf(w, v[u][k], acc[k]);
    }
    return L;
}

// Split partitions: one wave per (request, head) row, row-contiguous partials.
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeArgs a) {
    constexpr int PER = D / 64;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + wave;
    if (row >= a.BH) return;
    const int b = row / a.H_q;
    const bool fused = a.positions != nullptr;
    const int n = fused ? a.positions[b] + 1 : a.context_lens[b];
    const bool bad_len = fused ? (n < 1 || n > a.max_context_len) : (n < 0 || n > a.max_context_len);
    float* o = a.out + (size_t)row * D;
    if (bad_len || n == 0) {
#pragma unroll
        for (int k = 0; k < PER; ++k) o[lane + 64 * k] = bad_len ? __builtin_nanf("") : 0.0f;
        return;
    }
    const int np = min((n + a.part_tokens - 1) / a.part_tokens, a.n_parts);
    const float* lse = a.part_lse + (size_t)row * a.n_parts;
    const float* po = a.part_o + (size_t)row * a.n_parts * D;
    bool nan;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
    float L;
    if (np <= kFewPieces) {
        L = merge_few<D>(lse, 1, po, D, np, lane, acc, nan);
    } else {
        const float M = merge_max(lse, 1, np, lane, nan);
        L = merge_accumulate<D>(lse, 1, po, D, np, M, lane, acc);
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int k = 0; k < PER; ++k) o[lane + 64 * k] = nan ? __builtin_nanf("") : acc[k] * inv;
}

// Even split (a.even_meta set): four (request, head) rows per 4-wave workgroup.
// A row's pieces are those of super-runs r0 .. r1, the super-runs of tw blocks
// that meet the request's blocks, with ids (r + b) H_kv + g (g the row's KV
// head); a row one super-run covered was written by that workgroup.  Rows of at most kWideMerge pieces
// take a wave each; otherwise (a few long requests: a hundred pieces per row) the
// four waves share each row in turn, wave w adding pieces w, w + 4, ..., and the
// four sums are added in wave order.
constexpr int kWideMerge = 16;

struct EvenRow {
    int np;        // pieces to merge (0: nothing left to do for this row)
    size_t first;  // index of the first piece's row in part_lse (part_o: times D)
    bool fill;     // the row is written here as NaN (bad length) or zeros (empty)
    bool nan;
};

__device__ __forceinline__ EvenRow even_row(const MergeArgs& a, int row) {
    EvenRow e{0, 0, false, false};
    if (row >= a.BH) return e;
    const int b = row / a.H_q;
    const bool fused = a.positions != nullptr;
    const int n = fused ? a.positions[b] + 1 : a.context_lens[b];
    const bool bad_len = fused ? (n < 1 || n > a.max_context_len) : (n < 0 || n > a.max_context_len);
    if (bad_len || n == 0) {
        e.fill = true;
        e.nan = bad_len;
        return e;
    }
    const int tw = a.even_meta[0];
    const int pre = a.even_meta[2 + b];
    const int nb = a.even_meta[3 + b] - pre;
    const int r0 = pre / tw, r1 = (pre + nb - 1) / tw;
    if (r0 == r1) return e;
    // piece (r + b) H_kv + g holds its G heads' rows at ((r + b) H_kv + g) G + h - g G = (r + b) H_q + h
    e.np = r1 - r0 + 1;
    e.first = ((size_t)r0 + b) * a.H_q + (row - b * a.H_q);
    return e;
}

template <int D>
__global__ __launch_bounds__(256) void lse_merge_even_kernel(const MergeArgs a) {
    constexpr int PER = D / 64;
    __shared__ float s_acc[4][D];
    __shared__ float s_l[4];
    __shared__ int s_np[4];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int row0 = blockIdx.x * 4;
    const EvenRow mine_row = even_row(a, row0 + wave);
    if (lane == 0) s_np[wave] = mine_row.np;
    __syncthreads();
    const int npmax = max(max(s_np[0], s_np[1]), max(s_np[2], s_np[3]));
    if (npmax <= kWideMerge) {   // a wave per row
        const EvenRow& e = mine_row;
        float* o = a.out + (size_t)(row0 + wave) * D;
        if (e.fill) {
#pragma unroll
            for (int k = 0; k < PER; ++k) o[lane + 64 * k] = e.nan ? __builtin_nanf("") : 0.0f;
        }
        if (e.np == 0) return;
        bool nan;
        float acc[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
        float L;
        if (e.np <= kFewPieces) {
            L = merge_few<D>(a.part_lse + e.first, a.H_q, a.part_o + e.first * D, (size_t)a.H_q * D, e.np, lane, acc,
                             nan);
        } else {
            const float M = merge_max(a.part_lse + e.first, a.H_q, e.np, lane, nan);
            L = merge_accumulate<D>(a.part_lse + e.first, a.H_q, a.part_o + e.first * D, (size_t)a.H_q * D, e.np, M,
                                    lane, acc);
        }
        const float inv = 1.0f / L;
#pragma unroll
        for (int k = 0; k < PER; ++k) o[lane + 64 * k] = nan ? __builtin_nanf("") : acc[k] * inv;
        return;
    }
    for (int i = 0; i < 4; ++i) {   // the four waves on each row in turn (workgroup-uniform control)
        const EvenRow e = even_row(a, row0 + i);
        float* o = a.out + (size_t)(row0 + i) * D;
        if (e.fill && wave == 0) {
#pragma unroll
            for (int k = 0; k < PER; ++k) o[lane + 64 * k] = e.nan ? __builtin_nanf("") : 0.0f;
        }
        if (e.np == 0) continue;
        bool nan;
        const float M = merge_max(a.part_lse + e.first, a.H_q, e.np, lane, nan);
        float acc[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
        const int mine = e.np > wave ? (e.np - wave + 3) / 4 : 0;
        const size_t f = e.first + (size_t)wave * a.H_q;
        const float L = merge_accumulate<D>(a.part_lse + f, 4 * a.H_q, a.part_o + f * D, (size_t)4 * a.H_q * D,
                                            mine, M, lane, acc);
#pragma unroll
        for (int k = 0; k < PER; ++k) s_acc[wave][lane + 64 * k] = acc[k];
        if (lane == 0) s_l[wave] = L;
        __syncthreads();
        if (wave == 0) {
            const float inv = 1.0f / (((s_l[0] + s_l[1]) + s_l[2]) + s_l[3]);
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int d = lane + 64 * k;
                const float x = ((s_acc[0][d] + s_acc[1][d]) + s_acc[2][d]) + s_acc[3][d];
                o[d] = nan ? __builtin_nanf("") : x * inv;
            }
        }
        __syncthreads();   // the next row reuses s_acc
    }
}

hipError_t launch_lse_merge(int D, const MergeArgs& a, hipStream_t stream) {
    if (a.even_meta) {
        if (D == 64)
            hipLaunchKernelGGL(lse_merge_even_kernel<64>, dim3((unsigned)((a.BH + 3) / 4)), dim3(256), 0, stream, a);
        else if (D == 128)
            hipLaunchKernelGGL(lse_merge_even_kernel<128>, dim3((unsigned)((a.BH + 3) / 4)), dim3(256), 0, stream,
                               a);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)((a.BH + 3) / 4);
    if (D == 64)
        hipLaunchKernelGGL(lse_merge_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
    else if (D == 128)
        hipLaunchKernelGGL(lse_merge_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pkv
