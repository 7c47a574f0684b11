// lse_merge.hip -- combine split-KV partitions of paged decode attention.
//
// Partition i of a (request, head) row holds o_i = its softmax-normalised
// output over tokens [i*P, min((i+1)*P, n)) and lse_i = log2 of its sum of
// exp2 scores.  The whole-context output is
//   out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M),   M = max_i lse_i,
// an exact regrouping of the softmax sum.  One wave per row; partitions are
// added in index order, so the result does not depend on scheduling.  A NaN
// lse (a partition that met an out-of-range block id) makes the row NaN.
#include "pkv_launch.h"

namespace pkv {

template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeArgs a) {
    constexpr int PER = D / 64;   // output elements per lane
    constexpr int U = 8;          // partial rows in flight per lane
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
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
    // global max over all partitions (lane p holds partitions p, p + 64, ...)
    float M = -__builtin_inff();
    bool nan = false;
    for (int p = lane; p < np; p += 64) {
        const float x = lse[p];
        nan |= (x != x);
        M = fmaxf(M, x);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    nan = __any(nan);
    float L = 0.0f;
    for (int p0 = 0; p0 < np; p0 += 64) {
        // lane p holds the weight of partition p0 + p; the partial rows are then read
        // U at a time, in partition order, each weight taken from its lane
        const int pl = p0 + lane;
        const float wl = pl < np ? __builtin_amdgcn_exp2f(lse[pl] - M) : 0.0f;
        L += wl;
        const int cnt = min(64, np - p0);
        for (int q0 = 0; q0 < cnt; q0 += U) {
            float v[U][PER];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < PER; ++k)
                    v[u][k] = q0 + u < cnt ? po[(size_t)(p0 + q0 + u) * D + lane + 64 * k] : 0.0f;
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
    const float inv = 1.0f / L;
#pragma unroll
    for (int k = 0; k < PER; ++k) o[lane + 64 * k] = nan ? __builtin_nanf("") : acc[k] * inv;
}

hipError_t launch_lse_merge(int D, const MergeArgs& a, hipStream_t stream) {
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
