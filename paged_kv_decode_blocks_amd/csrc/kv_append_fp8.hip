// kv_append_fp8.hip -- quantize each request's new K/V rows into an FP8 pool.
//
// The block the new token needs is already in the request's table ("从
// PagedAttention 到 Prefill-Decode 分离的深度解析", section 2.2, step three);
// a low-precision cache stores the row in few bits with a fine-grained scale
// (same page, section 6.2).  Each (request, KV head, K or V) row is one wave:
// the lanes take D / 64 elements each, the row maximum comes from a wave
// reduction, and every lane writes its codes; lane 0 writes the row's scale.
// A request whose position or target block id is out of range is skipped.
#include "pkv_fp8.h"
#include "pkv_launch.h"

namespace pkv {

template <int SDT, int D>
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(const AppendFp8Args a) {
    constexpr int ES = Dt<SDT>::bytes;
    constexpr int PER = D / 64;                   // elements per lane
    const int wave = (int)((blockIdx.x * 256 + threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    if (wave >= a.B * a.H_kv * 2) return;         // whole waves exit together
    const int which = wave & 1;                   // 0: K, 1: V
    const int bg = wave >> 1;
    const int g = bg % a.H_kv;
    const int b = bg / a.H_kv;
    const int p = a.positions[b];
    if (p < 0 || p / kBlockSize >= a.bt_stride) return;
    const int blk = a.block_tables[(int64_t)b * a.bt_stride + p / kBlockSize];
    if ((unsigned)blk >= (unsigned)a.n_blocks) return;

    const char* src = (which ? a.v_new : a.k_new) + ((size_t)b * a.new_row_stride + (size_t)g * D + lane * PER) * ES;
    float x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if constexpr (SDT == DT_F32) {
            x[i] = reinterpret_cast<const float*>(src)[i];
        } else {
            const uint16_t u = reinterpret_cast<const uint16_t*>(src)[i];
            if constexpr (SDT == DT_F16) x[i] = (float)__builtin_bit_cast(_Float16, u);
            else x[i] = __uint_as_float((uint32_t)u << 16);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = group_max<64>(amax);
    const int E = fp8_row_exponent(amax);
    const float inv = pow2f(-E);
    const size_t row = ((size_t)blk * a.H_kv + g) * kBlockSize + p % kBlockSize;
    uint8_t* dst = (which ? a.v_pool : a.k_pool) + row * D + lane * PER;
#pragma unroll
    for (int i = 0; i < PER; ++i) dst[i] = (uint8_t)fp8_encode(x[i] * inv);
    if (lane == 0) (which ? a.v_scale : a.k_scale)[row] = pow2f(E);
}

template <int SDT, int D>
static hipError_t launch_t(const AppendFp8Args& a, hipStream_t stream) {
    const int64_t waves = (int64_t)a.B * a.H_kv * 2;
    if (waves == 0) return hipSuccess;
    hipLaunchKernelGGL((kv_append_fp8_kernel<SDT, D>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_kv_append_fp8(int src_dtype, int D, const AppendFp8Args& a, hipStream_t stream) {
    switch (src_dtype * 1000 + D) {
    case DT_F32 * 1000 + 64: return launch_t<DT_F32, 64>(a, stream);
    case DT_F32 * 1000 + 128: return launch_t<DT_F32, 128>(a, stream);
    case DT_F16 * 1000 + 64: return launch_t<DT_F16, 64>(a, stream);
    case DT_F16 * 1000 + 128: return launch_t<DT_F16, 128>(a, stream);
    case DT_BF16 * 1000 + 64: return launch_t<DT_BF16, 64>(a, stream);
    case DT_BF16 * 1000 + 128: return launch_t<DT_BF16, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
