// kv_append_mxfp4.hip -- quantize each request's new K/V rows into an MXFP4 pool.
//
// The block the new token needs is already in the request's table ("从
// PagedAttention 到 Prefill-Decode 分离的深度解析", section 2.2, step three);
// the row is stored as 4-bit codes with one power-of-two scale per 32 elements
// (same page, section 6.2; the format is described in pkv_mxfp4.h).  Each
// (request, KV head, K or V) row is one wave: lane l takes elements 2l and 2l+1
// (D / 2 lanes), the maximum of each 32-element block comes from a 16-lane
// reduction, every lane writes its code byte and the first lane of each 16
// writes the block's scale byte.  A request whose position or target block id
// is out of range is skipped.
#include "pkv_mxfp4.h"
#include "pkv_launch.h"

namespace pkv {

template <int SDT, int D>
__global__ __launch_bounds__(256) void kv_append_mxfp4_kernel(const AppendMx4Args a) {
    constexpr int ES = Dt<SDT>::bytes;
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

    const bool on = lane < D / 2;                 // D = 64: lanes 32..63 carry zeros and write nothing
    float x[2] = {0.0f, 0.0f};
    if (on) {
        const char* src = (which ? a.v_new : a.k_new) + ((size_t)b * a.new_row_stride + (size_t)g * D + 2 * lane) * ES;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if constexpr (SDT == DT_F32) {
                x[i] = reinterpret_cast<const float*>(src)[i];
            } else {
                const uint16_t u = reinterpret_cast<const uint16_t*>(src)[i];
                if constexpr (SDT == DT_F16) x[i] = (float)__builtin_bit_cast(_Float16, u);
                else x[i] = __uint_as_float((uint32_t)u << 16);
            }
        }
    }
    int E;
    const uint32_t byte = mx4_quantize_pair(x[0], x[1], E);
    const size_t row = ((size_t)blk * a.H_kv + g) * kBlockSize + p % kBlockSize;
    if (on) {
        (which ? a.v_pool : a.k_pool)[row * (D / 2) + lane] = (uint8_t)byte;
        if ((lane & 15) == 0) (which ? a.v_scale : a.k_scale)[row * (D / 32) + lane / 16] = (uint8_t)(E + 127);
    }
}

template <int SDT, int D>
static hipError_t launch_t(const AppendMx4Args& a, hipStream_t stream) {
    const int64_t waves = (int64_t)a.B * a.H_kv * 2;
    if (waves == 0) return hipSuccess;
    hipLaunchKernelGGL((kv_append_mxfp4_kernel<SDT, D>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_kv_append_mxfp4(int src_dtype, int D, const AppendMx4Args& a, hipStream_t stream) {
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
