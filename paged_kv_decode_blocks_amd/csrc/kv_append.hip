// kv_append.hip -- write each request's new K/V token into its pool slot.
//
// The caller has already allocated the block the new token needs and put it
// in the request's table ("从 PagedAttention 到 Prefill-Decode 分离的深度解析",
// section 2.2, step three); this kernel only moves bytes.  One thread copies
// 16 bytes of K and 16 bytes of V, so a (request, KV head) row of D elements
// is written by D*elem_bytes/16 consecutive threads with full-width stores.
// A request whose position or target block id is out of range is skipped.
#include "pkv_launch.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_append_kernel(const AppendArgs a) {
    const int chunks = a.D * a.elem_bytes / 16;            // 16-byte pieces per row
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)a.B * a.H_kv * chunks;
    if (tid >= total) return;
    const int c = (int)(tid % chunks);
    const int64_t bg = tid / chunks;
    const int g = (int)(bg % a.H_kv);
    const int b = (int)(bg / a.H_kv);
    const int p = a.positions[b];
    if (p < 0 || p / kBlockSize >= a.bt_stride) return;
    const int blk = a.block_tables[(int64_t)b * a.bt_stride + p / kBlockSize];
    if ((unsigned)blk >= (unsigned)a.n_blocks) return;
    const size_t dst = ((((size_t)blk * a.H_kv + g) * kBlockSize + p % kBlockSize) * a.D) * a.elem_bytes + c * 16;
    const size_t src = ((size_t)b * a.new_row_stride + (size_t)g * a.D) * a.elem_bytes + c * 16;
    st16(a.k_pool + dst, ld16_cached(a.k_new + src));
    st16(a.v_pool + dst, ld16_cached(a.v_new + src));
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.B * a.H_kv * (a.D * a.elem_bytes / 16);
    if (total == 0) return hipSuccess;
    const unsigned grid = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
