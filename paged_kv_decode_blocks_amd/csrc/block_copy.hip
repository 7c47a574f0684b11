// block_copy.hip -- whole-block device copies for copy-on-write of shared blocks.
//
// Several sequences may map one physical block (a shared prompt prefix,
// "从 PagedAttention 到 Prefill-Decode 分离的深度解析", section 2.3).  Before a
// sequence appends into a partly filled block that another sequence still maps,
// the host block manager gives it a fresh block, and this kernel copies the old
// block's contents there.  A block of one pool is H_kv * block_size * D
// contiguous elements, so a copy is a flat byte move: the launch is cut into
// 4 KiB pieces (256 threads x 16 bytes), one workgroup per piece, K pieces
// first, then V.  A pair whose ids are out of range is skipped.
#include "pkv_launch.h"

namespace pkv {

__global__ __launch_bounds__(256) void copy_blocks_kernel(const CopyArgs a) {
    const int64_t pieces = (a.block_bytes + kCopyPieceBytes - 1) / kCopyPieceBytes;
    const int64_t w = blockIdx.x;
    const int64_t per_pool = (int64_t)a.n * pieces;
    const bool is_v = w >= per_pool;
    const int64_t r = is_v ? w - per_pool : w;
    const int i = (int)(r / pieces);
    const int64_t off = (r % pieces) * kCopyPieceBytes + (int64_t)threadIdx.x * 16;
    const int s = a.src[i];
    const int d = a.dst[i];
    if ((unsigned)s >= (unsigned)a.n_blocks || (unsigned)d >= (unsigned)a.n_blocks) return;
    if (off >= a.block_bytes) return;
    char* pool = is_v ? a.v_pool : a.k_pool;
    st16(pool + (size_t)d * a.block_bytes + off, ld16_cached(pool + (size_t)s * a.block_bytes + off));
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
    const int64_t pieces = (a.block_bytes + kCopyPieceBytes - 1) / kCopyPieceBytes;
    const int64_t grid = (int64_t)a.n * 2 * pieces;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
