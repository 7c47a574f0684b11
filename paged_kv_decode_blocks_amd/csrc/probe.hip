// probe.hip -- a plain streaming-read kernel, used only to measure the HBM read
// bandwidth the device actually sustains (the practical ceiling next to the
// nameplate peak).  Not part of the decode step.
//
// Every lane reads 16 bytes per access with a grid-stride loop, four accesses
// in flight per iteration, and folds them into one word so the loads cannot be
// dropped; nothing is written unless the fold hits one specific value.
#include "pkv_launch.h"

namespace pkv {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p, size_t n16,
                                                          unsigned* sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    unsigned acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4_t a = __builtin_nontemporal_load(p + i);
        const u32x4_t b = __builtin_nontemporal_load(p + i + stride);
        const u32x4_t c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4_t d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const u32x4_t a = __builtin_nontemporal_load(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* sink, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<const u32x4_t*>(buf),
                       bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace pkv
