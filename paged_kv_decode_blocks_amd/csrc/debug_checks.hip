// debug_checks.hip -- a decode step's device-side metadata checked against the
// contract the kernels assume (a debugging aid: synchronous, not on the hot path).
//
// A request's logical block j lives in physical block block_tables[b][j], and
// every new token is given a slot of its own ("从 PagedAttention 到 Prefill-Decode
// 分离的深度解析", section 2.2, steps two and three).  The attention and append
// kernels check lengths and block ids themselves (a bad one gives a NaN row or a
// skipped append, never an access through it), but two appends of one step that
// name the same (block, slot) they cannot see: which write lands is unspecified.
// pkv_check_step_metadata reports all three kinds of violation.
#include "pkv.h"
#include "pkv_host.h"
#include "pkv_launch.h"

#include <mutex>

using pkv::fail;

namespace {

constexpr unsigned kBadRange = 1u;   // a length or a block id out of range
constexpr unsigned kAliased = 2u;    // two appends target one (block, slot)

// The verdict word; in host code its name is only a stand-in, the device address
// comes from hipGetSymbolAddress once per device.
static __device__ __align__(256) unsigned int check_flags;

constexpr int kMaxDevices = 64;
std::mutex g_flags_mu;
void* g_flags_ptr[kMaxDevices] = {};

int flags_for_current_device(unsigned** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device %d (at most %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_flags_mu);
    if (!g_flags_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_flags));
        if (e != hipSuccess || !p) return fail(PKV_ERR_HIP, "hipGetSymbolAddress(check_flags): %s", hipGetErrorString(e));
        g_flags_ptr[dev] = p;
    }
    *ptr = reinterpret_cast<unsigned*>(g_flags_ptr[dev]);
    return PKV_OK;
}

struct CheckArgs {
    const int32_t* bt;
    const int32_t* ctx;   // attention lengths, or NULL
    const int32_t* pos;   // append positions, or NULL
    int32_t bt_stride, B, bs, n_blocks, max_ctx;
    unsigned* flags;
};

// The (block, slot) request b appends to as one 64-bit key, or -1 if it appends
// nothing or its target is out of range (reported as a range violation).
__device__ long long append_key(const CheckArgs& a, int b) {
    if (!a.pos || b >= a.B) return -1;
    const int p = a.pos[b];
    if (p < 0 || (long long)p >= (long long)a.bt_stride * a.bs) return -1;
    const int id = a.bt[(long long)b * a.bt_stride + p / a.bs];
    if (id < 0 || id >= a.n_blocks) return -1;
    return (long long)id * a.bs + p % a.bs;
}

__global__ void clear_flags_kernel(unsigned* flags) { flags[0] = 0u; }

__global__ __launch_bounds__(256) void check_metadata_kernel(const CheckArgs a) {
    __shared__ long long s_key[256];
    const int b = blockIdx.x * 256 + threadIdx.x;
    unsigned f = 0;
    long long key = -1;
    if (b < a.B) {
        const bool append = a.pos != nullptr;
        const bool fused = append && a.max_ctx > 0;
        const long long n = append ? (long long)a.pos[b] + 1 : a.ctx[b];
        const long long cap = (long long)a.bt_stride * a.bs;
        if (append ? (n < 1 || n > cap) : (n < 0 || n > cap)) f |= kBadRange;
        if ((fused || !append) && n > a.max_ctx) f |= kBadRange;
        if (!(f & kBadRange)) {
            // blocks the step reads (attention) or writes (append): all of 0 .. n-1, or the target
            const int first = (append && !fused) ? (int)((n - 1) / a.bs) : 0;
            for (int j = first; j < (int)((n + a.bs - 1) / a.bs); ++j) {
                const int id = a.bt[(long long)b * a.bt_stride + j];
                if (id < 0 || id >= a.n_blocks) f |= kBadRange;
            }
            key = append_key(a, b);
        }
    }
    // every other request's target, 256 at a time through LDS
    for (int t0 = 0; t0 < a.B; t0 += 256) {
        __syncthreads();
        s_key[threadIdx.x] = append_key(a, t0 + threadIdx.x);
        __syncthreads();
        if (key >= 0)
            for (int i = 0; i < 256 && t0 + i < a.B; ++i)
                if (t0 + i != b && s_key[i] == key) f |= kAliased;
    }
    if (f) atomicOr(a.flags, f);
}

}  // namespace

extern "C" int pkv_check_step_metadata(const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                                       const int32_t* positions, int32_t B, int32_t block_size, int32_t n_blocks,
                                       int32_t max_context_len, void* stream) {
    if ((context_lens == nullptr) == (positions == nullptr))
        return fail(PKV_ERR_INVALID_ARG, "pass exactly one of context_lens and positions");
    if (B < 0 || bt_stride <= 0 || block_size <= 0 || n_blocks <= 0 || max_context_len < 0)
        return fail(PKV_ERR_INVALID_ARG, "B = %d, bt_stride = %d, block_size = %d, n_blocks = %d, max = %d", B,
                    bt_stride, block_size, n_blocks, max_context_len);
    if (B == 0) {
        pkv::clear_error();
        return PKV_OK;
    }
    if (!block_tables) return fail(PKV_ERR_NULL, "block_tables is NULL");
    unsigned* flags = nullptr;
    int st = flags_for_current_device(&flags);
    if (st) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    CheckArgs a{block_tables, context_lens, positions, bt_stride, B, block_size, n_blocks, max_context_len, flags};
    hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(1), 0, s, flags);
    hipLaunchKernelGGL(check_metadata_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    unsigned host = 0;
    if (e == hipSuccess) e = hipMemcpyAsync(&host, flags, sizeof host, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "metadata check: %s", hipGetErrorString(e));
    if (host & kBadRange) return fail(PKV_ERR_INVALID_ARG, "a length or block id is outside the contract's range");
    if (host & kAliased) return fail(PKV_ERR_ALIASED_APPEND, "two appends of the step target the same (block, slot)");
    pkv::clear_error();
    return PKV_OK;
}

namespace pkv {

// PKV_DEBUG_CHECKS=1: every append entry point runs the check first (synchronous).
int debug_check_appends(const int32_t* block_tables, int32_t bt_stride, const int32_t* positions, int32_t B,
                        int32_t block_size, int32_t n_blocks, int32_t max_context_len, void* stream) {
    const char* v = getenv("PKV_DEBUG_CHECKS");   // read per call: a process may switch it on at any point
    if (!(v && *v && *v != '0') || B <= 0 || !positions) return PKV_OK;
    return pkv_check_step_metadata(block_tables, bt_stride, nullptr, positions, B, block_size, n_blocks,
                                   max_context_len, stream);
}

}  // namespace pkv
