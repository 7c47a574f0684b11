// cu_streams.cpp -- streams restricted to a subset of compute units (C ABI in include/pkv.h).
//
// Decode attention is bound by memory bandwidth, so a small share of the
// GPU's SMs already draws most of it and the rest can serve other work ("Injecting
// Adrenaline into LLM Serving" review, section 3.3).  On MI355X the share is
// expressed as a CU mask on a stream; every decode entry point accepts such a
// stream.  The mask builder is host-only and needs no GPU.
#include <hip/hip_runtime.h>

#include <cstring>

#include "pkv.h"
#include "pkv_host.h"

using pkv::fail;

extern "C" {

int pkv_device_cu_count(void) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    int n = 0;
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "CU count: %s", hipGetErrorString(e));
    pkv::clear_error();
    return n;
}

int pkv_cu_mask(int32_t n_cus, int32_t count, int layout, uint32_t* mask, int32_t n_words) {
    if (!mask) return fail(PKV_ERR_NULL, "mask is NULL");
    if (n_words <= 0 || n_cus <= 0 || n_cus > 32 * (int64_t)n_words || count < 1 || count > n_cus)
        return fail(PKV_ERR_INVALID_ARG, "need 1 <= count (%d) <= n_cus (%d) <= 32 * n_words (%d)", count, n_cus,
                    32 * n_words);
    if (layout != 0 && layout != 1) return fail(PKV_ERR_INVALID_ARG, "layout = %d (0 = first, 1 = spread)", layout);
    std::memset(mask, 0, sizeof(uint32_t) * (size_t)n_words);
    for (int32_t j = 0; j < count; ++j) {
        const int64_t cu = layout == 0 ? j : (int64_t)j * n_cus / count;
        mask[cu / 32] |= 1u << (cu % 32);
    }
    pkv::clear_error();
    return PKV_OK;
}

int pkv_stream_create_cu_masked(const uint32_t* mask, int32_t n_words, void** stream) {
    if (!mask || !stream) return fail(PKV_ERR_NULL, "mask and stream must not be NULL");
    if (n_words <= 0 || n_words > 64) return fail(PKV_ERR_INVALID_ARG, "n_words = %d", n_words);
    bool any = false;
    for (int32_t w = 0; w < n_words; ++w) any |= mask[w] != 0;
    if (!any) return fail(PKV_ERR_INVALID_ARG, "the mask selects no CU");
    hipStream_t s = nullptr;
    const hipError_t e = hipExtStreamCreateWithCUMask(&s, (uint32_t)n_words, mask);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "CU-masked stream: %s", hipGetErrorString(e));
    *stream = s;
    pkv::clear_error();
    return PKV_OK;
}

int pkv_stream_destroy(void* stream) {
    if (!stream) return fail(PKV_ERR_NULL, "stream is NULL");
    const hipError_t e = hipStreamDestroy(reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "stream destroy: %s", hipGetErrorString(e));
    pkv::clear_error();
    return PKV_OK;
}

}  // extern "C"
