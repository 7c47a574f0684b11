// pkv_host.h -- host-side helpers shared by the C ABI translation units (internal to libpkv).
#pragma once

#include <cstdint>

namespace pkv {

// Record a formatted detail for pkv_last_error() (thread-local) and return status.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the detail after a successful call.
void clear_error();
// With PKV_DEBUG_CHECKS=1 in the environment: pkv_check_step_metadata on an append's
// positions (max_context_len 0 for a plain kv_append); PKV_OK otherwise.
int debug_check_appends(const int32_t* block_tables, int32_t bt_stride, const int32_t* positions, int32_t B,
                        int32_t block_size, int32_t n_blocks, int32_t max_context_len, void* stream);

}  // namespace pkv
