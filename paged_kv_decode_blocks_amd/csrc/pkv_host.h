// pkv_host.h -- host-side helpers shared by the C ABI translation units (internal to libpkv).
#pragma once

namespace pkv {

// Record a formatted detail for pkv_last_error() (thread-local) and return status.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the detail after a successful call.
void clear_error();

}  // namespace pkv
