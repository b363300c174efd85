// Error reporting shared by the library's translation units: a thread-local
// message behind pkv_last_error() and a helper that sets it and returns a code.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pkv.h"

namespace pkv {

std::string& last_error();

inline int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    last_error() = buf;
    return code;
}

inline int ok() {
    last_error().clear();
    return PKV_OK;
}

// Bytes of a query / output / input-row element (0: not such a type).
inline int elem_bytes(int dtype) {
    return dtype == PKV_F32 ? 4 : (dtype == PKV_F16 || dtype == PKV_BF16) ? 2 : 0;
}

// Bytes of a cache element: the types above plus the FP8 cache type.
inline int cache_elem_bytes(int dtype) { return dtype == PKV_FP8_E4M3 ? 1 : elem_bytes(dtype); }

}  // namespace pkv
