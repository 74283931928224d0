// Internal helpers shared by the translation units of libpagedkv.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "pagedkv.h"

namespace pkv {

// Record a failure message for pkv_last_error() (thread-local) and return `code`.
int fail(int code, const char* fmt, ...);
// Clear the message of the calling thread.
void clear_error();

inline const char* dtype_name(int32_t d) {
  switch (d) {
    case PKV_F32: return "f32";
    case PKV_BF16: return "bf16";
    case PKV_FP8_E4M3: return "fp8_e4m3";
    default: return "?";
  }
}

inline int elem_bytes(int32_t d) {
  switch (d) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

// Validate a cache descriptor; returns PKV_OK or an error (with message).
int check_desc(const pkv_cache_desc* c);

}  // namespace pkv
