// Internal declarations shared by the translation units of libsgg_lora.
#pragma once

#include <cstdarg>
#include <cstdint>

namespace sgg {

// Records a formatted message for lora_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the calling thread's message and returns SGG_OK.
int ok();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

}  // namespace sgg
