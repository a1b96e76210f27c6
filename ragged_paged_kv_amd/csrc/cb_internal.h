// Internal helpers shared by the library's translation units (not part of the C ABI).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "cbattn.h"

namespace cb {

// Records `msg` as this thread's last error and returns `status`.
int fail(int status, const std::string& msg);
// Clears this thread's last error; returns CB_OK.
int ok();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace cb
