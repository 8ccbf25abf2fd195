// Internal helpers shared by the libwush translation units: thread-local error
// text, status shortcuts and argument checks.  Not part of the public ABI.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/wush.h"

namespace wush {

// Record a formatted message as the thread's last error and return `st`.
wush_status fail(wush_status st, const char* fmt, ...);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace wush

#define WUSH_REQUIRE(cond, st, ...)                         \
  do {                                                      \
    if (!(cond)) return ::wush::fail((st), __VA_ARGS__);    \
  } while (0)
