// Internal: per-thread error message and status helpers shared by the C ABI
// translation units of libtreeattn.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "tree_attn.h"

namespace treeattn {

// Records the message for tree_last_error() and returns `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Shape, dtype and scale checks shared by the attention entry points; sets
// the error and returns TREE_E_ARG on failure.
int check_attn(const char* fn, int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t dtype);

}  // namespace treeattn
