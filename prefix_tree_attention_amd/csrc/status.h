// Internal: per-thread error message and status helpers shared by the C ABI
// translation units of libtreeattn.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "tree_attn.h"

namespace treeattn {

// Records the message for tree_last_error() and returns `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

}  // namespace treeattn
