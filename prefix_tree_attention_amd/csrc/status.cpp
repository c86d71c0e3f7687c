// Per-thread error state of libtreeattn (tree_last_error).  Host-only C++:
// together with pack.cpp it builds without the HIP runtime, which is how the
// packer is also compiled under AddressSanitizer and UBSan on the CPU.

#include <cstdarg>
#include <cstdio>
#include <string>

#include "status.h"

namespace treeattn {

namespace {
thread_local std::string g_last_error;
}

int set_error(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void clear_error() { g_last_error.clear(); }

}  // namespace treeattn

extern "C" const char* tree_last_error(void) { return treeattn::g_last_error.c_str(); }
