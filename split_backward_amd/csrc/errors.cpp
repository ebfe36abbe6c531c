// Thread-local error message of the C ABI.
#include <string>

#include "common.h"

namespace zb {
namespace {
thread_local std::string g_last_error = "no error";
}
void set_error(const std::string& msg) { g_last_error = msg; }
int32_t fail(int32_t code, const std::string& msg) {
    g_last_error = msg;
    return code;
}
}  // namespace zb

extern "C" const char* zb_last_error(void) { return zb::g_last_error.c_str(); }
extern "C" const char* zb_version(void) { return "zb-stage 0.1 (gfx950)"; }
