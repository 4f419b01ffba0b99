// status.hip -- per-thread error state of libgcq.so and its host launch helpers.
#include "gcq_internal.h"

#include <cstdlib>

namespace gcq {

namespace {
thread_local std::string g_last_error;
}

void set_error(const std::string& msg) { g_last_error = msg; }

void clear_error() { g_last_error.clear(); }

int fail(gc_status code, const std::string& msg)
{
    g_last_error = msg;
    return code;
}

int check_launch(const char* what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(GC_EHIP, std::string(what) + ": " + hipGetErrorString(e));
    return GC_OK;
}

const char* last_error() { return g_last_error.c_str(); }

size_t max_grid_blocks()
{
    static const size_t cap = [] {
        size_t c = size_t(1) << 20;
        if (const char* env = std::getenv("GCQ_MAX_GRID_BLOCKS")) {
            const long long v = std::atoll(env);
            if (v >= 1 && size_t(v) < c)
                c = size_t(v);
        }
        return c;
    }();
    return cap;
}

}  // namespace gcq

GCQ_API const char* gc_last_error(void) { return gcq::last_error(); }
