// status.hip -- per-thread error state of libgcq.so.
#include "gcq_internal.h"

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

}  // namespace gcq

GCQ_API const char* gc_last_error(void) { return gcq::last_error(); }
