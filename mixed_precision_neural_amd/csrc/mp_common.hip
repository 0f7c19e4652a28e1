// Status strings, the per-thread last HIP error and the version string.
#include <stdio.h>
#include <string.h>

#include "mp_internal.h"

namespace {
thread_local char g_last_error[256] = "";
}

namespace mp {
mp_status hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return MP_OK;
    snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", where, hipGetErrorString(e),
             static_cast<int>(e));
    return e == hipErrorOutOfMemory ? MP_ERR_OUT_OF_MEMORY : MP_ERR_HIP;
}
}  // namespace mp

extern "C" const char* mp_status_string(mp_status s) {
    switch (s) {
    case MP_OK: return "MP_OK";
    case MP_ERR_INVALID_ARGUMENT: return "MP_ERR_INVALID_ARGUMENT";
    case MP_ERR_MISALIGNED: return "MP_ERR_MISALIGNED";
    case MP_ERR_UNSUPPORTED: return "MP_ERR_UNSUPPORTED";
    case MP_ERR_HIP: return "MP_ERR_HIP";
    case MP_ERR_OUT_OF_MEMORY: return "MP_ERR_OUT_OF_MEMORY";
    }
    return "MP_ERR_UNKNOWN";
}

extern "C" const char* mp_last_hip_error(void) { return g_last_error; }

extern "C" const char* mp_version(void) { return "libmp 0.1 gfx950"; }
