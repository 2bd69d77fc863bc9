// common.hip -- error reporting and device checks shared by every entry point.
#include <cstdarg>
#include <cstring>
#include <mutex>

#include "common.hpp"

namespace bakron {

static thread_local char g_last_error[512] = "";

void set_error(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

int32_t check_device() {
    static std::mutex mu;
    static int cached[64] = {0};  // 0 unknown, 1 ok, 2 unsupported
    int dev = 0;
    BK_HIP_CHECK(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) {
        set_error("device index %d out of range", dev);
        return BAKRON_ERR_UNSUPPORTED_DEVICE;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        hipDeviceProp_t prop;
        BK_HIP_CHECK(hipGetDeviceProperties(&prop, dev));
        cached[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        if (cached[dev] == 2)
            set_error("device %d is %s; this library is built for gfx950 only", dev,
                      prop.gcnArchName);
    }
    return cached[dev] == 1 ? BAKRON_OK : BAKRON_ERR_UNSUPPORTED_DEVICE;
}

}  // namespace bakron

extern "C" const char *bakron_status_string(int32_t s) {
    switch (s) {
        case BAKRON_OK: return "ok";
        case BAKRON_ERR_INVALID_ARG: return "invalid argument";
        case BAKRON_ERR_WORKSPACE: return "workspace too small";
        case BAKRON_ERR_HIP: return "HIP runtime error";
        case BAKRON_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
        default: return "unknown status";
    }
}

extern "C" const char *bakron_last_error(void) { return bakron::g_last_error; }
