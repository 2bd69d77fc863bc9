// common.hpp -- shared host/device helpers of libbakron (HIP, gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "bakron.h"

namespace bakron {

// thread-local message behind bakron_last_error()
void set_error(const char *fmt, ...);
void clear_error();

// Returns BAKRON_OK when the current device is a gfx950 part (checked once per
// device and cached), else BAKRON_ERR_UNSUPPORTED_DEVICE / BAKRON_ERR_HIP.
int32_t check_device();

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// carve consecutive 256-byte aligned regions out of a workspace
struct Carver {
    char *base;
    size_t used = 0;
    explicit Carver(void *p) : base(static_cast<char *>(p)) {}
    template <class T>
    T *take(size_t count) {
        T *p = reinterpret_cast<T *>(base + used);
        used += align256(count * sizeof(T));
        return p;
    }
};

}  // namespace bakron

#define BK_HIP_CHECK(expr)                                                         \
    do {                                                                           \
        hipError_t bk_e_ = (expr);                                                 \
        if (bk_e_ != hipSuccess) {                                                 \
            ::bakron::set_error("%s failed: %s", #expr, hipGetErrorString(bk_e_)); \
            return BAKRON_ERR_HIP;                                                 \
        }                                                                          \
    } while (0)

#define BK_LAUNCH_CHECK(what)                                                      \
    do {                                                                           \
        hipError_t bk_e_ = hipGetLastError();                                      \
        if (bk_e_ != hipSuccess) {                                                 \
            ::bakron::set_error("launch of %s failed: %s", what,                   \
                                hipGetErrorString(bk_e_));                         \
            return BAKRON_ERR_HIP;                                                 \
        }                                                                          \
    } while (0)

#define BK_REQUIRE(cond, ...)                 \
    do {                                      \
        if (!(cond)) {                        \
            ::bakron::set_error(__VA_ARGS__); \
            return BAKRON_ERR_INVALID_ARG;    \
        }                                     \
    } while (0)
