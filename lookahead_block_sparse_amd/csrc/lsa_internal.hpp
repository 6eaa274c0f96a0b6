// Internal helpers shared by the LSA library sources (host and device).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "lsa.h"

namespace lsa {

// ---- errors -------------------------------------------------------------------------------
// Record a message for lsa_last_error() and return the status.
lsa_status fail(lsa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lsa_status hip_fail(hipError_t e, const char* what);

#define LSA_CHECK_ARG(cond, ...)                                     \
    do {                                                             \
        if (!(cond)) return ::lsa::fail(LSA_ERR_INVALID, __VA_ARGS__); \
    } while (0)
#define LSA_CHECK_SUP(cond, ...)                                         \
    do {                                                                 \
        if (!(cond)) return ::lsa::fail(LSA_ERR_UNSUPPORTED, __VA_ARGS__); \
    } while (0)
#define LSA_HIP(call)                                       \
    do {                                                    \
        hipError_t e_ = (call);                             \
        if (e_ != hipSuccess) return ::lsa::hip_fail(e_, #call); \
    } while (0)

// ---- device facts ---------------------------------------------------------------------------
struct DeviceInfo {
    int device = -1;
    int cu_count = 0;
};
// Properties of the current device (cached per device).
lsa_status current_device(DeviceInfo* out);

// Device-visible address of a buffer that is either device memory or pinned host memory mapped
// for the device (is_host tells which); fn names the calling entry point in error messages.
lsa_status device_view(const void* ptr, const char* fn, const char* what, const void** out, bool* is_host);

inline size_t elem_bytes(int32_t dtype) { return dtype == LSA_BF16 ? 2 : 4; }
inline bool dtype_ok(int32_t dtype) { return dtype == LSA_F32 || dtype == LSA_BF16; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- device-side helpers ----------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace lsa
