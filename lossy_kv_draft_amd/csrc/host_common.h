// Host-side helpers shared by the library's sources (not part of the ABI): error
// reporting, stream handles, sizes.  Host-only code (the file stager) includes this
// header alone.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <stdarg.h>

#include "../../include/vc.h"
#include "../../include/vc_model.h"

namespace vc {

// ---------------------------------------------------------------- errors
void set_error(const char* fmt, ...);
void clear_error();

#define VC_REQUIRE(cond, ...)                        \
  do {                                               \
    if (!(cond)) {                                   \
      ::vc::set_error(__VA_ARGS__);                  \
      return VC_ERR_INVALID_ARG;                     \
    }                                                \
  } while (0)

#define VC_UNSUPPORTED(cond, ...)                    \
  do {                                               \
    if (!(cond)) {                                   \
      ::vc::set_error(__VA_ARGS__);                  \
      return VC_ERR_UNSUPPORTED;                     \
    }                                                \
  } while (0)

#define VC_HIP(expr)                                                              \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) {                                                       \
      ::vc::set_error("%s failed: %s", #expr, hipGetErrorString(e_));             \
      return VC_ERR_HIP;                                                          \
    }                                                                             \
  } while (0)

#define VC_LAUNCHED(name)                                                         \
  do {                                                                            \
    hipError_t e_ = hipGetLastError();                                            \
    if (e_ != hipSuccess) {                                                       \
      ::vc::set_error("launch of %s failed: %s", name, hipGetErrorString(e_));    \
      return VC_ERR_HIP;                                                          \
    }                                                                             \
  } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool valid_dtype(int32_t t) { return t == VC_F32 || t == VC_BF16; }
inline size_t dtype_bytes(int32_t t) { return t == VC_F32 ? 4 : 2; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace vc
