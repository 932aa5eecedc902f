// Internal helpers shared by the HIP translation units of libmoonep (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/moonep.h"

namespace moonep {

// ---------------------------------------------------------------- errors

void set_error(const char* fmt, ...);

#define MOONEP_REQUIRE(cond, ...)          \
  do {                                     \
    if (!(cond)) {                         \
      ::moonep::set_error(__VA_ARGS__);    \
      return MOONEP_EINVAL;                \
    }                                      \
  } while (0)

// Clears an error left on this thread by an earlier HIP call made by someone else,
// so that MOONEP_LAUNCH_CHECK reports only this library's launches.
inline void clear_stale_error() { (void)hipGetLastError(); }

#define MOONEP_LAUNCH_CHECK(what)                                                       \
  do {                                                                                  \
    hipError_t e_ = hipGetLastError();                                                  \
    if (e_ != hipSuccess) {                                                             \
      ::moonep::set_error("%s: launch failed: %s", what, hipGetErrorString(e_));        \
      return MOONEP_EHIP;                                                               \
    }                                                                                   \
  } while (0)

// Validates the shared dimensions; returns MOONEP_OK or MOONEP_EINVAL with a message.
int check_dims(const moonep_dims& d, const char* who);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t n_pairs(const moonep_dims& d) { return (int64_t)d.R * d.S * d.K; }

inline size_t elem_bytes(moonep_dtype t) { return t == MOONEP_BF16 ? 2 : 4; }

inline hipStream_t as_stream(moonep_stream s) { return reinterpret_cast<hipStream_t>(s); }

inline unsigned ceil_div_u(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// Number of compute units of the current device (cached per device).
int device_cu_count();

// ---------------------------------------------------------------- device helpers

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32: round to nearest even).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const __bf16 h = (__bf16)f;
  uint16_t u;
  __builtin_memcpy(&u, &h, 2);
  return u;
}

}  // namespace moonep
