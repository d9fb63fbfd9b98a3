// Shared host/device helpers of the verify-step library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "spec_verify.h"

namespace spec {

constexpr int kWave = 64;

// ---------------------------------------------------------------- host: status reporting
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int launched(const char *what);  // SPEC_OK, or SPEC_EHIP with the runtime's message
int device_cus();                // compute units of the current device (cached per device)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- device: numerics
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static __forceinline__ float to_f32(float x) { return x; }
};
template <> struct Elem<uint16_t> {
  static constexpr int kPer16B = 8;
  __device__ static __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
};

// Unpack a 16-byte group of elements to fp32.
__device__ __forceinline__ void unpack16(const uint4 &v, float (&f)[4], float) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack16(const uint4 &v, float (&f)[8], uint16_t) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

}  // namespace spec

#define SPEC_REQUIRE(cond, code, ...)                 \
  do {                                                \
    if (!(cond)) return ::spec::fail((code), __VA_ARGS__); \
  } while (0)
