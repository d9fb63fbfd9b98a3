// Shared host/device helpers of the verify-step library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <atomic>

#include "spec_verify.h"

namespace spec {

constexpr int kWave = 64;

// ---------------------------------------------------------------- host: status reporting
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int launched(const char *what);  // SPEC_OK, or SPEC_EHIP with the runtime's message
int device_cus();                // compute units of the current device (cached per device)
// Raise `kernel`'s dynamic-LDS limit to `bytes` on the current device, once per device.
// `done` holds one bit per device id (< 64; higher ids set the attribute on every call); the
// bit is set with an atomic OR after the attribute call succeeds, so concurrent first calls
// at worst both set it (the call is idempotent).
int ensure_dynamic_lds(const void *kernel, size_t bytes, std::atomic<uint64_t> &done,
                       const char *who);

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

// ---------------------------------------------------------------- device: wave reductions
// Reductions over the 64 lanes of a wave, the result in every lane.  Inside each 16-lane row
// the values move by DPP permutations, which are plain VALU operands (no LDS round trip):
// the neighbour in the quad, the other pair of the quad, the other quad of the half row
// (half-row mirror), the other half of the row (row mirror).  The four row results are then
// read from lanes 0, 16, 32 and 48 and combined as (r0 op r1) op (r2 op r3), so the result is
// the same bits in every lane and on every call.  All 64 lanes must be active.
template <int Ctrl>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, Ctrl, 0xf, 0xf, false);
}
template <int Ctrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, dpp_move<Ctrl>(__builtin_bit_cast(int, v)));
}
template <int Ctrl>
__device__ __forceinline__ uint64_t dpp_move(uint64_t v) {
  const uint32_t lo = (uint32_t)dpp_move<Ctrl>((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)dpp_move<Ctrl>((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ int lane_value(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ uint64_t lane_value(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp_move<0xb1>(v));    // quad_perm [1, 0, 3, 2]
  v = op(v, dpp_move<0x4e>(v));    // quad_perm [2, 3, 0, 1]
  v = op(v, dpp_move<0x141>(v));   // row_half_mirror
  v = op(v, dpp_move<0x140>(v));   // row_mirror
  return op(op(lane_value(v, 0), lane_value(v, 16)), op(lane_value(v, 32), lane_value(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}
__device__ __forceinline__ int wave_sum(int v) {
  return wave_reduce(v, [](int x, int y) { return x + y; });
}
__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
  return wave_reduce(v, [](uint64_t x, uint64_t y) { return x + y; });
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ int wave_max(int v) {
  return wave_reduce(v, [](int x, int y) { return max(x, y); });
}

// (om, oa) beats (m, a): larger value, or the same value at a lower index.
__device__ __forceinline__ bool first_max_better(float m, int a, float om, int oa) {
  return om > m || (om == m && oa < a);
}

// Largest value over the wave and the lowest index holding it, in every lane.
__device__ __forceinline__ void wave_argmax(float &m, int &a) {
  auto step = [&](float om, int oa) {
    if (first_max_better(m, a, om, oa)) { m = om; a = oa; }
  };
  step(dpp_move<0xb1>(m), dpp_move<0xb1>(a));
  step(dpp_move<0x4e>(m), dpp_move<0x4e>(a));
  step(dpp_move<0x141>(m), dpp_move<0x141>(a));
  step(dpp_move<0x140>(m), dpp_move<0x140>(a));
  float bm = lane_value(m, 0);
  int ba = lane_value(a, 0);
#pragma unroll
  for (int q = 1; q < 4; ++q) {
    const float om = lane_value(m, 16 * q);
    const int oa = lane_value(a, 16 * q);
    if (first_max_better(bm, ba, om, oa)) { bm = om; ba = oa; }
  }
  m = bm;
  a = ba;
}

}  // namespace spec

#define SPEC_REQUIRE(cond, code, ...)                 \
  do {                                                \
    if (!(cond)) return ::spec::fail((code), __VA_ARGS__); \
  } while (0)
