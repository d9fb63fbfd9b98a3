// HBM probes: a plain streaming read and a plain copy of a device buffer, the ceilings the
// verify step's kernels are compared with on the same box (the lm-head and attention kernels
// are HBM-bound streams; decoding is bound by streaming weights from memory, butteryoon "Gemma 4
// MTP 서빙 가이드 해설", introduction).  Not part of the verify step.
//
// Both use the load style of the step's streaming kernels: 16-byte nontemporal loads, each
// wave reading 1 KB contiguous per instruction, eight loads in flight per thread, a grid of 8
// workgroups of 256 threads per compute unit striding over the buffer.  The read probe folds
// every word into one XOR per wave (so no load is dead) and writes 4 words per workgroup.
#include "common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kWGsPerCU = 8;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void hbm_read_probe(const u32x4_t *__restrict__ src,
                                                            size_t n16,
                                                            uint32_t *__restrict__ sink) {
  const size_t step = (size_t)kThreads * kUnroll;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * step + threadIdx.x; base < n16;
       base += (size_t)gridDim.x * step) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  acc = (uint32_t)spec::wave_reduce((int)acc, [](int x, int y) { return x ^ y; });
  if ((threadIdx.x & (spec::kWave - 1)) == 0)
    sink[(size_t)blockIdx.x * (kThreads / spec::kWave) + threadIdx.x / spec::kWave] = acc;
}

__global__ __launch_bounds__(kThreads) void hbm_copy_probe(const u32x4_t *__restrict__ src,
                                                            size_t n16,
                                                            u32x4_t *__restrict__ dst) {
  const size_t step = (size_t)kThreads * kUnroll;
  for (size_t base = (size_t)blockIdx.x * step + threadIdx.x; base < n16;
       base += (size_t)gridDim.x * step) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

}  // namespace

extern "C" int spec_hbm_probe_grid(void) { return spec::device_cus() * kWGsPerCU; }

extern "C" int spec_hbm_probe(int mode, const void *src, void *dst, size_t bytes, void *stream) {
  spec::clear_error();
  SPEC_REQUIRE(mode == 0 || mode == 1, SPEC_EINVAL, "spec_hbm_probe: mode %d is not 0 or 1", mode);
  SPEC_REQUIRE(src != nullptr && dst != nullptr, SPEC_EINVAL, "spec_hbm_probe: null pointer");
  SPEC_REQUIRE(bytes > 0 && bytes % 16 == 0, SPEC_EINVAL,
               "spec_hbm_probe: bytes=%zu must be a positive multiple of 16", bytes);
  SPEC_REQUIRE((reinterpret_cast<uintptr_t>(src) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(dst) & 15u) == 0,
               SPEC_EINVAL, "spec_hbm_probe: src and dst need 16-byte alignment");
  const int grid = spec_hbm_probe_grid();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const auto *s = static_cast<const u32x4_t *>(src);
  if (mode == 0)
    hipLaunchKernelGGL(hbm_read_probe, dim3(grid), dim3(kThreads), 0, st, s, bytes / 16,
                       static_cast<uint32_t *>(dst));
  else
    hipLaunchKernelGGL(hbm_copy_probe, dim3(grid), dim3(kThreads), 0, st, s, bytes / 16,
                       static_cast<u32x4_t *>(dst));
  return spec::launched("spec_hbm_probe");
}
