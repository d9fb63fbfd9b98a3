// Row softmax from the per-block statistics of the lm-head contraction: the reduction every
// finalize workgroup runs for its row, in a fixed order so all of them get the same bits.
//
// The contraction kernels leave, for every 256-row block of the vocabulary and every hidden row
// r, (block max of the logits, sum over the block of exp((z - block max) / T)) in stats and the
// block's first argmax in amax, and exp((z - block max) / T) in p.  A row's softmax is then
//   M = max over blocks, L = sum over blocks of sum_blk * exp((max_blk - M) / T),
//   p = exp((z - max_blk) / T) * exp((max_blk - M) / T) / L,
// (butteryoon "Gemma 4 MTP 서빙 가이드 해설", section 4: the target's own distribution p over
// the vocabulary at every verified position; temperature T, T <= 0 meaning greedy one-hot).
//
// Reduction order (fixed, so every workgroup that reduces a row gets the same bits): thread t
// merges blocks t, t + 256, t + 512, ... in that order; the 64 lanes of a wave are combined by
// the fixed DPP-and-readlane pattern of spec::wave_reduce (the same bits in every lane); the
// four waves' results are added in wave order.
#pragma once

#include "common.hpp"

namespace spec {

constexpr int kStatBlock = 256;        // vocabulary rows per statistics block
constexpr int kStatThreads = 256;      // threads of a workgroup that reduces a row
constexpr int kStatWaves = kStatThreads / kWave;
constexpr int kStatsPerThread = 4;     // blocks per thread and pass (V <= 262144 in one pass)
constexpr float kStatLog2e = 1.4426950408889634f;

__device__ __forceinline__ bool stat_better(float m, int a, float om, int oa) {
  return first_max_better(m, a, om, oa);
}

// log2(e) / T, or 0 for a greedy row (T <= 0).
__device__ __forceinline__ float stat_scale(float t) { return t > 0.f ? kStatLog2e / t : 0.f; }

struct RowPartial {
  float m;      // running max (-inf before any block)
  float s;      // running sum, relative to m
  int a;        // first argmax
};

// This thread's merge of blocks tid, tid + 256, ... of row r (stats laid out [nblk][R]).
__device__ __forceinline__ RowPartial stat_partial(const float2 *__restrict__ stats,
                                                   const int *__restrict__ amax, int R, int r,
                                                   int nblk, float c, int tid) {
  RowPartial w{-INFINITY, 0.f, 0x7fffffff};
  for (int b0 = 0; b0 < nblk; b0 += kStatThreads * kStatsPerThread) {
    float2 st[kStatsPerThread];
    int ia[kStatsPerThread];
#pragma unroll
    for (int i = 0; i < kStatsPerThread; ++i) {
      const int b = b0 + tid + i * kStatThreads;
      st[i] = b < nblk ? stats[(size_t)b * R + r] : make_float2(-INFINITY, 0.f);
      ia[i] = b < nblk ? amax[(size_t)b * R + r] : 0x7fffffff;
    }
#pragma unroll
    for (int i = 0; i < kStatsPerThread; ++i) {
      if (stat_better(w.m, w.a, st[i].x, ia[i])) w.a = ia[i];
      const float nm = fmaxf(w.m, st[i].x);
      if (nm != -INFINITY) {
        w.s = w.s * exp2f((w.m - nm) * c) + st[i].y * exp2f((st[i].x - nm) * c);
        w.m = nm;
      }
    }
  }
  return w;
}


// Global (max, first argmax) and sum of row partials over the workgroup, for NR rows at once
// (rows >= nrows are ignored).  sm / si / ss: LDS of kStatWaves * NR entries each.  Every
// thread gets the results.
template <int NR>
__device__ __forceinline__ void stat_reduce(const RowPartial (&w)[NR], float (&c)[NR], int nrows,
                                            float (&gmax)[NR], int (&garg)[NR], float (&gsum)[NR],
                                            float *sm, int *si, float *ss) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  float m[NR];
  int a[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    m[i] = w[i].m;
    a[i] = w[i].a;
    if (i < nrows) wave_argmax(m[i], a[i]);
    if (lane == 0) { sm[wave * NR + i] = m[i]; si[wave * NR + i] = a[i]; }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float gm = sm[i];
    int ga = si[i];
#pragma unroll
    for (int x = 1; x < kStatWaves; ++x)
      if (stat_better(gm, ga, sm[x * NR + i], si[x * NR + i])) { gm = sm[x * NR + i]; ga = si[x * NR + i]; }
    gmax[i] = gm;
    garg[i] = ga;
    float v = w[i].m == -INFINITY ? 0.f : w[i].s * exp2f((w[i].m - gm) * c[i]);
    if (i < nrows) v = wave_sum(v);
    if (lane == 0) ss[wave * NR + i] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float s = ss[i];
#pragma unroll
    for (int x = 1; x < kStatWaves; ++x) s += ss[x * NR + i];
    gsum[i] = s;
  }
}

// Rescale factor of block blk of a row: p = (value stored by the contraction) * factor.
__device__ __forceinline__ float stat_factor(float blk_max, float gmax, float c, float inv) {
  return exp2f((blk_max - gmax) * c) * inv;
}

}  // namespace spec
