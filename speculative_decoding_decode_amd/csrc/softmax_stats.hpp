// Row softmax of the lm-head from the statistics its contraction leaves, shared by the softmax
// finalize (spec_lm_head) and the row-statistics kernel of the fused lm-head + accept call
// (spec_lm_head_accept), so both compute every p entry with the same operations on the same
// values, bit for bit.
//
// What is computed (butteryoon "Gemma 4 MTP 서빙 가이드 해설", section 4: the target's own
// distribution p over the vocabulary at every verified position; temperature T per row, T <= 0
// meaning greedy one-hot).  With c = log2(e) / T:
//   block statistics   per 256-row vocabulary block and row: the block max m_b, the sum
//                      s_b = sum over the block of 2^((z - m_b) c), the block's first argmax;
//                      the contraction also writes e = 2^((z - m_b) c) in place of p;
//   row statistics     M = max over blocks, A = first argmax, L = sum_b s_b 2^((m_b - M) c);
//   p                  p = e * (2^((m_b - M) c) * (1 / L))   (greedy rows: p = [index == A]).
// Reduction order (fixed, so every workgroup that reduces a row gets the same bits): thread t
// of a 256-thread workgroup takes the maximum and then the rescaled sum of blocks t, t + 256,
// ... in order; the 64 lanes of a wave combine by the fixed DPP / readlane pattern of
// spec::wave_argmax and spec::wave_sum; the four waves' results are combined in wave order.
#pragma once

#include <limits.h>

#include "common.hpp"

namespace spec {

constexpr int kStatBlock = 256;        // vocabulary rows per statistics block
constexpr float kStatLog2e = 1.4426950408889634f;

// log2(e) / T, or 0 for a greedy row (T <= 0).
__device__ __forceinline__ float stat_scale(float t) { return t > 0.f ? kStatLog2e / t : 0.f; }

// Where the contraction leaves its statistics ([nblk][R], row fastest).
struct StatsOut {
  float2 *stats;      // (block max, block sum)
  int *amax;          // block first argmax
  int nblk;
};

// Workspace layout of the lm-head statistics (host side; defined in lm_head.hip): block
// statistics, then the row statistics of the fused call.
struct LmLayout {
  int nblk;
  size_t off_stats, off_amax, off_rows, bytes;
};
LmLayout lm_layout(int R, int V);
StatsOut lm_stats_out(const LmLayout &l, void *ws);
// Host-side argument checks of the lm-head calls.
int lm_head_check(const void *hidden, const void *weight, const float *temperature,
                  const float *probs, const float *logits, int R, int H, int V, spec_dtype dtype,
                  const char *who);
// Enqueue the contraction: logits (optional), e = 2^((z - block max) c) into `probs` for rows
// with T > 0, block statistics into `so`.
int lm_head_contract(const void *hidden, const void *weight, const float *temperature,
                     float *logits, float *probs, const StatsOut &so, int R, int H, int V,
                     spec_dtype dtype, hipStream_t st);

// ---------------------------------------------------------------- row statistics
struct RowStat {
  float m;     // row max M
  float inv;   // 1 / L
  float c;     // log2(e) / T, 0 for a greedy row
  int a;       // first argmax A
};

// Enqueue one workgroup per row writing RowStat rows[R] (the fused call's row statistics).
int lm_row_stats_launch(const StatsOut &so, const float *temperature, RowStat *rows, int R,
                        hipStream_t st);

// Row statistics of row r from its nblk block statistics, computed by a whole workgroup of
// THREADS threads in the order stated at the top of this file.  c = stat_scale(T of row r).
// All threads must call it; every thread gets the result.  sm, ss, si: LDS of THREADS / 64
// entries each.
template <int THREADS>
__device__ RowStat row_stat_wg(const float2 *__restrict__ stats, const int *__restrict__ amax,
                               int R, int r, int nblk, float c, float *sm, float *ss, int *si) {
  constexpr int NW = THREADS / kWave, U = 4;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  float m = -INFINITY, s = 0.f;
  int a = INT_MAX;
  for (int base = 0; base < nblk; base += THREADS * U) {
    float2 v[U];
    int ia[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = min(base + tid + THREADS * u, nblk - 1);
      v[u] = stats[(size_t)j * R + r];
      ia[u] = amax[(size_t)j * R + r];
    }
    // this thread's maximum (and first argmax) over the batch, then its rescaled sum
    float bm = -INFINITY;
    int ba = INT_MAX;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + tid + THREADS * u < nblk && first_max_better(bm, ba, v[u].x, ia[u])) { bm = v[u].x; ba = ia[u]; }
    if (bm != -INFINITY) {
      float bs = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (base + tid + THREADS * u < nblk) bs += v[u].y * exp2f((v[u].x - bm) * c);
      if (first_max_better(m, a, bm, ba)) a = ba;
      const float nm = fmaxf(m, bm);
      s = (m == -INFINITY ? 0.f : s * exp2f((m - nm) * c)) + bs * exp2f((bm - nm) * c);
      m = nm;
    }
  }
  float M = m;
  int A = a;
  wave_argmax(M, A);
  const float S = wave_sum(m == -INFINITY ? 0.f : s * exp2f((m - M) * c));
  if (lane == 0) { sm[wave] = M; ss[wave] = S; si[wave] = A; }
  __syncthreads();
  float Mw = sm[0];
  int Aw = si[0];
#pragma unroll
  for (int w = 1; w < NW; ++w)
    if (first_max_better(Mw, Aw, sm[w], si[w])) { Mw = sm[w]; Aw = si[w]; }
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += sm[w] == -INFINITY ? 0.f : ss[w] * exp2f((sm[w] - Mw) * c);
  return RowStat{Mw, 1.f / L, c, Aw};
}

// p = e * factor for an entry of the block whose max is blk_max.
__device__ __forceinline__ float stat_factor(float blk_max, const RowStat &rs) {
  return exp2f((blk_max - rs.m) * rs.c) * rs.inv;
}

}  // namespace spec
