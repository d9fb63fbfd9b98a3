// Accept / reject of the drafts and the correction or bonus draw.
//
// The pages: the target confirms the drafts up to the first one it rejects and generates the
// token at that position itself, keeping the output distribution that of the target alone
// (llm-wiki "Gemma 4 MTP: 드래프터가 초안을 쓰고 타깃이 검증하는 추론 가속 구조", section
// "투기적 디코딩의 기본 구조"; butteryoon "Gemma 4 MTP 서빙 가이드 해설", section 4 accept/reject
// step); when every draft is accepted the same forward also yields one extra token (GeekNews
// "Gemma 4 가속하기 : 다중 토큰 예측 drafter로 더 빠른 추론", section "MTP가 동작하는 방식").
// The rule is Leviathan et al.'s: accept draft i iff
// u_i < min(1, p_i(d_i) / q_i(d_i)); on the first rejection draw from norm(max(0, p - q)); after
// k acceptances draw the bonus token from p.
//
// Exactness on the GPU:
//  * the test u*q < p is evaluated on fp64 values; the product of two fp32 numbers is exact in
//    fp64, so the decision does not depend on rounding;
//  * the draw is an inverse CDF over integer weights floor(x * 2^38) summed in uint64, so every
//    reduction order gives the same bits; normalisation is never computed (the threshold is
//    floor(m * W / 2^24), m = floor(u * 2^24), W the weight total).
//
// Two kernels:
//  accept_chunks   grid (nchunks, B): every workgroup finds n for its sequence (one wave:
//                  lane i tests draft i, a ballot gives the first rejection) and sums the
//                  weights of one vocabulary chunk of the row it will be drawn from;
//  accept_draw     grid (B): one workgroup per sequence scans the chunk sums, finds the chunk
//                  holding the threshold, scans inside it and writes n and the tokens.
// (A single kernel whose last chunk workgroup per sequence draws, found with a completion
// counter, measured slower on MI355X at batch 1: the counter's round trip and the device-scope
// reads of the chunk sums cost more than the second launch.)
//
// spec_lm_head_accept runs the lm-head contraction, the row statistics (lm_row_stats, once per
// row) and these two kernels back to back, without the softmax finalize pass over p: the accept
// kernels form the p values they need (at the drafts and in the chunks of row n) from the
// contraction's exp values and the row statistics, with the operations of the finalize
// (softmax_stats.hpp), so the results equal spec_lm_head + spec_accept bit for bit.  This is the sampling pipeline run as part of the verify forward, the role the serving
// guide gives its dedicated sampling backend (butteryoon "Gemma 4 MTP 서빙 가이드 해설",
// section 7 settings table).
#include "common.hpp"
#include "softmax_stats.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 63;
constexpr float kFixedScale = 274877906944.0f;   // 2^38
constexpr int kUniformBits = 24;
constexpr int kMaxE = 64;                        // elements per thread per chunk (V <= 4M)
constexpr long kChunkWGs = 2048;                 // chunk workgroups worth one round on the GPU

__device__ __forceinline__ uint64_t fixed_weight(float x) {
  const float s = x * kFixedScale;   // exact: power-of-two scaling
  return s > 0.f ? static_cast<uint64_t>(s) : 0ull;   // truncation == floor for s >= 0
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC'11): ten rounds of two 32 x 32 -> 64-bit products with the published multipliers, the
// new counter (hi(p2) ^ c1 ^ k0, lo(p2), hi(p0) ^ c3 ^ k1, lo(p0)), and the key bumped by the
// published Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p2 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p2 >> 32) ^ c[1] ^ k0, n1 = (uint32_t)p2;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1, n3 = (uint32_t)p0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
  }
}

// The verify step's u[b][i]: word i mod 4 of Philox4x32-10 at counter (i div 4, b, offset) and
// key seed, top 24 bits, as a multiple of 2^-24.
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t offset, int b, int i) {
  uint32_t c[4] = {(uint32_t)(i >> 2), (uint32_t)b, (uint32_t)offset, (uint32_t)(offset >> 32)};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint32_t w = (i & 3) == 0 ? c[0] : (i & 3) == 1 ? c[1] : (i & 3) == 2 ? c[2] : c[3];
  return (float)(w >> 8) * (1.0f / 16777216.0f);
}

// Where a kernel takes u[b][i] from: the caller's array, or the generator.
struct UniformSource {
  const float *u;          // [B, K1], or null: Philox with seed / offset
  uint64_t seed, offset;
  __device__ __forceinline__ float operator()(int b, int K1, int i) const {
    return u != nullptr ? u[(size_t)b * K1 + i] : philox_uniform(seed, offset, b, i);
  }
};

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
  const uint32_t lo = __shfl_up((uint32_t)v, d), hi = __shfl_up((uint32_t)(v >> 32), d);
  return ((uint64_t)hi << 32) | lo;
}

// Sum over the workgroup (integers: exact in any order); sh holds kThreads / 64 entries.
__device__ __forceinline__ uint64_t wg_sum(uint64_t v, uint64_t *sh) {
  const int lane = threadIdx.x & (spec::kWave - 1), wave = threadIdx.x / spec::kWave;
  v = spec::wave_sum(v);
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  uint64_t t = 0;
#pragma unroll
  for (int x = 0; x < kThreads / spec::kWave; ++x) t += sh[x];
  __syncthreads();
  return t;
}

// Inclusive prefix sum over the workgroup in thread order; sh holds kThreads / 64 entries.
__device__ __forceinline__ uint64_t wg_inclusive_scan(uint64_t v, uint64_t *sh) {
  const int lane = threadIdx.x & (spec::kWave - 1), wave = threadIdx.x / spec::kWave;
#pragma unroll
  for (int d = 1; d < spec::kWave; d <<= 1) {
    const uint64_t o = shfl_up_u64(v, d);
    if (lane >= d) v += o;
  }
  if (lane == spec::kWave - 1) sh[wave] = v;
  __syncthreads();
  uint64_t base = 0;
#pragma unroll
  for (int x = 0; x < kThreads / spec::kWave; ++x)
    if (x < wave) base += sh[x];
  __syncthreads();
  return v + base;
}

// E contiguous entries of a row starting at j0 (zero past V); a multiple of 4 is read as float4s.
template <int E>
__device__ __forceinline__ void load_run(const float *__restrict__ row, int j0, int V, float (&x)[E]) {
  if (E % 4 == 0 && j0 + E <= V && (V & 3) == 0) {
#pragma unroll
    for (int g = 0; g < E / 4; ++g) {
      const float4 t = *reinterpret_cast<const float4 *>(row + j0 + 4 * g);
      x[4 * g] = t.x; x[4 * g + 1] = t.y; x[4 * g + 2] = t.z; x[4 * g + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = j0 + e < V ? row[j0 + e] : 0.f;
  }
}

__device__ __forceinline__ uint64_t residual(uint64_t P, uint64_t Q) { return P > Q ? P - Q : 0ull; }

// Where the target's p comes from.
//  * normalised p [B * K1, V] (spec_accept): `stats` is null;
//  * the lm-head contraction's output (spec_lm_head_accept): `p` holds e = 2^((z - block max) c)
//    for the rows with T > 0, and p = e * 2^((block max - M) c) / L is formed here from the
//    block maxima and the row statistics with the same operations as the lm-head's softmax
//    finalize, so every p value equals the one spec_lm_head would have stored, bit for bit;
//    greedy rows (T <= 0) are the one-hot vector at the row's first argmax.
struct PSource {
  const float *p;
  const float2 *stats;           // [nblk][R] block (max, sum), or null
  const spec::RowStat *rows;     // [R] row statistics (lm_row_stats), or null
};

// The E entries j0 .. j0 + E - 1 of p's row `row` (E divides 256, so they share one block).
template <int E, bool FS>
__device__ __forceinline__ void p_run(const PSource &ps, int row, int R, int j0, int V,
                                      const spec::RowStat &rs, float (&x)[E]) {
  if constexpr (FS) {
    if (rs.c == 0.f) {                                   // greedy row: one-hot at A
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = (j0 + e == rs.a) ? 1.f : 0.f;
      return;
    }
    const int blk = min(j0, V - 1) / spec::kStatBlock;
    const float bm = ps.stats[(size_t)blk * R + row].x;
    load_run<E>(ps.p + (size_t)row * V, j0, V, x);
    const float f = spec::stat_factor(bm, rs);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] *= f;
  } else {
    load_run<E>(ps.p + (size_t)row * V, j0, V, x);
  }
}

// Row statistics of the K1 rows of sequence b into LDS (spec_lm_head_accept): lanes of wave 0.
// A barrier must follow before they are read.
__device__ __forceinline__ void seq_row_stats(const PSource &ps, int b, int K1,
                                              spec::RowStat *rs_sh) {
  if (threadIdx.x < K1) rs_sh[threadIdx.x] = ps.rows[(size_t)b * K1 + threadIdx.x];
}

// Grid: (nchunks, B).  Every workgroup finds n for its sequence (wave 0: lane i tests draft i
// exactly in fp64, a ballot gives the first rejection) and sums the integer weights of its
// chunk of the row the draw uses.  Round trips: drafts (and, from statistics, the rows'
// partials), then p and q at the drafts, then the chunk.
template <int E, bool FS>
__global__ __launch_bounds__(kThreads) void accept_chunks(
    const int32_t *__restrict__ draft, const float *__restrict__ q, PSource ps, UniformSource us,
    uint64_t *__restrict__ wsum, uint64_t *__restrict__ psum, int32_t *__restrict__ nbuf, int k,
    int V, int nchunks) {
  __shared__ uint64_t red[kThreads / spec::kWave];
  __shared__ int n_sh;
  __shared__ spec::RowStat rs_sh[FS ? kMaxK + 1 : 1];
  const int b = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int K1 = k + 1, R = (int)gridDim.y * K1;

  // drafts and uniforms (wave 0), p (or e and its block max) and q at the drafts
  int d = -1;
  float ul = 0.f, pe = 0.f, bm = 0.f;
  double qd = 0.0;
  if (tid < k) {
    d = draft[(size_t)b * k + tid];
    ul = us(b, K1, tid);
    if (d >= 0 && d < V) {
      qd = q[((size_t)b * k + tid) * V + d];
      pe = ps.p[((size_t)b * K1 + tid) * V + d];
      if constexpr (FS) bm = ps.stats[(size_t)(d / spec::kStatBlock) * R + (size_t)b * K1 + tid].x;
    }
  }
  if constexpr (FS) {
    seq_row_stats(ps, b, K1, rs_sh);
    __syncthreads();
  }
  if (tid < spec::kWave) {
    bool ok = false;
    if (tid < k && d >= 0 && d < V) {
      double pd = pe;
      if constexpr (FS) {
        const spec::RowStat rs = rs_sh[tid];
        pd = rs.c == 0.f ? (d == rs.a ? 1.0 : 0.0) : (double)(pe * spec::stat_factor(bm, rs));
      }
      ok = (double)ul * qd < pd;
    }
    const uint64_t acc = __ballot(ok);
    // lanes >= k never accept, so ~acc has a set bit at or below k
    if (tid == 0) n_sh = min(k, __builtin_ctzll(~acc));
  }
  __syncthreads();
  const int n = n_sh;
  const bool corr = n < k;
  const spec::RowStat rsn = FS ? rs_sh[FS ? n : 0] : spec::RowStat{0.f, 0.f, 0.f, 0};
  const int j0 = c * kThreads * E + tid * E;
  float pv[E], qv[E];
  p_run<E, FS>(ps, b * K1 + n, R, j0, V, rsn, pv);
  if (corr) load_run<E>(q + ((size_t)b * k + n) * V, j0, V, qv);
  uint64_t sp = 0, sw = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t P = fixed_weight(pv[e]);
    sp += P;
    if (corr) sw += residual(P, fixed_weight(qv[e]));
  }
  sp = wg_sum(sp, red);
  if (corr) sw = wg_sum(sw, red);
  if (tid == 0) {
    wsum[(size_t)b * nchunks + c] = corr ? sw : sp;
    psum[(size_t)b * nchunks + c] = sp;
    if (c == 0) nbuf[b] = n;
  }
}

// Grid: (B).  One workgroup per sequence scans the chunk sums, finds the chunk holding the
// threshold, scans inside it, and writes n and the tokens.  Round trips: n, the chunk sums, the
// uniform, the drafts (and, from statistics, the rows' partials) together; then the chosen
// chunk.
template <int E, bool FS>
__global__ __launch_bounds__(kThreads) void accept_draw(
    const int32_t *__restrict__ draft, const float *__restrict__ q, PSource ps, UniformSource us,
    const uint64_t *__restrict__ wsum, const uint64_t *__restrict__ psum,
    const int32_t *__restrict__ nbuf, int32_t *__restrict__ n_out, int32_t *__restrict__ tokens,
    float *__restrict__ u_out, int k, int V, int nchunks) {
  __shared__ uint64_t red[kThreads / spec::kWave];
  __shared__ int found_sh;
  __shared__ uint64_t base_sh;
  __shared__ spec::RowStat rs_sh[FS ? kMaxK + 1 : 1];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int K1 = k + 1, R = (int)gridDim.x * K1;
  if (tid == 0) found_sh = 0;   // ordered before the scans by the barriers inside wg_sum
  // everything independent of n at once (nchunks <= kThreads)
  const int n = nbuf[b];
  const uint64_t cw = tid < nchunks ? wsum[(size_t)b * nchunks + tid] : 0ull;
  const uint64_t cp = tid < nchunks ? psum[(size_t)b * nchunks + tid] : 0ull;
  const float uk = us(b, K1, k);
  if (u_out != nullptr && tid < K1) u_out[(size_t)b * K1 + tid] = us(b, K1, tid);
  const int dtok = tid < k ? draft[(size_t)b * k + tid] : -1;
  if constexpr (FS) seq_row_stats(ps, b, K1, rs_sh);   // the barriers of wg_sum follow

  const uint64_t wtot = wg_sum(cw, red);
  const bool corr = n < k;
  const bool fallback = corr && wtot == 0ull;   // every correction weight 0: draw from p
  const uint64_t mine = fallback ? cp : cw;
  const uint64_t total = fallback ? wg_sum(cp, red) : wtot;

  int y = 0;
  if (total > 0ull) {
    const float uf = uk * 16777216.0f;   // exact scaling by 2^24
    uint64_t m = uf > 0.f ? static_cast<uint64_t>(uf) : 0ull;
    if (m > (1ull << kUniformBits) - 1) m = (1ull << kUniformBits) - 1;
    const uint64_t t = (m * total) >> kUniformBits;   // m < 2^24, total < 2^40

    // 1) the chunk whose running sum first exceeds t (one chunk per thread)
    {
      const uint64_t incl = wg_inclusive_scan(mine, red), excl = incl - mine;
      if (excl <= t && t < incl) { found_sh = tid; base_sh = excl; }
    }
    __syncthreads();
    const int cstar = found_sh;
    const uint64_t t2 = t - base_sh;

    // 2) inside the chunk: running weights in index order, E contiguous elements per thread
    const bool wcorr = corr && !fallback;
    const int j0 = cstar * kThreads * E + tid * E;
    const spec::RowStat rsn = FS ? rs_sh[FS ? n : 0] : spec::RowStat{0.f, 0.f, 0.f, 0};
    float pv[E], qv[E];
    p_run<E, FS>(ps, b * K1 + n, R, j0, V, rsn, pv);
    if (wcorr) load_run<E>(q + ((size_t)b * k + n) * V, j0, V, qv);
    uint64_t w[E], wsum_t = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t P = fixed_weight(pv[e]);
      w[e] = wcorr ? residual(P, fixed_weight(qv[e])) : P;
      wsum_t += w[e];
    }
    {
      const uint64_t incl = wg_inclusive_scan(wsum_t, red), excl = incl - wsum_t;
      if (excl <= t2 && t2 < incl) {
        uint64_t run = excl;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (t2 < run + w[e]) { found_sh = j0 + e; break; }
          run += w[e];
        }
      }
    }
    __syncthreads();
    y = found_sh;
  }
  if (tid <= k) tokens[(size_t)b * K1 + tid] = tid < n ? dtok : (tid == n ? y : -1);
  if (tid == 0) n_out[b] = n;
}

struct AcceptPlan {
  int E, chunk, nchunks;
  size_t off_w, off_p, off_n, bytes;
};

AcceptPlan plan(int B, int V) {
  AcceptPlan pl;
  // chunk = 256 * E elements, E a power of two chosen so that a row has at most 256 chunks
  // (one chunk sum per thread of the draw kernel; V = 262144 gives 256 chunks of 1024), and
  // larger while the batch would need more than kChunkWGs workgroups (then every workgroup
  // streams more of its row instead of the grid running in several rounds).  The chunking
  // only groups exact integer sums, so it never changes a result.
  int E = 1;
  while (E < kMaxE && (long)kThreads * E * kThreads < V) E *= 2;
  while (E < kMaxE && (long)B * spec::ceil_div(V, kThreads * E) > kChunkWGs) E *= 2;
  pl.E = E;
  pl.chunk = kThreads * E;
  pl.nchunks = spec::ceil_div(V, pl.chunk);
  const size_t sums = (size_t)B * pl.nchunks * sizeof(uint64_t);
  pl.off_w = 0;
  pl.off_p = spec::align_up(sums, 256);
  pl.off_n = pl.off_p + spec::align_up(sums, 256);
  pl.bytes = pl.off_n + spec::align_up((size_t)B * sizeof(int32_t), 256);
  return pl;
}

template <int E, bool FS>
int launch(const AcceptPlan &pl, const int32_t *draft, const float *q, const PSource &ps,
           UniformSource us, float *u_out, int32_t *n_accepted, int32_t *tokens, int B, int k,
           int V, char *ws, hipStream_t st) {
  uint64_t *wsum = reinterpret_cast<uint64_t *>(ws + pl.off_w);
  uint64_t *psum = reinterpret_cast<uint64_t *>(ws + pl.off_p);
  int32_t *nbuf = reinterpret_cast<int32_t *>(ws + pl.off_n);
  hipLaunchKernelGGL((accept_chunks<E, FS>), dim3(pl.nchunks, B), dim3(kThreads), 0, st, draft,
                     q, ps, us, wsum, psum, nbuf, k, V, pl.nchunks);
  int rc = spec::launched("accept_chunks");
  if (rc != SPEC_OK) return rc;
  hipLaunchKernelGGL((accept_draw<E, FS>), dim3(B), dim3(kThreads), 0, st, draft, q, ps, us,
                     wsum, psum, nbuf, n_accepted, tokens, u_out, k, V, pl.nchunks);
  return spec::launched("accept_draw");
}

template <bool FS>
int launch_e(const AcceptPlan &pl, const int32_t *draft, const float *q, const PSource &ps,
             UniformSource us, float *u_out, int32_t *n_accepted, int32_t *tokens, int B, int k,
             int V, char *ws, hipStream_t st) {
  switch (pl.E) {
    case 1: return launch<1, FS>(pl, draft, q, ps, us, u_out, n_accepted, tokens, B, k, V, ws, st);
    case 2: return launch<2, FS>(pl, draft, q, ps, us, u_out, n_accepted, tokens, B, k, V, ws, st);
    case 4: return launch<4, FS>(pl, draft, q, ps, us, u_out, n_accepted, tokens, B, k, V, ws, st);
    case 8: return launch<8, FS>(pl, draft, q, ps, us, u_out, n_accepted, tokens, B, k, V, ws, st);
    case 16: return launch<16, FS>(pl, draft, q, ps, us, u_out, n_accepted, tokens, B, k, V, ws, st);
    case 32: return launch<32, FS>(pl, draft, q, ps, us, u_out, n_accepted, tokens, B, k, V, ws, st);
    default: return launch<64, FS>(pl, draft, q, ps, us, u_out, n_accepted, tokens, B, k, V, ws, st);
  }
}

int accept_check(const char *who, const int32_t *draft, const float *q, int32_t *n_accepted,
                 int32_t *tokens, int B, int k, int V) {
  SPEC_REQUIRE(B > 0 && V > 0 && k >= 0, SPEC_EINVAL, "%s: B=%d k=%d V=%d out of range", who, B,
               k, V);
  SPEC_REQUIRE(B <= 65535, SPEC_EUNSUPPORTED,
               "%s: B=%d sequences exceed 65535 (grid y of the accept kernel)", who, B);
  SPEC_REQUIRE(k <= kMaxK, SPEC_EUNSUPPORTED, "%s: k=%d exceeds %d (one wave per sequence)", who,
               k, kMaxK);
  SPEC_REQUIRE((long)V <= (long)kMaxE * kThreads * kThreads, SPEC_EUNSUPPORTED,
               "%s: V=%d exceeds %ld", who, V, (long)kMaxE * kThreads * kThreads);
  SPEC_REQUIRE(n_accepted && tokens && (k == 0 || (draft && q)), SPEC_EINVAL,
               "%s: null pointer argument", who);
  return SPEC_OK;
}

// Shared by spec_accept and spec_accept_philox: checks, workspace, launch.
int accept_run(const char *who, const int32_t *draft, const float *q, const float *p,
               UniformSource us, float *u_out, int32_t *n_accepted, int32_t *tokens, int B,
               int k, int V, void *workspace, size_t workspace_bytes, void *stream) {
  int rc = accept_check(who, draft, q, n_accepted, tokens, B, k, V);
  if (rc != SPEC_OK) return rc;
  SPEC_REQUIRE(p != nullptr, SPEC_EINVAL, "%s: null pointer argument", who);
  const AcceptPlan pl = plan(B, V);
  SPEC_REQUIRE(workspace != nullptr && workspace_bytes >= pl.bytes, SPEC_EWORKSPACE,
               "%s: workspace of %zu bytes needed, %zu given", who, pl.bytes, workspace_bytes);
  const PSource ps{p, nullptr, nullptr};
  return launch_e<false>(pl, draft, q, ps, us, u_out, n_accepted, tokens, B, k, V,
                         static_cast<char *>(workspace), static_cast<hipStream_t>(stream));
}

// Workspace of spec_lm_head_accept: the contraction's output e [R, V], its block and row
// statistics, the accept step's chunk sums.
struct FusedPlan {
  spec::LmLayout lm;
  AcceptPlan acc;
  size_t off_e, off_lm, off_acc, bytes;
};

FusedPlan fused_plan(int B, int k, int V) {
  FusedPlan f;
  const int R = B * (k + 1);
  f.lm = spec::lm_layout(R, V);
  f.acc = plan(B, V);
  f.off_e = 0;
  f.off_lm = spec::align_up((size_t)R * V * sizeof(float), 256);
  f.off_acc = f.off_lm + spec::align_up(f.lm.bytes, 256);
  f.bytes = f.off_acc + f.acc.bytes;
  return f;
}

}  // namespace

extern "C" size_t spec_accept_workspace(int B, int k, int V) {
  if (B <= 0 || V <= 0 || k < 0) {
    spec::fail(SPEC_EINVAL, "spec_accept_workspace: B=%d k=%d V=%d out of range", B, k, V);
    return 0;
  }
  return plan(B, V).bytes;
}

extern "C" int spec_accept(const int32_t *draft, const float *q, const float *p,
                           const float *uniforms, int32_t *n_accepted, int32_t *tokens, int B,
                           int k, int V, void *workspace, size_t workspace_bytes, void *stream) {
  spec::clear_error();
  SPEC_REQUIRE(uniforms != nullptr, SPEC_EINVAL, "spec_accept: null pointer argument");
  return accept_run("spec_accept", draft, q, p, UniformSource{uniforms, 0, 0}, nullptr,
                    n_accepted, tokens, B, k, V, workspace, workspace_bytes, stream);
}

extern "C" int spec_accept_philox(const int32_t *draft, const float *q, const float *p,
                                  uint64_t seed, uint64_t offset, float *uniforms_out,
                                  int32_t *n_accepted, int32_t *tokens, int B, int k, int V,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  spec::clear_error();
  return accept_run("spec_accept_philox", draft, q, p, UniformSource{nullptr, seed, offset},
                    uniforms_out, n_accepted, tokens, B, k, V, workspace, workspace_bytes,
                    stream);
}

extern "C" size_t spec_lm_head_accept_workspace(int B, int k, int H, int V) {
  spec::clear_error();
  if (B <= 0 || k < 0 || H <= 0 || V <= 0 || k > kMaxK) {
    spec::fail(SPEC_EINVAL, "spec_lm_head_accept_workspace: B=%d k=%d H=%d V=%d out of range",
               B, k, H, V);
    return 0;
  }
  return fused_plan(B, k, V).bytes;
}

extern "C" int spec_lm_head_accept(const void *hidden, const void *weight,
                                   const float *temperature, const int32_t *draft,
                                   const float *q, const float *uniforms, uint64_t seed,
                                   uint64_t offset, float *uniforms_out, int32_t *n_accepted,
                                   int32_t *tokens, int B, int k, int H, int V, spec_dtype dtype,
                                   void *workspace, size_t workspace_bytes, void *stream) {
  spec::clear_error();
  const char *who = "spec_lm_head_accept";
  int rc = accept_check(who, draft, q, n_accepted, tokens, B, k, V);
  if (rc != SPEC_OK) return rc;
  SPEC_REQUIRE((long)B * (k + 1) <= 65535, SPEC_EUNSUPPORTED,
               "%s: B*(k+1)=%ld rows exceed 65535", who, (long)B * (k + 1));
  const int R = B * (k + 1);
  const FusedPlan f = fused_plan(B, k, V);
  SPEC_REQUIRE(workspace != nullptr && workspace_bytes >= f.bytes, SPEC_EWORKSPACE,
               "%s: workspace of %zu bytes needed, %zu given", who, f.bytes, workspace_bytes);
  char *ws = static_cast<char *>(workspace);
  float *e = reinterpret_cast<float *>(ws + f.off_e);
  rc = spec::lm_head_check(hidden, weight, temperature, e, nullptr, R, H, V, dtype, who);
  if (rc != SPEC_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const spec::StatsOut so = spec::lm_stats_out(f.lm, ws + f.off_lm);
  spec::RowStat *rows = reinterpret_cast<spec::RowStat *>(ws + f.off_lm + f.lm.off_rows);
  rc = spec::lm_head_contract(hidden, weight, temperature, nullptr, e, so, R, H, V, dtype, st);
  if (rc != SPEC_OK) return rc;
  rc = spec::lm_row_stats_launch(so, temperature, rows, R, st);
  if (rc != SPEC_OK) return rc;
  const PSource ps{e, so.stats, rows};
  const UniformSource us{uniforms, seed, offset};
  return launch_e<true>(f.acc, draft, q, ps, us, uniforms_out, n_accepted, tokens, B, k, V,
                        ws + f.off_acc, st);
}
