// Accept / reject of the drafts and the correction or bonus draw.
//
// The pages: the target confirms the drafts up to the first one it rejects and generates the
// token at that position itself, keeping the output distribution that of the target alone
// (llm-wiki "Gemma 4 MTP: 드래프터가 초안을 쓰고 타깃이 검증하는 추론 가속 구조", section
// "투기적 디코딩의 기본 구조"; butteryoon "Gemma 4 MTP 서빙 가이드 해설", section 4 accept/reject
// step); when every draft is accepted the same forward also yields one extra token (news.hada.io
// 29214, section "MTP가 동작하는 방식").  The rule is Leviathan et al.'s: accept draft i iff
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
#include "common.hpp"

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

// Number of accepted drafts of sequence b.  Must be called by a whole wave (lanes 0..63).
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

// ul: this lane's uniform (lane i < k tests draft i).
__device__ int accepted_count(const int32_t *__restrict__ draft, const float *__restrict__ q,
                              const float *__restrict__ p, float ul, int b, int k, int V,
                              int lane) {
  bool ok = false;
  if (lane < k) {
    const int d = draft[(size_t)b * k + lane];
    if (d >= 0 && d < V) {
      const double qd = q[((size_t)b * k + lane) * V + d];
      const double pd = p[((size_t)b * (k + 1) + lane) * V + d];
      ok = (double)ul * qd < pd;
    }
  }
  const uint64_t acc = __ballot(ok);
  // lanes >= k never accept, so ~acc has a set bit at or below k
  return min(k, __builtin_ctzll(~acc));
}

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

// Chunk c of a sequence's row: elements [c * chunk, (c + 1) * chunk), chunk = kThreads * E;
// thread t owns the E contiguous elements starting at c * chunk + t * E (E is 4 for one
// sequence over a 256k vocabulary, larger for big batches; a multiple of 4 is read as float4s).
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

// Grid: (nchunks, B).  Round trips: drafts, then p/q at the drafts (n), then the chunk of the
// row the draw uses.  (Loading every row's chunk with the drafts, to pick row n from registers,
// measured slower at batch 1: the extra bytes cost more than the round trip.)
template <int E>
__global__ __launch_bounds__(kThreads) void accept_chunks(
    const int32_t *__restrict__ draft, const float *__restrict__ q, const float *__restrict__ p,
    UniformSource us, uint64_t *__restrict__ wsum, uint64_t *__restrict__ psum,
    int32_t *__restrict__ nbuf, int k, int V, int nchunks) {
  __shared__ int n_sh;
  __shared__ uint64_t red[kThreads / spec::kWave];
  const int b = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int K1 = k + 1;
  if (tid < spec::kWave) {
    const float ul = tid < k ? us(b, K1, tid) : 0.f;
    const int n = accepted_count(draft, q, p, ul, b, k, V, tid);
    if (tid == 0) n_sh = n;
  }
  __syncthreads();
  const int n = n_sh;
  const int j0 = c * kThreads * E + tid * E;
  float pv[E], qv[E];
  load_run<E>(p + ((size_t)b * K1 + n) * V, j0, V, pv);
  const bool corr = n < k;
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

// Grid: (B).  Round trips: n, chunk sums, uniform and drafts together; then the chosen chunk.
template <int E>
__global__ __launch_bounds__(kThreads) void accept_draw(
    const int32_t *__restrict__ draft, const float *__restrict__ q, const float *__restrict__ p,
    UniformSource us, const uint64_t *__restrict__ wsum,
    const uint64_t *__restrict__ psum, const int32_t *__restrict__ nbuf,
    int32_t *__restrict__ n_out, int32_t *__restrict__ tokens, float *__restrict__ u_out, int k,
    int V, int nchunks) {
  __shared__ uint64_t red[kThreads / spec::kWave];
  __shared__ int found_sh;
  __shared__ uint64_t base_sh;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int K1 = k + 1;
  if (tid == 0) found_sh = 0;   // ordered before the scans by the barriers inside wg_sum
  // everything independent of n at once (nchunks <= kThreads)
  const int n = nbuf[b];
  const uint64_t cw = tid < nchunks ? wsum[(size_t)b * nchunks + tid] : 0ull;
  const uint64_t cp = tid < nchunks ? psum[(size_t)b * nchunks + tid] : 0ull;
  const float uk = us(b, K1, k);
  if (u_out != nullptr && tid < K1) u_out[(size_t)b * K1 + tid] = us(b, K1, tid);
  const int dtok = tid < k ? draft[(size_t)b * k + tid] : -1;

  const uint64_t wtot = wg_sum(cw, red);
  const bool fallback = n < k && wtot == 0ull;   // every correction weight 0: draw from p
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
    const bool corr = n < k && !fallback;
    const int j0 = cstar * kThreads * E + tid * E;
    float pv[E], qv[E];
    load_run<E>(p + ((size_t)b * K1 + n) * V, j0, V, pv);
    if (corr) load_run<E>(q + ((size_t)b * k + n) * V, j0, V, qv);
    uint64_t w[E], wsum_t = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t P = fixed_weight(pv[e]);
      w[e] = corr ? residual(P, fixed_weight(qv[e])) : P;
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

template <int E>
int launch(const AcceptPlan &pl, const int32_t *draft, const float *q, const float *p,
           UniformSource us, float *u_out, int32_t *n_accepted, int32_t *tokens, int B, int k,
           int V, uint64_t *wsum, uint64_t *psum, int32_t *nbuf, hipStream_t st) {
  hipLaunchKernelGGL((accept_chunks<E>), dim3(pl.nchunks, B), dim3(kThreads), 0, st, draft, q,
                     p, us, wsum, psum, nbuf, k, V, pl.nchunks);
  int rc = spec::launched("accept_chunks");
  if (rc != SPEC_OK) return rc;
  hipLaunchKernelGGL((accept_draw<E>), dim3(B), dim3(kThreads), 0, st, draft, q, p, us,
                     wsum, psum, nbuf, n_accepted, tokens, u_out, k, V, pl.nchunks);
  return spec::launched("accept_draw");
}

// Shared by spec_accept and spec_accept_philox: checks, workspace, launch.
int accept_run(const char *who, const int32_t *draft, const float *q, const float *p,
               UniformSource us, float *u_out, int32_t *n_accepted, int32_t *tokens, int B,
               int k, int V, void *workspace, size_t workspace_bytes, void *stream) {
  SPEC_REQUIRE(B > 0 && V > 0 && k >= 0, SPEC_EINVAL, "%s: B=%d k=%d V=%d out of range", who, B,
               k, V);
  SPEC_REQUIRE(B <= 65535, SPEC_EUNSUPPORTED,
               "%s: B=%d sequences exceed 65535 (grid y of the chunk kernel)", who, B);
  SPEC_REQUIRE(k <= kMaxK, SPEC_EUNSUPPORTED, "%s: k=%d exceeds %d (one wave per sequence)", who,
               k, kMaxK);
  SPEC_REQUIRE((long)V <= (long)kMaxE * kThreads * kThreads, SPEC_EUNSUPPORTED,
               "%s: V=%d exceeds %ld", who, V, (long)kMaxE * kThreads * kThreads);
  SPEC_REQUIRE(p && n_accepted && tokens && (k == 0 || (draft && q)), SPEC_EINVAL,
               "%s: null pointer argument", who);
  const AcceptPlan pl = plan(B, V);
  SPEC_REQUIRE(workspace != nullptr && workspace_bytes >= pl.bytes, SPEC_EWORKSPACE,
               "%s: workspace of %zu bytes needed, %zu given", who, pl.bytes, workspace_bytes);
  char *ws = static_cast<char *>(workspace);
  uint64_t *wsum = reinterpret_cast<uint64_t *>(ws + pl.off_w);
  uint64_t *psum = reinterpret_cast<uint64_t *>(ws + pl.off_p);
  int32_t *nbuf = reinterpret_cast<int32_t *>(ws + pl.off_n);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (pl.E) {
    case 1: return launch<1>(pl, draft, q, p, us, u_out, n_accepted, tokens, B, k, V, wsum, psum, nbuf, st);
    case 2: return launch<2>(pl, draft, q, p, us, u_out, n_accepted, tokens, B, k, V, wsum, psum, nbuf, st);
    case 4: return launch<4>(pl, draft, q, p, us, u_out, n_accepted, tokens, B, k, V, wsum, psum, nbuf, st);
    case 8: return launch<8>(pl, draft, q, p, us, u_out, n_accepted, tokens, B, k, V, wsum, psum, nbuf, st);
    case 16: return launch<16>(pl, draft, q, p, us, u_out, n_accepted, tokens, B, k, V, wsum, psum, nbuf, st);
    case 32: return launch<32>(pl, draft, q, p, us, u_out, n_accepted, tokens, B, k, V, wsum, psum, nbuf, st);
    default: return launch<64>(pl, draft, q, p, us, u_out, n_accepted, tokens, B, k, V, wsum, psum, nbuf, st);
  }
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
