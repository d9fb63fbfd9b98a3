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

__device__ __forceinline__ uint64_t fixed_weight(float x) {
  const float s = x * kFixedScale;   // exact: power-of-two scaling
  return s > 0.f ? static_cast<uint64_t>(s) : 0ull;   // truncation == floor for s >= 0
}

// Number of accepted drafts of sequence b.  Must be called by a whole wave (lanes 0..63).
__device__ int accepted_count(const int32_t *__restrict__ draft, const float *__restrict__ q,
                              const float *__restrict__ p, const float *__restrict__ u,
                              int b, int k, int V, int lane) {
  bool ok = false;
  if (lane < k) {
    const int d = draft[(size_t)b * k + lane];
    if (d >= 0 && d < V) {
      const double qd = q[((size_t)b * k + lane) * V + d];
      const double pd = p[((size_t)b * (k + 1) + lane) * V + d];
      const double ud = u[(size_t)b * (k + 1) + lane];
      ok = ud * qd < pd;
    }
  }
  const uint64_t acc = __ballot(ok);
  // lanes >= k never accept, so ~acc has a set bit at or below k
  return min(k, __builtin_ctzll(~acc));
}

template <typename U>
__device__ U block_sum(U v, U *sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) sh[tid] += sh[tid + s];
    __syncthreads();
  }
  const U r = sh[0];
  __syncthreads();
  return r;
}

// In-place inclusive scan of sh[0..kThreads) (uint64), Hillis-Steele.
__device__ void block_inclusive_scan(uint64_t *sh) {
  const int tid = threadIdx.x;
  for (int off = 1; off < kThreads; off <<= 1) {
    const uint64_t add = tid >= off ? sh[tid - off] : 0ull;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void accept_chunks(
    const int32_t *__restrict__ draft, const float *__restrict__ q, const float *__restrict__ p,
    const float *__restrict__ u, uint64_t *__restrict__ wsum, uint64_t *__restrict__ psum,
    int32_t *__restrict__ nbuf, int k, int V, int chunk, int nchunks) {
  __shared__ int n_sh;
  __shared__ uint64_t red[kThreads];
  const int b = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  if (tid < spec::kWave) {
    const int n = accepted_count(draft, q, p, u, b, k, V, tid);
    if (tid == 0) n_sh = n;
  }
  __syncthreads();
  const int n = n_sh;
  const float *prow = p + ((size_t)b * (k + 1) + n) * V;
  const float *qrow = n < k ? q + ((size_t)b * k + n) * V : nullptr;
  const int lo = c * chunk, hi = min(V, lo + chunk);
  uint64_t sw = 0, sp = 0;
  for (int j = lo + tid; j < hi; j += kThreads) {
    const uint64_t P = fixed_weight(prow[j]);
    sp += P;
    if (qrow) {
      const uint64_t Q = fixed_weight(qrow[j]);
      sw += P > Q ? P - Q : 0ull;
    }
  }
  sp = block_sum(sp, red);
  if (qrow) sw = block_sum(sw, red);
  if (tid == 0) {
    wsum[(size_t)b * nchunks + c] = qrow ? sw : sp;
    psum[(size_t)b * nchunks + c] = sp;
    if (c == 0) nbuf[b] = n;
  }
}

__global__ __launch_bounds__(kThreads) void accept_draw(
    const int32_t *__restrict__ draft, const float *__restrict__ q, const float *__restrict__ p,
    const float *__restrict__ u, const uint64_t *__restrict__ wsum,
    const uint64_t *__restrict__ psum, const int32_t *__restrict__ nbuf,
    int32_t *__restrict__ n_out, int32_t *__restrict__ tokens, int k, int V, int chunk,
    int nchunks) {
  __shared__ uint64_t sh[kThreads];
  __shared__ int found_sh;
  __shared__ uint64_t base_sh;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n = nbuf[b];
  const int K1 = k + 1;

  // chunk sums; the correction weights fall back to p's when they are all zero
  const uint64_t *cs = wsum + (size_t)b * nchunks;
  const int per = (nchunks + kThreads - 1) / kThreads;   // chunks per thread (contiguous)
  uint64_t mine = 0;
  for (int e = 0; e < per; ++e) {
    const int c = tid * per + e;
    if (c < nchunks) mine += cs[c];
  }
  const uint64_t wtot = block_sum(mine, sh);
  const bool fallback = n < k && wtot == 0ull;
  if (fallback) {
    cs = psum + (size_t)b * nchunks;
    mine = 0;
    for (int e = 0; e < per; ++e) {
      const int c = tid * per + e;
      if (c < nchunks) mine += cs[c];
    }
  }
  const uint64_t total = fallback ? block_sum(mine, sh) : wtot;

  int y = 0;
  if (total > 0ull) {
    const float uk = u[(size_t)b * K1 + k];
    const float uf = uk * 16777216.0f;   // exact scaling by 2^24
    uint64_t m = uf > 0.f ? static_cast<uint64_t>(uf) : 0ull;
    if (m > (1ull << kUniformBits) - 1) m = (1ull << kUniformBits) - 1;
    const uint64_t t = (m * total) >> kUniformBits;   // m < 2^24, total < 2^40

    // 1) the chunk whose running sum first exceeds t
    sh[tid] = mine;
    __syncthreads();
    block_inclusive_scan(sh);
    if (tid == 0) found_sh = -1;
    __syncthreads();
    {
      const uint64_t incl = sh[tid], excl = incl - mine;
      if (excl <= t && t < incl) {   // exactly one thread owns t
        uint64_t run = excl;
        for (int e = 0; e < per; ++e) {
          const int c = tid * per + e;
          if (c >= nchunks) break;
          if (t < run + cs[c]) { found_sh = c; base_sh = run; break; }
          run += cs[c];
        }
      }
    }
    __syncthreads();
    const int cstar = found_sh;
    const uint64_t t2 = t - base_sh;

    // 2) inside the chunk: running weights in index order
    const float *prow = p + ((size_t)b * K1 + n) * V;
    const float *qrow = (n < k && !fallback) ? q + ((size_t)b * k + n) * V : nullptr;
    const int lo = cstar * chunk, hi = min(V, lo + chunk);
    const int epl = (chunk + kThreads - 1) / kThreads;   // elements per thread (contiguous)
    const int j0 = lo + tid * epl;
    uint64_t wsum_t = 0;
    for (int e = 0; e < epl; ++e) {
      const int j = j0 + e;
      if (j >= hi) break;
      const uint64_t P = fixed_weight(prow[j]);
      uint64_t w = P;
      if (qrow) { const uint64_t Q = fixed_weight(qrow[j]); w = P > Q ? P - Q : 0ull; }
      wsum_t += w;
    }
    sh[tid] = wsum_t;
    __syncthreads();
    block_inclusive_scan(sh);
    if (tid == 0) found_sh = -1;
    __syncthreads();
    {
      const uint64_t incl = sh[tid], excl = incl - wsum_t;
      if (excl <= t2 && t2 < incl) {
        uint64_t run = excl;
        for (int e = 0; e < epl; ++e) {
          const int j = j0 + e;
          if (j >= hi) break;
          const uint64_t P = fixed_weight(prow[j]);
          uint64_t w = P;
          if (qrow) { const uint64_t Q = fixed_weight(qrow[j]); w = P > Q ? P - Q : 0ull; }
          if (t2 < run + w) { found_sh = j; break; }
          run += w;
        }
      }
    }
    __syncthreads();
    y = found_sh;
  }
  if (tid <= k) {
    int tok = -1;
    if (tid < n) tok = draft[(size_t)b * k + tid];
    else if (tid == n) tok = y;
    tokens[(size_t)b * K1 + tid] = tok;
  }
  if (tid == 0) n_out[b] = n;
}

struct AcceptPlan {
  int chunk, nchunks;
  size_t off_w, off_p, off_n, bytes;
};

AcceptPlan plan(int B, int V) {
  AcceptPlan pl;
  // chunk = 256 * E elements; at most 256 chunks per sequence (256 * 256 elements or fewer
  // per thread pass); V = 262144 gives 256 chunks of 1024.
  const int E = max(1, spec::ceil_div(V, kThreads * 256));
  pl.chunk = kThreads * E;
  pl.nchunks = spec::ceil_div(V, pl.chunk);
  const size_t sums = (size_t)B * pl.nchunks * sizeof(uint64_t);
  pl.off_w = 0;
  pl.off_p = spec::align_up(sums, 256);
  pl.off_n = pl.off_p + spec::align_up(sums, 256);
  pl.bytes = pl.off_n + spec::align_up((size_t)B * sizeof(int32_t), 256);
  return pl;
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
  SPEC_REQUIRE(B > 0 && V > 0 && k >= 0, SPEC_EINVAL,
               "spec_accept: B=%d k=%d V=%d out of range", B, k, V);
  SPEC_REQUIRE(k <= kMaxK, SPEC_EUNSUPPORTED, "spec_accept: k=%d exceeds %d (one wave per sequence)",
               k, kMaxK);
  SPEC_REQUIRE(p && uniforms && n_accepted && tokens && (k == 0 || (draft && q)), SPEC_EINVAL,
               "spec_accept: null pointer argument");
  const AcceptPlan pl = plan(B, V);
  SPEC_REQUIRE(workspace != nullptr && workspace_bytes >= pl.bytes, SPEC_EWORKSPACE,
               "spec_accept: workspace of %zu bytes needed, %zu given", pl.bytes, workspace_bytes);
  char *ws = static_cast<char *>(workspace);
  uint64_t *wsum = reinterpret_cast<uint64_t *>(ws + pl.off_w);
  uint64_t *psum = reinterpret_cast<uint64_t *>(ws + pl.off_p);
  int32_t *nbuf = reinterpret_cast<int32_t *>(ws + pl.off_n);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(accept_chunks, dim3(pl.nchunks, B), dim3(kThreads), 0, st, draft, q, p,
                     uniforms, wsum, psum, nbuf, k, V, pl.chunk, pl.nchunks);
  int rc = spec::launched("accept_chunks");
  if (rc != SPEC_OK) return rc;
  hipLaunchKernelGGL(accept_draw, dim3(B), dim3(kThreads), 0, st, draft, q, p, uniforms, wsum,
                     psum, nbuf, n_accepted, tokens, k, V, pl.chunk, pl.nchunks);
  return spec::launched("accept_draw");
}
