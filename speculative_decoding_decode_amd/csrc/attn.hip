// Verify attention: K1 = k + 1 causal queries per sequence against a paged KV cache.
//
// The target checks all k drafts (and the bonus position) in one forward (llm-wiki "Gemma 4
// MTP: 드래프터가 초안을 쓰고 타깃이 검증하는 추론 가속 구조", section "투기적 디코딩의 기본
// 구조"); the cache it reads is the pool it shares with the drafter (butteryoon "Gemma 4 MTP 서빙
// 가이드 해설", section 1 table, KV-cache row).  Its layers mix sliding-window heads of dim 256
// and global heads of dim 512 (same guide, section 7 settings table).  Query i of sequence b
// sits at position t = ctx_b - K1 + i and sees keys s in [lo, t], lo = 0 (global) or
// t - window + 1 (sliding), clipped at 0.
//
// Design (gfx950): the visible page range of a sequence is split across workgroups
// ("split-K" over the context).  A workgroup owns one (sequence, KV head, split, chunk of up
// to 32 query rows) and walks its pages: each 16-token page of K and of V is one contiguous
// 16*D block per head, read with coalesced 16-byte loads into LDS; 16 lanes score one query
// row against the 16 keys and keep the running max / sum with wavefront shuffles (online
// softmax); the value update then runs one output column per thread.  The workgroup writes
// (max, sum, unnormalised output) and a second kernel merges the splits with log-sum-exp
// weights.  All exponentials are base 2 with log2(e) folded into the query scale.
#include <math.h>

#include "common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kPage = 16;
constexpr int kRows = 32;            // query rows per workgroup
constexpr int kTargetWGs = 4096;     // splits are sized so the grid reaches about this many
constexpr int kMinPagesPerSplit = 1;
constexpr int kMaxPagesPerSplit = 256;   // page ids of a split are staged in LDS
constexpr int kMaxSplits = 4096;
constexpr float kLog2e = 1.4426950408889634f;

struct Span {
  int ctx, p0, np;   // clamped context, first page, pages holding visible keys
};

__device__ __host__ inline Span seq_span(int ctx, int K1, int window, int max_pages) {
  Span s;
  ctx = ctx < 0 ? 0 : ctx;
  ctx = ctx > max_pages * kPage ? max_pages * kPage : ctx;
  s.ctx = ctx;
  if (ctx == 0) { s.p0 = 0; s.np = 0; return s; }
  int lo = window > 0 ? ctx - K1 - window + 1 : 0;
  lo = lo < 0 ? 0 : lo;
  s.p0 = lo / kPage;
  s.np = (ctx - 1) / kPage - s.p0 + 1;
  return s;
}

template <int D, typename T>
struct AttnShape {
  static constexpr int kEPG = 16 / (int)sizeof(T);       // elements per 16-byte group
  static constexpr int kGPR = D / kEPG;                  // 16-byte groups per row
  static constexpr int kKStr = D + kEPG;                 // LDS row stride of K/V tiles
  static constexpr int kTileG = kPage * kGPR;            // 16-byte groups per K (or V) page tile
  static constexpr int kGPT = (kTileG + kThreads - 1) / kThreads;   // per thread
  static constexpr int kQPT = (kRows * kGPR + kThreads - 1) / kThreads;
  static constexpr int kCPT = D >= 256 ? D / 256 : 1;    // output columns per thread
  static constexpr int kNCol = D / kCPT;                 // threads covering one row's columns
  static constexpr int kRG = kThreads / kNCol;           // row groups
  static constexpr int kRPT = kRows / kRG;               // rows per thread
  static constexpr size_t kLds = (size_t)kRows * D * 4 + 2ull * kPage * kKStr * sizeof(T) +
                                 (size_t)kRows * kPage * 4;
};

// Grid: (nsplit, Hkv * nrowchunk, B).
// Memory round trips before the first page is in LDS: the split's page ids (issued first),
// then the queries and the first page's K/V together; while a page is being scored the next
// page's K/V are already in flight in registers.
template <int D, typename T>
__global__ __launch_bounds__(kThreads) void attn_partial(
    const T *__restrict__ q, const T *__restrict__ kpool, const T *__restrict__ vpool,
    const int32_t *__restrict__ table, const int32_t *__restrict__ ctx_lens,
    float2 *__restrict__ part_ml, float *__restrict__ part_acc, int K1, int Hq, int Hkv,
    int num_pages, int max_pages, int window, float qscale, int pps, int nsplit, int GK1) {
  using S = AttnShape<D, T>;
  extern __shared__ __align__(16) unsigned char smem[];
  float *qs = reinterpret_cast<float *>(smem);                     // [kRows][D]
  T *ks = reinterpret_cast<T *>(qs + kRows * D);                   // [16][kKStr]
  T *vs = ks + kPage * S::kKStr;                                   // [16][kKStr]
  float *ss = reinterpret_cast<float *>(vs + kPage * S::kKStr);    // [kRows][16]
  __shared__ float m_sh[kRows], l_sh[kRows], alpha_sh[kRows];
  __shared__ int tq_sh[kRows];
  __shared__ int pid_sh[kMaxPagesPerSplit];

  const int tid = threadIdx.x;
  const int b = blockIdx.z, g = blockIdx.y % Hkv, rc = blockIdx.y / Hkv, s = blockIdx.x;
  const int G = Hq / Hkv;
  const Span sp = seq_span(ctx_lens[b], K1, window, max_pages);
  const int ns = (sp.np + pps - 1) / pps;
  if (s >= ns) return;
  const int pg_begin = sp.p0 + s * pps;
  const int npg = min(sp.p0 + sp.np, pg_begin + pps) - pg_begin;
  const int rr0 = rc * kRows;
  const int nr = min(kRows, GK1 - rr0);

  // (1) page ids of the split, then the queries (registers).  Loads are unconditional with
  // clamped indices so the wait counts the compiler inserts stay exact.
  const int pid_reg = table[(size_t)b * max_pages + pg_begin + min(tid, npg - 1)];
  uint4 qraw[S::kQPT];
#pragma unroll
  for (int x = 0; x < S::kQPT; ++x) {
    const int e = min(tid + x * kThreads, nr * S::kGPR - 1);
    const int r = e / S::kGPR, gi = e - r * S::kGPR;
    const int rr = rr0 + r, i = rr / G, h = g * G + (rr - i * G);
    qraw[x] = *reinterpret_cast<const uint4 *>(q + (((size_t)b * K1 + i) * Hq + h) * D + gi * S::kEPG);
  }
  if (tid < npg) pid_sh[tid] = (pid_reg >= 0 && pid_reg < num_pages) ? pid_reg : -1;
  if (tid < kRows) {
    m_sh[tid] = -INFINITY;
    l_sh[tid] = 0.f;
    tq_sh[tid] = tid < nr ? sp.ctx - K1 + (rr0 + tid) / G : -1;
  }
  __syncthreads();

  // (2) K/V of page 0 in flight while the queries land in LDS
  uint4 kcur[S::kGPT], vcur[S::kGPT], knxt[S::kGPT], vnxt[S::kGPT];
  auto fetch = [&](uint4(&kr)[S::kGPT], uint4(&vr)[S::kGPT], int i) {
    const int pid = pid_sh[i];
    const T *kb = kpool + ((size_t)(pid < 0 ? 0 : pid) * Hkv + g) * kPage * D;
    const T *vb = vpool + ((size_t)(pid < 0 ? 0 : pid) * Hkv + g) * kPage * D;
#pragma unroll
    for (int x = 0; x < S::kGPT; ++x) {
      const int e = tid + x * kThreads;
      const bool ok = pid >= 0 && e < S::kTileG;
      kr[x] = ok ? *reinterpret_cast<const uint4 *>(kb + e * S::kEPG) : uint4{0u, 0u, 0u, 0u};
      vr[x] = ok ? *reinterpret_cast<const uint4 *>(vb + e * S::kEPG) : uint4{0u, 0u, 0u, 0u};
    }
  };
  fetch(kcur, vcur, 0);
#pragma unroll
  for (int x = 0; x < S::kQPT; ++x) {
    const int e = tid + x * kThreads;
    if (e < nr * S::kGPR) {
      float f[S::kEPG];
      spec::unpack16(qraw[x], f, T{});
#pragma unroll
      for (int y = 0; y < S::kEPG; ++y) qs[e * S::kEPG + y] = f[y] * qscale;   // row-major [r][D]
    }
  }

  float acc[S::kRPT][S::kCPT];
#pragma unroll
  for (int ri = 0; ri < S::kRPT; ++ri)
#pragma unroll
    for (int c = 0; c < S::kCPT; ++c) acc[ri][c] = 0.f;
  const int rg = tid / S::kNCol, col0 = tid - rg * S::kNCol;

  for (int i = 0; i < npg; ++i) {
#pragma unroll
    for (int x = 0; x < S::kGPT; ++x) {
      const int e = tid + x * kThreads;
      if (e < S::kTileG) {
        const int row = e / S::kGPR, gi = e - row * S::kGPR;
        *reinterpret_cast<uint4 *>(ks + row * S::kKStr + gi * S::kEPG) = kcur[x];
        *reinterpret_cast<uint4 *>(vs + row * S::kKStr + gi * S::kEPG) = vcur[x];
      }
    }
    if (i + 1 < npg) fetch(knxt, vnxt, i + 1);
    const bool page_ok = pid_sh[i] >= 0;   // uniform
    const int pg = pg_begin + i;
    __syncthreads();

    // scores and online-softmax state: 16 consecutive lanes = one query row x 16 keys
    for (int base = 0; base < nr * kPage; base += kThreads) {
      const int idx = base + tid, rr = idx >> 4, j = idx & 15;
      const bool rowok = rr < nr;
      float sc = -INFINITY;
      if (rowok && page_ok) {
        const int pos = pg * kPage + j, t = tq_sh[rr];
        if (pos <= t && (window == 0 || t - pos < window)) {
          const T *kr = ks + j * S::kKStr;
          const float *qr = qs + rr * D;
          float dot = 0.f;
#pragma unroll 4
          for (int d0 = 0; d0 < D; d0 += S::kEPG) {
            float kf[S::kEPG];
            spec::unpack16(*reinterpret_cast<const uint4 *>(kr + d0), kf, T{});
#pragma unroll
            for (int x = 0; x < S::kEPG; ++x) dot = fmaf(qr[d0 + x], kf[x], dot);
          }
          sc = dot;
        }
      }
      float mx = sc;
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
      const float m_old = rowok ? m_sh[rr] : -INFINITY;
      const float m_new = fmaxf(m_old, mx);
      const float pj = sc == -INFINITY ? 0.f : exp2f(sc - m_new);
      float sum = pj;
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 16);
      if (rowok) {
        ss[rr * kPage + j] = pj;
        if (j == 0) {
          const float alpha = m_old == -INFINITY ? 0.f : exp2f(m_old - m_new);
          l_sh[rr] = l_sh[rr] * alpha + sum;
          m_sh[rr] = m_new;
          alpha_sh[rr] = alpha;
        }
      }
    }
    __syncthreads();

    // value update: acc[row][col] = alpha * acc + sum_j p_j v_j[col]; the 16 values of this
    // thread's columns are read once and reused for every row
    float vv[kPage][S::kCPT];
#pragma unroll
    for (int j = 0; j < kPage; ++j)
#pragma unroll
      for (int c = 0; c < S::kCPT; ++c)
        vv[j][c] = spec::Elem<T>::to_f32(vs[j * S::kKStr + col0 + c * S::kNCol]);
#pragma unroll
    for (int ri = 0; ri < S::kRPT; ++ri) {
      const int rr = rg + ri * S::kRG;
      if (rr < nr) {
        const float a = alpha_sh[rr];
        const float4 *pr4 = reinterpret_cast<const float4 *>(ss + rr * kPage);
        float pj[kPage];
#pragma unroll
        for (int j4 = 0; j4 < kPage / 4; ++j4) {
          const float4 t = pr4[j4];
          pj[4 * j4] = t.x; pj[4 * j4 + 1] = t.y; pj[4 * j4 + 2] = t.z; pj[4 * j4 + 3] = t.w;
        }
#pragma unroll
        for (int c = 0; c < S::kCPT; ++c) {
          float o = acc[ri][c] * a;
#pragma unroll
          for (int j = 0; j < kPage; ++j) o = fmaf(pj[j], vv[j][c], o);
          acc[ri][c] = o;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < S::kGPT; ++x) { kcur[x] = knxt[x]; vcur[x] = vnxt[x]; }
  }

  const size_t base = ((size_t)(b * Hkv + g) * nsplit + s) * GK1 + rr0;
  if (tid < nr) part_ml[base + tid] = make_float2(m_sh[tid], l_sh[tid]);
#pragma unroll
  for (int ri = 0; ri < S::kRPT; ++ri) {
    const int rr = rg + ri * S::kRG;
    if (rr < nr) {
#pragma unroll
      for (int c = 0; c < S::kCPT; ++c)
        part_acc[(base + rr) * D + col0 + c * S::kNCol] = acc[ri][c];
    }
  }
}

// Grid: (K1 * Hq, D / 64, B).  Merges the splits of one output row (64 columns per workgroup)
// with log-sum-exp weights.  Thread (c, sg) sums the splits s = sg (mod 4) of column c; the
// split loads are issued 16 at a time so a merge costs a few memory round trips.
constexpr int kCombCols = 64;
constexpr int kCombGroups = kThreads / kCombCols;   // 4
constexpr int kCombBatch = 32;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_combine(
    const float2 *__restrict__ part_ml, const float *__restrict__ part_acc,
    const int32_t *__restrict__ ctx_lens, float *__restrict__ out, int K1, int Hq, int Hkv,
    int max_pages, int window, int pps, int nsplit, int GK1) {
  __shared__ float w_sh[kMaxSplits];
  __shared__ float red[kThreads];
  const int tid = threadIdx.x;
  const int row = blockIdx.x, b = blockIdx.z;
  const int i = row / Hq, h = row - i * Hq;
  const int G = Hq / Hkv, g = h / G, rr = i * G + (h - g * G);
  const Span sp = seq_span(ctx_lens[b], K1, window, max_pages);
  const int ns = (sp.np + pps - 1) / pps;
  const size_t base = (size_t)(b * Hkv + g) * nsplit * GK1 + rr;   // + s * GK1

  // all loads of the merge at once: (max, sum) of every split and up to kCombBatch partial
  // outputs per thread (split s = sg + kCombGroups * u of column d)
  const int c = tid % kCombCols, sg = tid / kCombCols;
  const int d = blockIdx.y * kCombCols + c;
  float2 ml[kMaxSplits / kThreads];
#pragma unroll
  for (int x = 0; x < kMaxSplits / kThreads; ++x) {
    const int s = tid + x * kThreads;
    ml[x] = s < ns ? part_ml[base + (size_t)s * GK1] : make_float2(-INFINITY, 0.f);
  }
  float v[kCombBatch];
#pragma unroll
  for (int u = 0; u < kCombBatch; ++u) {
    const int s = sg + u * kCombGroups;
    v[u] = s < ns ? part_acc[(base + (size_t)s * GK1) * D + d] : 0.f;
  }
  float m = -INFINITY;
#pragma unroll
  for (int x = 0; x < kMaxSplits / kThreads; ++x) m = fmaxf(m, ml[x].x);
  red[tid] = m;
  __syncthreads();
  for (int h2 = kThreads / 2; h2 > 0; h2 >>= 1) {
    if (tid < h2) red[tid] = fmaxf(red[tid], red[tid + h2]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float l = 0.f;
#pragma unroll
  for (int x = 0; x < kMaxSplits / kThreads; ++x) {
    const int s = tid + x * kThreads;
    if (s < ns) {
      const float w = ml[x].x == -INFINITY ? 0.f : exp2f(ml[x].x - M);
      w_sh[s] = w;
      l += w * ml[x].y;
    }
  }
  red[tid] = l;
  __syncthreads();
  for (int h2 = kThreads / 2; h2 > 0; h2 >>= 1) {
    if (tid < h2) red[tid] += red[tid + h2];
    __syncthreads();
  }
  const float L = red[0];
  __syncthreads();

  float o = 0.f;
#pragma unroll
  for (int u = 0; u < kCombBatch; ++u) {
    const int s = sg + u * kCombGroups;
    if (s < ns) o = fmaf(w_sh[s], v[u], o);
  }
  for (int s0 = sg + kCombGroups * kCombBatch; s0 < ns; s0 += kCombGroups * kCombBatch) {
    float v2[kCombBatch];
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u) {
      const int s = s0 + u * kCombGroups;
      v2[u] = s < ns ? part_acc[(base + (size_t)s * GK1) * D + d] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u) {
      const int s = s0 + u * kCombGroups;
      if (s < ns) o = fmaf(w_sh[s], v2[u], o);
    }
  }
  red[tid] = o;
  __syncthreads();
  if (sg == 0) {
    const float tot = ((red[c] + red[c + kCombCols]) + red[c + 2 * kCombCols]) + red[c + 3 * kCombCols];
    out[(((size_t)b * K1 + i) * Hq + h) * D + d] = L > 0.f ? tot / L : 0.f;
  }
}

struct AttnPlan {
  int pps, nsplit, nrowchunk, GK1;
  size_t off_ml, off_acc, bytes;
};

AttnPlan plan(int B, int K1, int Hq, int Hkv, int D, int max_pages, int window) {
  AttnPlan pl;
  pl.GK1 = (Hq / Hkv) * K1;
  pl.nrowchunk = spec::ceil_div(pl.GK1, kRows);
  int span = max_pages;
  if (window > 0) span = min(max_pages, spec::ceil_div(window + K1 - 1, kPage) + 1);
  span = max(span, 1);
  const long units = (long)B * Hkv * pl.nrowchunk;
  const int wanted = (int)max(1L, (kTargetWGs + units - 1) / units);
  pl.pps = max(kMinPagesPerSplit, spec::ceil_div(span, wanted));
  pl.pps = min(max(pl.pps, spec::ceil_div(span, kMaxSplits)), kMaxPagesPerSplit);
  pl.nsplit = spec::ceil_div(span, pl.pps);
  const size_t rows = (size_t)B * Hkv * pl.nsplit * pl.GK1;
  pl.off_ml = 0;
  pl.off_acc = spec::align_up(rows * sizeof(float2), 256);
  pl.bytes = pl.off_acc + spec::align_up(rows * D * sizeof(float), 256);
  return pl;
}

template <int D, typename T>
int launch(const void *q, const void *kp, const void *vp, const int32_t *table,
           const int32_t *ctx, float *out, int B, int K1, int Hq, int Hkv, int num_pages,
           int max_pages, int window, float scale, const AttnPlan &pl, char *ws,
           hipStream_t st) {
  using S = AttnShape<D, T>;
  static bool attr_set = false;   // per instantiation; setting it twice is harmless
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_partial<D, T>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)S::kLds) != hipSuccess)
      return spec::fail(SPEC_EHIP, "spec_verify_attn: cannot reserve %zu bytes of LDS", S::kLds);
    attr_set = true;
  }
  float2 *ml = reinterpret_cast<float2 *>(ws + pl.off_ml);
  float *acc = reinterpret_cast<float *>(ws + pl.off_acc);
  dim3 grid(pl.nsplit, Hkv * pl.nrowchunk, B);
  hipLaunchKernelGGL((attn_partial<D, T>), grid, dim3(kThreads), S::kLds, st,
                     static_cast<const T *>(q), static_cast<const T *>(kp),
                     static_cast<const T *>(vp), table, ctx, ml, acc, K1, Hq, Hkv, num_pages,
                     max_pages, window, scale * kLog2e, pl.pps, pl.nsplit, pl.GK1);
  int rc = spec::launched("attn_partial");
  if (rc != SPEC_OK) return rc;
  hipLaunchKernelGGL((attn_combine<D>), dim3(K1 * Hq, D / kCombCols, B), dim3(kThreads), 0, st, ml, acc, ctx,
                     out, K1, Hq, Hkv, max_pages, window, pl.pps, pl.nsplit, pl.GK1);
  return spec::launched("attn_combine");
}

template <typename T>
int dispatch_d(int D, const void *q, const void *kp, const void *vp, const int32_t *table,
               const int32_t *ctx, float *out, int B, int K1, int Hq, int Hkv, int num_pages,
               int max_pages, int window, float scale, const AttnPlan &pl, char *ws,
               hipStream_t st) {
  switch (D) {
    case 64: return launch<64, T>(q, kp, vp, table, ctx, out, B, K1, Hq, Hkv, num_pages, max_pages, window, scale, pl, ws, st);
    case 128: return launch<128, T>(q, kp, vp, table, ctx, out, B, K1, Hq, Hkv, num_pages, max_pages, window, scale, pl, ws, st);
    case 256: return launch<256, T>(q, kp, vp, table, ctx, out, B, K1, Hq, Hkv, num_pages, max_pages, window, scale, pl, ws, st);
    default: return launch<512, T>(q, kp, vp, table, ctx, out, B, K1, Hq, Hkv, num_pages, max_pages, window, scale, pl, ws, st);
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int B, int K1, int Hq, int Hkv, int D, int page_size, int max_pages, int window) {
  SPEC_REQUIRE(B > 0 && K1 > 0 && Hq > 0 && Hkv > 0 && max_pages > 0, SPEC_EINVAL,
               "spec_verify_attn: B=%d K1=%d Hq=%d Hkv=%d max_pages_per_seq=%d must be positive",
               B, K1, Hq, Hkv, max_pages);
  SPEC_REQUIRE(Hq % Hkv == 0, SPEC_EINVAL, "spec_verify_attn: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  SPEC_REQUIRE(window >= 0, SPEC_EINVAL, "spec_verify_attn: window=%d is negative", window);
  SPEC_REQUIRE(K1 <= 64, SPEC_EUNSUPPORTED, "spec_verify_attn: K1=%d exceeds 64", K1);
  SPEC_REQUIRE(D == 64 || D == 128 || D == 256 || D == 512, SPEC_EUNSUPPORTED,
               "spec_verify_attn: head dim %d not in {64, 128, 256, 512}", D);
  SPEC_REQUIRE(page_size == kPage, SPEC_EUNSUPPORTED, "spec_verify_attn: page_size=%d, only 16", page_size);
  SPEC_REQUIRE((long)max_pages <= (long)kMaxSplits * kMaxPagesPerSplit, SPEC_EUNSUPPORTED,
               "spec_verify_attn: max_pages_per_seq=%d exceeds %d", max_pages,
               kMaxSplits * kMaxPagesPerSplit);
  return SPEC_OK;
}

}  // namespace

extern "C" size_t spec_verify_attn_workspace(int B, int K1, int Hq, int Hkv, int D,
                                             int page_size, int max_pages_per_seq, int window) {
  spec::clear_error();
  if (check_shape(B, K1, Hq, Hkv, D, page_size, max_pages_per_seq, window) != SPEC_OK) return 0;
  return plan(B, K1, Hq, Hkv, D, max_pages_per_seq, window).bytes;
}

extern "C" int spec_verify_attn(const void *q, const void *k_pool, const void *v_pool,
                                const int32_t *page_table, const int32_t *ctx_lens, float *out,
                                int B, int K1, int Hq, int Hkv, int D, int page_size,
                                int num_pages, int max_pages_per_seq, int window, float scale,
                                spec_dtype dtype, void *workspace, size_t workspace_bytes,
                                void *stream) {
  spec::clear_error();
  int rc = check_shape(B, K1, Hq, Hkv, D, page_size, max_pages_per_seq, window);
  if (rc != SPEC_OK) return rc;
  SPEC_REQUIRE(q && k_pool && v_pool && page_table && ctx_lens && out, SPEC_EINVAL,
               "spec_verify_attn: null pointer argument");
  SPEC_REQUIRE(num_pages > 0, SPEC_EINVAL, "spec_verify_attn: num_pages=%d must be positive", num_pages);
  SPEC_REQUIRE(dtype == SPEC_F32 || dtype == SPEC_BF16, SPEC_EUNSUPPORTED,
               "spec_verify_attn: unsupported dtype %d", (int)dtype);
  SPEC_REQUIRE(aligned16(q) && aligned16(k_pool) && aligned16(v_pool), SPEC_EINVAL,
               "spec_verify_attn: q, k_pool and v_pool need 16-byte alignment");
  const AttnPlan pl = plan(B, K1, Hq, Hkv, D, max_pages_per_seq, window);
  SPEC_REQUIRE(workspace != nullptr && workspace_bytes >= pl.bytes, SPEC_EWORKSPACE,
               "spec_verify_attn: workspace of %zu bytes needed, %zu given", pl.bytes, workspace_bytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  if (dtype == SPEC_BF16)
    return dispatch_d<uint16_t>(D, q, k_pool, v_pool, page_table, ctx_lens, out, B, K1, Hq, Hkv,
                                num_pages, max_pages_per_seq, window, scale, pl, ws, st);
  return dispatch_d<float>(D, q, k_pool, v_pool, page_table, ctx_lens, out, B, K1, Hq, Hkv,
                           num_pages, max_pages_per_seq, window, scale, pl, ws, st);
}
