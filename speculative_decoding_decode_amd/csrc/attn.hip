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
constexpr int kWaves = kThreads / 64;
constexpr int kPage = 16;
constexpr int kRows = 32;            // query rows per workgroup
constexpr int kTargetWGs = 4096;     // splits are sized so the grid reaches about this many
constexpr long kSmallWork = 2048;    // page-heads below which splits may be a single page
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D, typename T>
struct AttnShape {
  static constexpr int kEPG = 16 / (int)sizeof(T);       // elements per 16-byte group
  static constexpr int kGPR = D / kEPG;                  // 16-byte groups per row
  static constexpr int kStr = D + kEPG;                  // LDS row stride (elements), 16-byte pad
  static constexpr int kTileG = kPage * kGPR;            // 16-byte groups per K (or V) page tile
  static constexpr int kGPT = (kTileG + kThreads - 1) / kThreads;   // per thread
  static constexpr int kQPT = (kRows * kGPR + kThreads - 1) / kThreads;
  static constexpr int kDT = D / 16;                     // 16-wide tiles of the head dim
  static constexpr int kDTW = kDT / kWaves;              // of them per wave
  static constexpr size_t kLds = (size_t)(kRows + 2 * kPage) * kStr * sizeof(T);
};

// MFMA helpers: QK^T per K-step, PV per page.  16x16 accumulator layout: lane l holds rows
// (or d) 4*(l/16) + i, i = 0..3, of column l % 16.
template <typename T> struct AttnMma;
template <> struct AttnMma<uint16_t> {
  static constexpr int kStepQK = 32;   // head-dim elements per QK MFMA step (16x16x32 bf16)
  // S^T[key][row] += K[key][d0 + ...] . Q[row][d0 + ...]
  __device__ static __forceinline__ f32x4_t qk(const uint16_t *krow, const uint16_t *qrow, int lq, f32x4_t c) {
    const uint4 a = *reinterpret_cast<const uint4 *>(krow + lq * 8);
    const uint4 b = *reinterpret_cast<const uint4 *>(qrow + lq * 8);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // O^T[d][row] += V^T[d][keys 4*lq + i] . P^T[keys 4*lq + i][row].  P is split into a bf16
  // head and a bf16 tail (p = hi + lo to 2^-17 relative), two MFMAs, so the products keep
  // fp32-level accuracy while V stays exact bf16.
  __device__ static __forceinline__ f32x4_t pv(const uint16_t *vs, int str, int dcol, int lq,
                                               const float (&p)[4], f32x4_t c) {
    bf16x4_t a, hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = __builtin_bit_cast(__bf16, vs[(4 * lq + i) * str + dcol]);
      hi[i] = static_cast<__bf16>(p[i]);
      lo[i] = static_cast<__bf16>(p[i] - static_cast<float>(hi[i]));
    }
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, hi, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, lo, c, 0, 0, 0);
  }
};
template <> struct AttnMma<float> {
  static constexpr int kStepQK = 16;   // four 16x16x4 fp32 MFMAs, one per fragment element
  __device__ static __forceinline__ f32x4_t qk(const float *krow, const float *qrow, int lq, f32x4_t c) {
    const float4 a = *reinterpret_cast<const float4 *>(krow + lq * 4);
    const float4 b = *reinterpret_cast<const float4 *>(qrow + lq * 4);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
    return c;
  }
  // MFMA j contracts the keys 4*lq + j (K slot lq), so P stays in fp32 and needs no transpose.
  __device__ static __forceinline__ f32x4_t pv(const float *vs, int str, int dcol, int lq,
                                               const float (&p)[4], f32x4_t c) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(vs[(4 * lq + j) * str + dcol], p[j], c, 0, 0, 0);
    return c;
  }
};

// Grid: (B * Hkv * nrowchunk, nsplit).
// Round trips before the first page is in LDS: the split's page ids, then the queries and the
// first page's K/V together; while a page is being processed the next page's K/V are in flight
// in registers.  Per page, every wave computes the whole 16-key x (up to 32)-row score tile
// with MFMAs (so scores never go through LDS), runs the online softmax in registers (4 keys
// per lane, two cross-lane shuffles for the row max and sum), and accumulates its quarter of
// the head dim with MFMAs whose B operand is the probability tile as the score MFMA left it.
template <int D, typename T>
__global__ __launch_bounds__(kThreads) void attn_partial(
    const T *__restrict__ q, const T *__restrict__ kpool, const T *__restrict__ vpool,
    const int32_t *__restrict__ table, const int32_t *__restrict__ ctx_lens,
    float2 *__restrict__ part_ml, float *__restrict__ part_acc, int K1, int Hq, int Hkv,
    int num_pages, int max_pages, int window, float qscale, int pps, int nsplit, int GK1) {
  using S = AttnShape<D, T>;
  using M = AttnMma<T>;
  constexpr int RT = kRows / 16;                                   // row tiles
  extern __shared__ __align__(16) unsigned char smem[];
  T *qs = reinterpret_cast<T *>(smem);                             // [kRows][kStr]
  T *ks = qs + kRows * S::kStr;                                    // [16][kStr]
  T *vs = ks + kPage * S::kStr;                                    // [16][kStr]
  __shared__ int pid_sh[kMaxPagesPerSplit];

  const int tid = threadIdx.x, lane = tid & (spec::kWave - 1), wave = tid / spec::kWave;
  const int lr = lane & 15, lq = lane >> 4;
  // blockIdx.x enumerates (sequence, KV head, row chunk) units and blockIdx.y the splits in
  // reverse: the highest splits, which only the longest sequences have, are dispatched first,
  // so ragged batches run longest-first instead of ending on a few long workgroups.
  const int nrc = (GK1 + kRows - 1) / kRows;
  const int unit = blockIdx.x, s = nsplit - 1 - (int)blockIdx.y;
  const int b = unit / (Hkv * nrc), g = (unit / nrc) % Hkv, rc = unit % nrc;
  const int G = Hq / Hkv;
  const Span sp = seq_span(ctx_lens[b], K1, window, max_pages);
  const int ns = (sp.np + pps - 1) / pps;
  if (s >= ns) return;
  const int pg_begin = sp.p0 + s * pps;
  const int npg = min(sp.p0 + sp.np, pg_begin + pps) - pg_begin;
  const int rr0 = rc * kRows;
  const int nr = min(kRows, GK1 - rr0);

  // (1) page ids of the split, then the queries.  Loads are unconditional with clamped
  // indices so the wait counts the compiler inserts stay exact.
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
  __syncthreads();

  // (2) K/V of page 0 in flight while the queries land in LDS (rows >= nr zero)
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
    if (e < kRows * S::kGPR) {
      const int r = e / S::kGPR, gi = e - r * S::kGPR;
      *reinterpret_cast<uint4 *>(qs + r * S::kStr + gi * S::kEPG) =
          e < nr * S::kGPR ? qraw[x] : uint4{0u, 0u, 0u, 0u};
    }
  }

  // per-lane rows: rt * 16 + lr; their query positions and running (max, sum)
  int trow[RT];
  float m_run[RT], l_run[RT];
  f32x4_t o[RT][S::kDTW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + lr;
    trow[rt] = r < nr ? sp.ctx - K1 + (rr0 + r) / G : -1;
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < S::kDTW; ++dt) o[rt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const bool two_tiles = nr > 16;   // uniform

  for (int i = 0; i < npg; ++i) {
#pragma unroll
    for (int x = 0; x < S::kGPT; ++x) {
      const int e = tid + x * kThreads;
      if (e < S::kTileG) {
        const int row = e / S::kGPR, gi = e - row * S::kGPR;
        *reinterpret_cast<uint4 *>(ks + row * S::kStr + gi * S::kEPG) = kcur[x];
        *reinterpret_cast<uint4 *>(vs + row * S::kStr + gi * S::kEPG) = vcur[x];
      }
    }
    if (i + 1 < npg) fetch(knxt, vnxt, i + 1);
    const bool page_ok = pid_sh[i] >= 0;   // uniform
    const int pg = pg_begin + i;
    __syncthreads();

    if (page_ok) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (rt == 1 && !two_tiles) break;
        // scores S^T[key 4*lq + e][row rt*16 + lr]
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d0 = 0; d0 < D; d0 += M::kStepQK)
          sc = M::qk(ks + lr * S::kStr + d0, qs + (rt * 16 + lr) * S::kStr + d0, lq, sc);
        float sv[4];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = pg * kPage + 4 * lq + e, t = trow[rt];
          const bool vis = pos <= t && (window == 0 || t - pos < window);
          sv[e] = vis ? sc[e] * qscale : -INFINITY;
          mx = fmaxf(mx, sv[e]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[rt], mx);
        float pr[4], sum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pr[e] = sv[e] == -INFINITY ? 0.f : exp2f(sv[e] - m_new);
          sum += pr[e];
        }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        const float alpha = m_run[rt] == -INFINITY ? 0.f : exp2f(m_run[rt] - m_new);
        l_run[rt] = l_run[rt] * alpha + sum;
        m_run[rt] = m_new;
#pragma unroll
        for (int dt = 0; dt < S::kDTW; ++dt) {
          o[rt][dt] *= alpha;
          o[rt][dt] = M::pv(vs, S::kStr, (wave * S::kDTW + dt) * 16 + lr, lq, pr, o[rt][dt]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < S::kGPT; ++x) { kcur[x] = knxt[x]; vcur[x] = vnxt[x]; }
  }

  // partial outputs: lane holds O^T[d = dtile*16 + 4*lq + e][row rt*16 + lr]
  const size_t base = ((size_t)(b * Hkv + g) * nsplit + s) * GK1 + rr0;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + lr;
    if (r < nr) {
      if (wave == 0 && lq == 0) part_ml[base + r] = make_float2(m_run[rt], l_run[rt]);
#pragma unroll
      for (int dt = 0; dt < S::kDTW; ++dt) {
        const int d = (wave * S::kDTW + dt) * 16 + 4 * lq;
        *reinterpret_cast<float4 *>(part_acc + (base + r) * D + d) =
            make_float4(o[rt][dt][0], o[rt][dt][1], o[rt][dt][2], o[rt][dt][3]);
      }
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
  // Beyond a small amount of work, splits hold at least GK1 / 2 pages so the partial outputs
  // (GK1 x D fp32 per split) stay within 1/8 of the KV bytes they summarise; below it, latency
  // rules and splits may be single pages.
  const int pmin = (long)span * units > kSmallWork ? max(1, spec::ceil_div(pl.GK1, 2)) : 1;
  pl.pps = max(max(kMinPagesPerSplit, pmin), spec::ceil_div(span, wanted));
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
  dim3 grid(B * Hkv * pl.nrowchunk, pl.nsplit);
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
