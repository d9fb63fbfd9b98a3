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
// Design (gfx950): the work is the flat list of (sequence, KV head, row chunk, visible page)
// items, and the grid is about one workgroup per resident slot of the GPU ("stream-K"): every
// workgroup takes an equal contiguous share of the list, whatever the lengths of the sequences
// in a ragged batch, so every slot has the same number of pages to read.  The share is
// computed on the device from the context lengths (each workgroup and each merge wave derives
// the same numbers).  Within a share a workgroup walks the pages of each (sequence, KV head, row chunk)
// unit it touches: each 16-token page of K and of V is one contiguous 16*D block per head,
// read with nontemporal 16-byte loads (each page is read once per call) two pages ahead.  At
// head dims 64 and 128, in fp32, and at head dim 256 with two row tiles, pages are staged
// through LDS; at head dim 512, and 256 with one row tile, in bf16, each wave loads its
// quarter of the head dim straight into MFMA operand registers (unit_quarter).  Scores come
// from MFMAs (keys x rows tile), the online softmax runs in registers with wavefront shuffles,
// and the value update is a second MFMA per 16 columns of the head dim.  For every unit it touches
// the workgroup writes one partial (max, sum, unnormalised output); a second kernel merges the
// partials of each output row with log-sum-exp weights, one workgroup per row.  All
// exponentials are base 2 with log2(e) folded into the query scale.
#include <math.h>

#include "common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPage = 16;
constexpr int kMaxPagesPerPiece = 256;   // page ids of one piece are staged in LDS
constexpr int kMaxPiecesPerUnit = 4096;  // partials merged for one output row
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
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // one 16-byte group

// DPP row_ror:8 on every dword: lane i of each 16-lane row takes lane i ^ 8 of the same row.
__device__ __forceinline__ u32x4_t rows_ror8(u32x4_t v) {
  return u32x4_t{(uint32_t)spec::dpp_move<0x128>((int)v[0]), (uint32_t)spec::dpp_move<0x128>((int)v[1]),
                 (uint32_t)spec::dpp_move<0x128>((int)v[2]), (uint32_t)spec::dpp_move<0x128>((int)v[3])};
}
__device__ __forceinline__ u32x4_t rows_pick(bool first, u32x4_t a, u32x4_t b) {
  return u32x4_t{first ? a[0] : b[0], first ? a[1] : b[1], first ? a[2] : b[2], first ? a[3] : b[3]};
}

template <int D, typename T, int RT>
struct AttnShape {
  static constexpr int kEPG = 16 / (int)sizeof(T);       // elements per 16-byte group
  static constexpr int kGPR = D / kEPG;                  // 16-byte groups per row
  static constexpr int kStr = D + kEPG;                  // LDS row stride (elements), 16-byte pad
  static constexpr int kTileG = kPage * kGPR;            // 16-byte groups per K (or V) page tile
  static constexpr int kGPT = (kTileG + kThreads - 1) / kThreads;   // per thread
  static constexpr int kRowsWG = 16 * RT;                // query rows of one workgroup
  static constexpr int kQPT = (kRowsWG * kGPR + kThreads - 1) / kThreads;
  static constexpr int kDT = D / 16;                     // 16-wide tiles of the head dim
  static constexpr int kDTW = kDT / kWaves;              // of them per wave
  static constexpr size_t kTiles = (size_t)(kRowsWG + 2 * kPage) * kStr * sizeof(T);
  // Waves per SIMD the register budget is set for (one wave of each workgroup per SIMD): as
  // many workgroups as a CU's 160 KB of LDS holds, capped where the page buffers and output
  // tiles (growing with D * RT * element size) would no longer fit the registers.
  static constexpr int kRowBytes = D * RT * (int)sizeof(T);
  static constexpr int kRegCap = kRowBytes <= 512 ? 4 : kRowBytes <= 1024 ? 3 : kRowBytes <= 2048 ? 2 : 1;
  // Split scores: at D >= 256 each wave computes the scores over its quarter of the head dim
  // and the four partial tiles are summed through LDS (kSplitBytes of scratch) instead of
  // every wave computing the whole dot product, wherever the scratch costs no workgroup slot.
  static constexpr size_t kSplitBytes = (size_t)kWaves * RT * 64 * 16;
  static constexpr int kWGs(size_t lds) {
    const int n = (int)((160u * 1024u) / lds);
    return n < kRegCap ? n : kRegCap;
  }
  static constexpr bool kSplit = D >= 256 && kWGs(kTiles + kSplitBytes) >= kWGs(kTiles);
  // Head dim 512, and head dim 256 at one row tile, in bf16: each wave streams its quarter of
  // the head dim straight into MFMA operand registers (unit_quarter below); LDS holds only the
  // double-buffered score exchange (and at two row tiles, after a piece's pages, its partial
  // on the way out: 66 KB at D = 512), and registers set the resident workgroups per CU: four at
  // D = 256 (103 VGPRs, the most without spills), two at D = 512 (a third fits at one row tile,
  // but the batch-32 workload streamed 3% slower with it on MI355X).  Head dim 256 at two row
  // tiles stays with the LDS-staged path, which measured 6% faster there (15.9 against 16.9 us
  // per sliding layer at batch 8, k = 5).
  static constexpr bool kQuarter = (D == 512 || (D == 256 && RT == 1)) && sizeof(T) == 2;
  static constexpr size_t kQuarterXch = 2 * (size_t)kWaves * RT * 64 * 16;   // score exchange
  static constexpr size_t kQuarterStg =                                      // partial (RT 2)
      RT == 2 ? (size_t)kWaves * 16 * RT * (D / 4 + 4) * 4 : 0;
  static constexpr size_t kQuarterLds = kQuarterXch > kQuarterStg ? kQuarterXch : kQuarterStg;
  static constexpr size_t kLds = kQuarter ? kQuarterLds : kTiles + (kSplit ? kSplitBytes : 0);
  static constexpr int kQuarterWaves = D == 512 ? 2 : 4;
  static constexpr int kWavesPerEU = kQuarter ? kQuarterWaves : kWGs(kLds);
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
  // head and a bf16 tail (p = hi + lo to 2^-17 relative) so the products keep fp32-level
  // accuracy while V stays exact bf16.  Both halves go through one 16x16x32 MFMA: the
  // contraction index is only a label shared by the two operands, so this lane's 8 slots
  // carry its 4 keys twice, (V, hi) in the first four and (V, lo) in the last four, and no
  // lane needs another lane's probabilities.
  __device__ static __forceinline__ f32x4_t pv(const uint16_t *vs, int str, int dcol, int lq,
                                               const float (&p)[4], f32x4_t c) {
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 v = __builtin_bit_cast(__bf16, vs[(4 * lq + i) * str + dcol]);
      const __bf16 hi = static_cast<__bf16>(p[i]);
      a[i] = v;
      a[i + 4] = v;
      b[i] = hi;
      b[i + 4] = static_cast<__bf16>(p[i] - static_cast<float>(hi));
    }
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// ---------------------------------------------------------------- the stream-K split
// Item list: for b = 0..B-1, unit j = 0..U-1 (U = Hkv * row chunks, j = g * nrc + rc), the
// np_b visible pages of sequence b.  Unit (b, j) starts at U * P_b + j * np_b, P_b = sum of
// np over the sequences before b.  Workgroup w owns items [w * C, (w + 1) * C); the piece it
// computes of unit u = b * U + j is stored at partial index w + u (consecutive pieces along
// the list raise w, u or both, so the index is unique and below nwg + B * U).

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uni64(long long v) {
  const unsigned long long u = static_cast<unsigned long long>(v);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(u));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(u >> 32));
  return static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo);
}

struct StreamPlan {
  long long total;   // items
  int C;             // items per workgroup
  int ctx0, np0, incl0;   // this lane's sequence (= lane) of the first 64: context, visible
                          // pages, inclusive prefix sum of visible pages
};

// Quotient of non-negative a / b, in 32 bits when both fit.
__device__ __forceinline__ long long div_nn(long long a, long long b) {
  if (((a | b) >> 31) == 0) return (long long)((unsigned)a / (unsigned)b);
  return a / b;
}

// Same result in every lane of every wave that calls it with the same arguments.  c_floor
// (from the host) keeps the pieces of one unit within kMaxPiecesPerUnit.
__device__ StreamPlan stream_plan(const int32_t *__restrict__ ctx_lens, int B, int K1, int window,
                                  int max_pages, int U, int nwg, int c_floor, int lane) {
  StreamPlan pl;
  long long tot = 0;
  for (int c0 = 0; c0 < B; c0 += spec::kWave) {
    const int c = ctx_lens[min(c0 + lane, B - 1)];
    const int np = c0 + lane < B ? seq_span(c, K1, window, max_pages).np : 0;
    const int incl = wave_incl_scan(np, lane);
    if (c0 == 0) {
      pl.ctx0 = c;
      pl.np0 = np;
      pl.incl0 = incl;
    }
    tot += __shfl(incl, spec::kWave - 1);
  }
  pl.total = uni64(tot * U);
  const long long c = div_nn(pl.total + nwg - 1, nwg);
  pl.C = uni((int)max((long long)c_floor, c));
  return pl;
}

// Context length of sequence b (uniform b): from the plan's registers for the first 64.
__device__ __forceinline__ int ctx_of(const int32_t *__restrict__ ctx_lens, const StreamPlan &pl, int b) {
  return b < spec::kWave ? uni(__shfl(pl.ctx0, b)) : ctx_lens[b];
}

// Visible pages of the sequences before b (uniform b).
__device__ __forceinline__ long long pages_before(const int32_t *__restrict__ ctx_lens,
                                                  const StreamPlan &pl, int b, int K1, int window,
                                                  int max_pages, int lane) {
  if (b < spec::kWave) return b == 0 ? 0 : uni(__shfl(pl.incl0, b - 1));
  long long Pb = __shfl(pl.incl0, spec::kWave - 1);
  for (int c0 = spec::kWave; c0 < b; c0 += spec::kWave) {
    const int bb = min(c0 + lane, b - 1);
    Pb += spec::wave_sum(c0 + lane < b ? seq_span(ctx_lens[bb], K1, window, max_pages).np : 0);
  }
  return uni64(Pb);
}

// ---------------------------------------------------------------- head dims 256 and 512, bf16
// One (sequence, KV head, row chunk) unit's pages [pg_begin, pg_begin + npg), with wave w owning
// the head-dim quarter [DQ w, DQ w + DQ), DQ = D / 4, of the scores and of the output.  Nothing is staged in
// LDS: each wave loads its quarter of every page's K and V straight into MFMA operand registers,
// and the only exchange between waves is the sum of the four partial score tiles of a page
// (double-buffered in LDS, one workgroup barrier per page).
//  * Scores S^T = K Q^T.  The contraction over the head dim may take its dims in any order that
//    K and Q share, so K is loaded with 128-byte runs per key row: in instruction h of a 128-byte
//    segment, lane 16 G + 8 q + r reads 16-byte slot 4 q + G of key 8 h + r; the A fragment of the
//    segment's first / second 32-dim K-step (lane 16 G + j: slot 4 s + G of key j) is then, per
//    dword, instruction 0 or 1 kept or rotated by eight lanes within the 16-lane row (DPP).  Q's
//    B fragments use the plain layout (row j, slot 4 s + G), loaded once per unit.
//  * Values O^T[d][row] += V^T[d][key] P^T[key][row].  With E = DQ / 16 dims per lane, lane
//    16 G + c loads V[keys 4 G .. 4 G + 3][dims E c .. E c + E - 1] of the quarter (four loads of
//    2 E bytes, 32 E contiguous bytes per key row and instruction).  In value tile t (t < E) the
//    A-operand row i stands for dim E i + t, so lane 16 G + c takes element t of its own four
//    registers: no transpose, no LDS.  P is split into a bf16 head and tail (the two halves of
//    the 32-wide contraction), as in AttnMma<uint16_t>::pv.  Accumulator lane (j, q) element e
//    of tile t is output dim E (4 q + e) + t of the quarter.
template <int D, int RT>
__device__ __forceinline__ void unit_quarter(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kpool,
    const uint16_t *__restrict__ vpool, const int32_t *__restrict__ table, int *pid_sh,
    f32x4_t *sred, float2 *__restrict__ part_ml, float *__restrict__ part_acc, int b, int K1,
    int Hq, int Hkv, int num_pages, int max_pages, int window, float qscale, int g, int G,
    int rr0, int nr, int pg_begin, int npg, long long piece, int rstride, int ctx) {
  constexpr int DQ = D / 4, kPage = 16;
  constexpr int KS = DQ / 32;            // 32-dim K-steps of the quarter
  constexpr int SEG = DQ / 64;           // 128-byte segments of a key row's quarter
  constexpr int E = DQ / 16;             // V dims per lane, value tiles per wave
  typedef uint32_t vreg_t __attribute__((ext_vector_type(E / 2)));
  static_assert(SEG >= 1 && (E == 4 || E == 8), "quarters of 64 or 128 dims");
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  const int tid = threadIdx.x, lane = tid & (spec::kWave - 1), wave = tid / spec::kWave;
  const int lr = lane & 15, lq = lane >> 4;
  const int r8 = lane & 7, qq = (lane >> 3) & 1;

  // (1) page ids of the piece, then the query fragments of this wave's quarter
  const int pid_reg = table[(size_t)b * max_pages + pg_begin + min(tid, npg - 1)];
  u32x4_t qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + lr;
    const int rr = rr0 + min(row, nr - 1), i = rr / G, h = g * G + (rr - i * G);
    const uint16_t *qrow = q + (((size_t)b * K1 + i) * Hq + h) * D + DQ * wave + 8 * lq;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(qrow + 32 * s);
      qf[rt][s] = row < nr ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  if (tid < npg) pid_sh[tid] = (pid_reg >= 0 && pid_reg < num_pages) ? pid_reg : -1;
  __syncthreads();

  struct PageRegs {
    u32x4_t k[2 * SEG];   // 2 s + h: keys 8 h .. 8 h + 7, 128-byte run of segment s
    vreg_t v[4];          // keys 4 lq + x, dims E lr .. E lr + E - 1 of the quarter
  };
  // A fetch past the piece reads the pools' first 16 bytes in every lane, so the loads stay
  // unconditional (exact waits) without a trip to memory.
  auto fetch = [&](PageRegs &pr, int i) __attribute__((always_inline)) {
    const bool real = i < npg;
    const int pid = pid_sh[min(i, npg - 1)];
    const size_t base = real ? ((size_t)(pid < 0 ? 0 : pid) * Hkv + g) * kPage * D : 0;
#pragma unroll
    for (int s = 0; s < SEG; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const size_t off = real ? (size_t)(8 * h + r8) * D + DQ * wave + 64 * s + 8 * (4 * qq + lq) : 0;
        pr.k[2 * s + h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(kpool + base + off));
      }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const size_t off = real ? (size_t)(4 * lq + x) * D + DQ * wave + E * lr : 0;
      pr.v[x] = __builtin_nontemporal_load(reinterpret_cast<const vreg_t *>(vpool + base + off));
    }
  };

  int trow[RT];
  float m_run[RT], l_run[RT];
  f32x4_t acc[RT][E];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + lr;
    trow[rt] = r < nr ? ctx - K1 + (rr0 + r) / G : -1;
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int t = 0; t < E; ++t) acc[rt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const bool two_tiles = nr > 16;   // uniform
  int par = 0;                      // score-exchange buffer of the next page that is computed

  auto page = [&](const PageRegs &pr, int i) __attribute__((always_inline)) {
    if (pid_sh[i] < 0) return;       // uniform: an invalid page id hides its keys
    const int pg = pg_begin + i;
    f32x4_t part[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) part[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SEG; ++s) {
      const u32x4_t k0 = pr.k[2 * s], k1 = pr.k[2 * s + 1];
      const u32x4_t f0 = rows_pick(lr < 8, k0, rows_ror8(k1));
      const u32x4_t f1 = rows_pick(lr < 8, rows_ror8(k0), k1);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (rt == 1 && !two_tiles) break;
        part[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f0),
                                                           __builtin_bit_cast(bf16x8, qf[rt][2 * s]), part[rt], 0, 0, 0);
        part[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f1),
                                                           __builtin_bit_cast(bf16x8, qf[rt][2 * s + 1]), part[rt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) sred[((par * kWaves + wave) * RT + rt) * 64 + lane] = part[rt];
    __syncthreads();
    f32x4_t scs[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4_t t = sred[((par * kWaves) * RT + rt) * 64 + lane];
#pragma unroll
      for (int w2 = 1; w2 < kWaves; ++w2) t += sred[((par * kWaves + w2) * RT + rt) * 64 + lane];
      scs[rt] = t;
    }
    par ^= 1;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (rt == 1 && !two_tiles) break;
      const f32x4_t sc = scs[rt];
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
      float pr_[4], sum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pr_[e] = sv[e] == -INFINITY ? 0.f : exp2f(sv[e] - m_new);
        sum += pr_[e];
      }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      const float alpha = m_run[rt] == -INFINITY ? 0.f : exp2f(m_run[rt] - m_new);
      l_run[rt] = l_run[rt] * alpha + sum;
      m_run[rt] = m_new;
      bf16x8 bp;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 hi = static_cast<__bf16>(pr_[e]);
        bp[e] = hi;
        bp[e + 4] = static_cast<__bf16>(pr_[e] - static_cast<float>(hi));
      }
#pragma unroll
      for (int t = 0; t < E; ++t) {
        bf16x8 av;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const uint32_t w32 = pr.v[x][t >> 1];
          const __bf16 vv = __builtin_bit_cast(__bf16, (uint16_t)((t & 1) ? (w32 >> 16) : (w32 & 0xffffu)));
          av[x] = vv;
          av[x + 4] = vv;
        }
        acc[rt][t] *= alpha;
        acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bp, acc[rt][t], 0, 0, 0);
      }
    }
  };

  PageRegs ra, rb;
  fetch(ra, 0);
  fetch(rb, 1);
  for (int i = 0; i < npg; i += 2) {
    page(ra, i);
    fetch(ra, i + 2);
    if (i + 1 < npg) page(rb, i + 1);
    fetch(rb, i + 3);
  }
  __syncthreads();   // every wave is done with pid_sh and the exchange buffers

  // the piece's partial: lane (j, q) element e of tile t is dim DQ w + E (4 q + e) + t of row j.
  const size_t base = (size_t)piece * rstride;
  if constexpr (RT == 2) {
    // A lane holds 16-byte pieces of 4 (hd256) or 1 (hd512) lines of a row, so stored as they
    // lie one instruction would touch 64 lines; instead each wave puts its quarter of the rows
    // in LDS (the exchange buffers are free now) and writes it back row by row, eight lanes to
    // a 128-byte line, with nontemporal stores (the merge reads them once, from another CU).
    // At the batch-8 global layer this took the call (partial + merge) from 79.6 to 75.8 us on
    // MI355X, the batch-1 / 32K layer moved by less than the spread; at one row tile the
    // batch-1 sliding layer's merge lost 0.6 us (its partials no longer cache-resident) and
    // the batch-32 layers did not move, so one row tile keeps cached stores.  Nontemporal
    // stores of the pieces as they lie were much slower (batch-1 / 32K 65 -> 86 us).
    constexpr int SQ = DQ + 4;   // padded LDS row stride (floats)
    float *stg = reinterpret_cast<float *>(sred) + (size_t)wave * 16 * RT * SQ;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = rt * 16 + lr;
      if (r < nr && wave == 0 && lq == 0) part_ml[base + r] = make_float2(m_run[rt], l_run[rt]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int t0 = 0; t0 < E; t0 += 4)
          *reinterpret_cast<f32x4_t *>(stg + r * SQ + E * (4 * lq + e) + t0) =
              f32x4_t{acc[rt][t0][e], acc[rt][t0 + 1][e], acc[rt][t0 + 2][e], acc[rt][t0 + 3][e]};
    }
    __syncthreads();
    constexpr int C4 = DQ / 4;   // 16-byte pieces of a row's quarter
    for (int idx = lane; idx < nr * C4; idx += spec::kWave) {
      const int row = idx / C4, c = idx - row * C4;
      const f32x4_t v = *reinterpret_cast<const f32x4_t *>(stg + row * SQ + 4 * c);
      __builtin_nontemporal_store(
          v, reinterpret_cast<f32x4_t *>(part_acc + (base + row) * D + DQ * wave + 4 * c));
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = rt * 16 + lr;
      if (r < nr) {
        if (wave == 0 && lq == 0) part_ml[base + r] = make_float2(m_run[rt], l_run[rt]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float *dst = part_acc + (base + r) * D + DQ * wave + E * (4 * lq + e);
#pragma unroll
          for (int t0 = 0; t0 < E; t0 += 4)
            *reinterpret_cast<float4 *>(dst + t0) = make_float4(
                acc[rt][t0][e], acc[rt][t0 + 1][e], acc[rt][t0 + 2][e], acc[rt][t0 + 3][e]);
        }
      }
    }
  }
}

// Grid: nwg workgroups (one per resident slot, or more for very long contexts); a row chunk
// is 16 * RT query rows.  Per unit: round trips before the first page is in LDS are the
// piece's page ids, then the queries and the first two pages' K/V together.  Two register
// buffers alternate, so while page i is processed pages i + 1 and i + 2 are in flight.  Every
// fetch is unconditional (an invalid page id re-reads page 0 of the pool, whose data is never
// used; a fetch past the piece reads a 16-byte location every lane shares), which keeps the
// wait before each LDS write at "all but the newest page".  Per page, every wave gets the
// whole 16-key x (16 * RT)-row score tile in MFMA accumulator layout: at small head dims by
// computing all of it, at D >= 256 (kSplit) by computing its quarter of the head dim and
// summing the four quarters from LDS in wave order (the same bits in every wave).  It runs
// the online softmax in registers (4 keys per lane, two cross-lane shuffles for the row max
// and sum), and accumulates its quarter of the head dim with MFMAs whose B operand is the
// probability tile as the score MFMA left it.
template <int D, typename T, int RT>
__global__ __launch_bounds__(kThreads, (AttnShape<D, T, RT>::kWavesPerEU)) void attn_partial(
    const T *__restrict__ q, const T *__restrict__ kpool, const T *__restrict__ vpool,
    const int32_t *__restrict__ table, const int32_t *__restrict__ ctx_lens,
    float2 *__restrict__ part_ml, float *__restrict__ part_acc, int B, int K1, int Hq, int Hkv,
    int num_pages, int max_pages, int window, float qscale, int nwg, int c_floor, int GK1) {
  using S = AttnShape<D, T, RT>;
  using M = AttnMma<T>;
  constexpr int kRowsWG = S::kRowsWG;
  extern __shared__ __align__(16) unsigned char smem[];
  T *qs = reinterpret_cast<T *>(smem);                             // [kRowsWG][kStr]
  T *ks = qs + kRowsWG * S::kStr;                                  // [16][kStr]
  T *vs = ks + kPage * S::kStr;                                    // [16][kStr]
  f32x4_t *sred = reinterpret_cast<f32x4_t *>(smem + S::kTiles);   // [kWaves][RT][64] partial scores
  __shared__ int pid_sh[kMaxPagesPerPiece];

  const int tid = threadIdx.x, lane = tid & (spec::kWave - 1), wave = tid / spec::kWave;
  const int lr = lane & 15, lq = lane >> 4;
  const int G = Hq / Hkv;
  const int nrc = (GK1 + kRowsWG - 1) / kRowsWG, U = Hkv * nrc;
  const int rstride = min(GK1, kRowsWG);
  const int w = blockIdx.x;

  const StreamPlan sp_all = stream_plan(ctx_lens, B, K1, window, max_pages, U, nwg, c_floor, lane);
  long long p = (long long)w * sp_all.C;
  const long long pend = min(sp_all.total, p + sp_all.C);
  if (p >= pend) return;

  // the sequence holding item p: U * P_b <= p < U * P_(b+1)
  int b = 0;
  long long Pb = 0;
  {
    unsigned long long hit = __ballot(sp_all.np0 > 0 && (long long)(sp_all.incl0 - sp_all.np0) * U <= p &&
                                      p < (long long)sp_all.incl0 * U);
    if (hit) {
      const int l = __ffsll(static_cast<long long>(hit)) - 1;
      b = uni(l);
      Pb = uni(__shfl(sp_all.incl0 - sp_all.np0, l));
    } else {
      long long carry = __shfl(sp_all.incl0, spec::kWave - 1);
      for (int c0 = spec::kWave; c0 < B; c0 += spec::kWave) {
        const int np = c0 + lane < B
                           ? seq_span(ctx_lens[min(c0 + lane, B - 1)], K1, window, max_pages).np
                           : 0;
        const int incl = wave_incl_scan(np, lane);
        const long long lo = (carry + incl - np) * U, hi = (carry + incl) * U;
        hit = __ballot(np > 0 && lo <= p && p < hi);
        if (hit) {
          const int l = __ffsll(static_cast<long long>(hit)) - 1;
          b = uni(c0 + l);
          Pb = uni64(carry + __shfl(incl - np, l));
          break;
        }
        carry += __shfl(incl, spec::kWave - 1);
      }
    }
  }
  Span sp = seq_span(ctx_of(ctx_lens, sp_all, b), K1, window, max_pages);
  if (sp.np == 0) return;   // no sequence holds p: cannot happen for consistent inputs
  const long long off0 = p - Pb * U;
  int j = uni((int)div_nn(off0, sp.np));
  int o = uni((int)(off0 - (long long)j * sp.np));

  while (true) {
    const int take = (int)min((long long)(sp.np - o), pend - p);
    if (take <= 0) break;   // cannot happen for consistent inputs; keeps every wave finite
    const int g = j / nrc, rc = j - (j / nrc) * nrc;
    const int pg_begin = sp.p0 + o;
    const int npg = take;
    const int rr0 = rc * kRowsWG;
    const int nr = min(kRowsWG, GK1 - rr0);
    const long long piece = (long long)w + (long long)b * U + j;

    if constexpr (S::kQuarter) {
      unit_quarter<D, RT>(reinterpret_cast<const uint16_t *>(q), reinterpret_cast<const uint16_t *>(kpool),
                       reinterpret_cast<const uint16_t *>(vpool), table, pid_sh,
                       reinterpret_cast<f32x4_t *>(smem), part_ml, part_acc, b, K1, Hq, Hkv,
                       num_pages, max_pages, window, qscale, g, G, rr0, nr, pg_begin, npg, piece,
                       rstride, sp.ctx);
    } else {
    // (1) page ids of the piece, then the queries.  Loads are unconditional with clamped
    // indices so the wait counts the compiler inserts stay exact.
    const int pid_reg = table[(size_t)b * max_pages + pg_begin + min(tid, npg - 1)];
    u32x4_t qraw[S::kQPT];
#pragma unroll
    for (int x = 0; x < S::kQPT; ++x) {
      const int e = min(tid + x * kThreads, nr * S::kGPR - 1);
      const int r = e / S::kGPR, gi = e - r * S::kGPR;
      const int rr = rr0 + r, i = rr / G, h = g * G + (rr - i * G);
      qraw[x] = *reinterpret_cast<const u32x4_t *>(q + (((size_t)b * K1 + i) * Hq + h) * D + gi * S::kEPG);
    }
    if (tid < npg) pid_sh[tid] = (pid_reg >= 0 && pid_reg < num_pages) ? pid_reg : -1;
    __syncthreads();

    // (2) K/V of pages 0 and 1 in flight while the queries land in LDS (rows >= nr zero)
    u32x4_t ka[S::kGPT], va[S::kGPT], kb[S::kGPT], vb[S::kGPT];
    // A fetch past the piece reads the pools' first 16 bytes in every lane (an L1 hit after
    // the first), so the loads stay unconditional without costing a trip to memory.
    auto fetch = [&](u32x4_t(&kr)[S::kGPT], u32x4_t(&vr)[S::kGPT], int i) __attribute__((always_inline)) {
      const bool real = i < npg;
      const int pid = pid_sh[min(i, npg - 1)];
      const size_t off = real ? ((size_t)(pid < 0 ? 0 : pid) * Hkv + g) * kPage * D : 0;
#pragma unroll
      for (int x = 0; x < S::kGPT; ++x) {
        const int e = real ? min(tid + x * kThreads, S::kTileG - 1) : 0;
        kr[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(kpool + off + e * S::kEPG));
        vr[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(vpool + off + e * S::kEPG));
      }
    };
    auto stage = [&](const u32x4_t(&kr)[S::kGPT], const u32x4_t(&vr)[S::kGPT]) __attribute__((always_inline)) {
#pragma unroll
      for (int x = 0; x < S::kGPT; ++x) {
        const int e = tid + x * kThreads;
        if (S::kTileG % kThreads == 0 || e < S::kTileG) {   // static except at D = 64
          const int row = e / S::kGPR, gi = e - row * S::kGPR;
          *reinterpret_cast<u32x4_t *>(ks + row * S::kStr + gi * S::kEPG) = kr[x];
          *reinterpret_cast<u32x4_t *>(vs + row * S::kStr + gi * S::kEPG) = vr[x];
        }
      }
    };
    fetch(ka, va, 0);
    fetch(kb, vb, 1);
#pragma unroll
    for (int x = 0; x < S::kQPT; ++x) {
      const int e = tid + x * kThreads;
      if ((kRowsWG * S::kGPR) % kThreads == 0 || e < kRowsWG * S::kGPR) {
        const int r = e / S::kGPR, gi = e - r * S::kGPR;
        *reinterpret_cast<u32x4_t *>(qs + r * S::kStr + gi * S::kEPG) =
            e < nr * S::kGPR ? qraw[x] : u32x4_t{0u, 0u, 0u, 0u};
      }
    }

    // per-lane rows: rt * 16 + lr; their query positions and running (max, sum)
    int trow[RT];
    float m_run[RT], l_run[RT];
    f32x4_t acc[RT][S::kDTW];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = rt * 16 + lr;
      trow[rt] = r < nr ? sp.ctx - K1 + (rr0 + r) / G : -1;
      m_run[rt] = -INFINITY;
      l_run[rt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < S::kDTW; ++dt) acc[rt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const bool two_tiles = nr > 16;   // uniform

    // one page of the piece, already in LDS
    auto page = [&](int i) __attribute__((always_inline)) {
      if (pid_sh[i] < 0) return;       // uniform: an invalid page id hides its keys
      const int pg = pg_begin + i;
      // scores S^T[key 4*lq + e][row rt*16 + lr]
      f32x4_t scs[RT];
      if constexpr (S::kSplit) {
        // this wave's quarter of the head dim, then the four quarters summed in wave order
        constexpr int DQ = D / kWaves;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          f32x4_t part = {0.f, 0.f, 0.f, 0.f};
          if (rt == 0 || two_tiles) {
#pragma unroll
            for (int d0 = 0; d0 < DQ; d0 += M::kStepQK)
              part = M::qk(ks + lr * S::kStr + wave * DQ + d0,
                           qs + (rt * 16 + lr) * S::kStr + wave * DQ + d0, lq, part);
          }
          sred[(wave * RT + rt) * 64 + lane] = part;
        }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          f32x4_t t = sred[rt * 64 + lane];
#pragma unroll
          for (int w2 = 1; w2 < kWaves; ++w2) t += sred[(w2 * RT + rt) * 64 + lane];
          scs[rt] = t;
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          scs[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (rt == 1 && !two_tiles) break;
#pragma unroll
          for (int d0 = 0; d0 < D; d0 += M::kStepQK)
            scs[rt] = M::qk(ks + lr * S::kStr + d0, qs + (rt * 16 + lr) * S::kStr + d0, lq, scs[rt]);
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (rt == 1 && !two_tiles) break;
        const f32x4_t sc = scs[rt];
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
          acc[rt][dt] *= alpha;
          acc[rt][dt] = M::pv(vs, S::kStr, (wave * S::kDTW + dt) * 16 + lr, lq, pr, acc[rt][dt]);
        }
      }
    };

    // Both halves always stage and fetch (an exit between them would reach the next stage on
    // a path without the second half's loads, and its wait would then have to drain
    // everything).
    for (int i = 0; i < npg; i += 2) {
      stage(ka, va);
      fetch(ka, va, i + 2);
      __syncthreads();
      page(i);
      __syncthreads();
      stage(kb, vb);
      fetch(kb, vb, i + 3);
      __syncthreads();
      if (i + 1 < npg) page(i + 1);
      __syncthreads();
    }

    // the piece's partial: lane holds O^T[d = dtile*16 + 4*lq + e][row rt*16 + lr].  The
    // outputs leave with nontemporal stores of whole 128-byte lines (the merge reads them once,
    // from another CU): lanes lr and lr ^ 8 swap one of each pair of dim tiles (DPP row_ror:8),
    // so the first store of a pair writes rows 0..7 and the second rows 8..15, each row's two
    // tiles side by side.  At the batch-8 sliding layers this took the call (partial + merge)
    // from 24.0 to 22.6 us on MI355X; cached stores leave the partials for the write-back at
    // the kernel's end, and nontemporal 64-byte halves gained only 1.1 us.
    const size_t base = (size_t)piece * rstride;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = rt * 16 + lr;
      if (r < nr) {
        if (wave == 0 && lq == 0) part_ml[base + r] = make_float2(m_run[rt], l_run[rt]);
      }
      if constexpr (S::kDTW % 2 == 0) {   // uniform: every lane takes part in the swaps
        const bool lo = lr < 8;
#pragma unroll
        for (int dt = 0; dt < S::kDTW; dt += 2) {
          const f32x4_t x0 = acc[rt][dt], x1 = acc[rt][dt + 1];
          f32x4_t p0, p1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p0[e] = spec::dpp_move<0x128>(x0[e]);
            p1[e] = spec::dpp_move<0x128>(x1[e]);
          }
          const int d = (wave * S::kDTW + dt + (lo ? 0 : 1)) * 16 + 4 * lq;
          const int rA = lo ? r : r - 8, rB = lo ? r + 8 : r;
          if (rA < nr)
            __builtin_nontemporal_store(lo ? x0 : p1,
                                        reinterpret_cast<f32x4_t *>(part_acc + (base + rA) * D + d));
          if (rB < nr)
            __builtin_nontemporal_store(lo ? p0 : x1,
                                        reinterpret_cast<f32x4_t *>(part_acc + (base + rB) * D + d));
        }
      } else if (r < nr) {
#pragma unroll
        for (int dt = 0; dt < S::kDTW; ++dt) {
          const int d = (wave * S::kDTW + dt) * 16 + 4 * lq;
          __builtin_nontemporal_store(acc[rt][dt],
                                      reinterpret_cast<f32x4_t *>(part_acc + (base + r) * D + d));
        }
      }
    }
    }   // the staged path

    p += take;
    if (p >= pend) break;
    o = 0;
    if (++j == U) {   // next sequence with visible pages
      j = 0;
      bool more = false;
      while (b + 1 < B) {
        ++b;
        sp = seq_span(ctx_of(ctx_lens, sp_all, b), K1, window, max_pages);
        if (sp.np > 0) { more = true; break; }
      }
      if (!more) break;   // items left but no sequence: cannot happen for consistent inputs
    }
  }
}

// Grid: B * K1 * Hq workgroups of CW waves, one per output row (b, i, h).  Every wave finds
// the row's pieces (the same plan as the partial kernel) and their common maximum; wave v then
// sums the weighted partial outputs of pieces v, v + CW, ..., D / 64 columns per lane, with
// the loads of up to kBatch pieces issued together, and one LDS exchange adds the waves' sums.
// CW = 8 when units have many pieces (few long sequences), 2 when they have a handful (many
// sequences), so that all rows' workgroups are resident at once.
// Pieces per unit (about nwg / units, plus the two boundary pieces) up to which two waves
// merge a row.
constexpr int kCombFewPieces = 16;

template <int D, int CW>
__global__ __launch_bounds__(CW * 64) void attn_combine(
    const float2 *__restrict__ part_ml, const float *__restrict__ part_acc,
    const int32_t *__restrict__ ctx_lens, float *__restrict__ out, int B, int K1, int Hq, int Hkv,
    int max_pages, int window, int nwg, int c_floor, int GK1, int rows_wg) {
  constexpr int NC = D / spec::kWave;                 // columns per lane
  constexpr int kBatch = NC >= 8 ? 8 : 64 / NC > 16 ? 16 : 64 / NC;
  typedef float vecc_t __attribute__((ext_vector_type(NC)));
  __shared__ __align__(16) float red_acc[CW - 1][D];
  __shared__ float red_l[CW];
  const int tid = threadIdx.x, lane = tid & (spec::kWave - 1), wave = tid / spec::kWave;
  const long long row = blockIdx.x;
  const int h = (int)(row % Hq), i = (int)((row / Hq) % K1), b = (int)(row / ((long long)Hq * K1));
  const int G = Hq / Hkv, g = h / G, rr = i * G + (h - g * G);
  const int nrc = (GK1 + rows_wg - 1) / rows_wg, U = Hkv * nrc;
  const int rc = rr / rows_wg, r = rr - rc * rows_wg;
  const int rstride = min(GK1, rows_wg);
  float *o = out + row * D + lane * NC;

  const StreamPlan pl = stream_plan(ctx_lens, B, K1, window, max_pages, U, nwg, c_floor, lane);
  const long long Pb = pages_before(ctx_lens, pl, b, K1, window, max_pages, lane);
  const Span sp = seq_span(ctx_of(ctx_lens, pl, b), K1, window, max_pages);
  if (sp.np == 0) {   // uniform over the workgroup
    if (wave == 0) *reinterpret_cast<vecc_t *>(o) = vecc_t(0.f);
    return;
  }
  const int j = g * nrc + rc;
  const long long start = Pb * U + (long long)j * sp.np;
  const long long w0 = div_nn(start, pl.C), w1 = div_nn(start + sp.np - 1, pl.C);
  const int n = (int)(w1 - w0 + 1);
  const long long piece0 = w0 + (long long)b * U + j;
  const float2 *mlp = part_ml + (size_t)piece0 * rstride + r;
  const float *ap = part_acc + ((size_t)piece0 * rstride + r) * D + lane * NC;
  const size_t astep = (size_t)rstride * D;
  const int nmine = n > wave ? (n - wave + CW - 1) / CW : 0;   // pieces wave, wave + CW, ..

  // this wave's first batch of partial outputs is in flight while the maximum is reduced
  vecc_t v[kBatch];
#pragma unroll
  for (int t = 0; t < kBatch; ++t)
    v[t] = *reinterpret_cast<const vecc_t *>(ap + (size_t)min(wave + CW * t, n - 1) * astep);
  float mx = -INFINITY;
  for (int c0 = 0; c0 < n; c0 += spec::kWave) {
    const float2 x = mlp[(size_t)min(c0 + lane, n - 1) * rstride];
    if (c0 + lane < n) mx = fmaxf(mx, x.x);
  }
  const float m = spec::wave_max(mx);

  // weights of this wave's pieces: lane t of a round holds piece wave + CW * (t0 + t)
  vecc_t a = vecc_t(0.f);
  float l = 0.f;
  for (int t0 = 0; t0 < nmine; t0 += spec::kWave) {
    const int k = wave + CW * min(t0 + lane, nmine - 1);
    const float2 x = mlp[(size_t)k * rstride];
    const float wk = (t0 + lane < nmine && x.x != -INFINITY) ? exp2f(x.x - m) : 0.f;
    l += wk * x.y;
    const int cnt = min(spec::kWave, nmine - t0);
    for (int u0 = 0; u0 < cnt; u0 += kBatch) {
      if (t0 + u0 > 0) {
#pragma unroll
        for (int t = 0; t < kBatch; ++t)
          v[t] = *reinterpret_cast<const vecc_t *>(
              ap + (size_t)(wave + CW * min(t0 + u0 + t, nmine - 1)) * astep);
      }
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const float wt = __shfl(wk, u0 + t);
        if (u0 + t < cnt) a += wt * v[t];
      }
    }
  }
  l = spec::wave_sum(l);
  if (wave > 0) {
    *reinterpret_cast<vecc_t *>(&red_acc[wave - 1][lane * NC]) = a;
    if (lane == 0) red_l[wave] = l;
  }
  __syncthreads();
  if (wave == 0) {
    float L = l;
#pragma unroll
    for (int x = 0; x < CW - 1; ++x) {
      a += *reinterpret_cast<const vecc_t *>(&red_acc[x][lane * NC]);
      L += red_l[x + 1];
    }
    *reinterpret_cast<vecc_t *>(o) = L > 0.f ? a / L : vecc_t(0.f);
  }
}

struct AttnPlan {
  int GK1, rt, rows_wg, nwg, c_floor;
  size_t off_ml, off_acc, bytes;
};

template <int D, typename T, int RT>
int waves_per_eu() { return AttnShape<D, T, RT>::kWavesPerEU; }

int slots_per_cu(int D, bool bf16, int rt) {
#define SLOT_CASE(DD)                                                                           \
  if (D == DD)                                                                                 \
    return bf16 ? (rt == 1 ? waves_per_eu<DD, uint16_t, 1>() : waves_per_eu<DD, uint16_t, 2>()) \
                : (rt == 1 ? waves_per_eu<DD, float, 1>() : waves_per_eu<DD, float, 2>());
  SLOT_CASE(64) SLOT_CASE(128) SLOT_CASE(256) SLOT_CASE(512)
#undef SLOT_CASE
  return 1;
}

AttnPlan plan(int B, int K1, int Hq, int Hkv, int D, int max_pages, int window, bool bf16) {
  AttnPlan pl;
  pl.GK1 = (Hq / Hkv) * K1;
  pl.rt = pl.GK1 <= 16 ? 1 : 2;
  pl.rows_wg = 16 * pl.rt;
  const int nrc = spec::ceil_div(pl.GK1, pl.rows_wg);
  int span = max_pages;
  if (window > 0) span = min(max_pages, spec::ceil_div(window + K1 - 1, kPage) + 1);
  span = max(span, 1);
  const long long units = (long long)B * Hkv * nrc;
  const long long upper = units * span;                 // items, at most
  const long long slots = (long long)spec::device_cus() * slots_per_cu(D, bf16, pl.rt);
  long long nwg = max(slots, (upper + kMaxPagesPerPiece - 1) / kMaxPagesPerPiece);
  nwg = max(1LL, min(nwg, upper));
  pl.nwg = (int)nwg;
  // pieces of one unit stay within kMaxPiecesPerUnit: np / C + 2 <= kMaxPiecesPerUnit
  pl.c_floor = max(1, spec::ceil_div(max_pages, kMaxPiecesPerUnit - 2));
  const size_t pieces = (size_t)nwg + (size_t)units;
  const size_t rows = pieces * (size_t)min(pl.GK1, pl.rows_wg);
  pl.off_ml = 0;
  pl.off_acc = spec::align_up(rows * sizeof(float2), 256);
  pl.bytes = pl.off_acc + spec::align_up(rows * D * sizeof(float), 256);
  return pl;
}

template <int D, typename T, int RT>
int launch_partial(const void *q, const void *kp, const void *vp, const int32_t *table,
                   const int32_t *ctx, int B, int K1, int Hq, int Hkv, int num_pages,
                   int max_pages, int window, float scale, const AttnPlan &pl, float2 *ml,
                   float *acc, hipStream_t st) {
  using S = AttnShape<D, T, RT>;
  static std::atomic<uint64_t> lds_set{0};   // per instantiation: one bit per device
  const int rc = spec::ensure_dynamic_lds(reinterpret_cast<const void *>(&attn_partial<D, T, RT>),
                                          S::kLds, lds_set, "spec_verify_attn");
  if (rc != SPEC_OK) return rc;
  hipLaunchKernelGGL((attn_partial<D, T, RT>), dim3(pl.nwg), dim3(kThreads), S::kLds, st,
                     static_cast<const T *>(q), static_cast<const T *>(kp),
                     static_cast<const T *>(vp), table, ctx, ml, acc, B, K1, Hq, Hkv, num_pages,
                     max_pages, window, scale * kLog2e, pl.nwg, pl.c_floor, pl.GK1);
  return spec::launched("attn_partial");
}

template <int D, typename T>
int launch(const void *q, const void *kp, const void *vp, const int32_t *table,
           const int32_t *ctx, float *out, int B, int K1, int Hq, int Hkv, int num_pages,
           int max_pages, int window, float scale, const AttnPlan &pl, char *ws,
           hipStream_t st) {
  float2 *ml = reinterpret_cast<float2 *>(ws + pl.off_ml);
  float *acc = reinterpret_cast<float *>(ws + pl.off_acc);
  int rc = pl.rt == 1
               ? launch_partial<D, T, 1>(q, kp, vp, table, ctx, B, K1, Hq, Hkv, num_pages,
                                         max_pages, window, scale, pl, ml, acc, st)
               : launch_partial<D, T, 2>(q, kp, vp, table, ctx, B, K1, Hq, Hkv, num_pages,
                                         max_pages, window, scale, pl, ml, acc, st);
  if (rc != SPEC_OK) return rc;
  const long long rows = (long long)B * K1 * Hq;
  const long long units = (long long)B * Hkv * spec::ceil_div(pl.GK1, pl.rows_wg);
  if (pl.nwg / units + 2 <= kCombFewPieces) {
    hipLaunchKernelGGL((attn_combine<D, 2>), dim3((unsigned)rows), dim3(2 * 64), 0, st, ml, acc,
                       ctx, out, B, K1, Hq, Hkv, max_pages, window, pl.nwg, pl.c_floor, pl.GK1,
                       pl.rows_wg);
  } else {
    hipLaunchKernelGGL((attn_combine<D, 8>), dim3((unsigned)rows), dim3(8 * 64), 0, st, ml, acc,
                       ctx, out, B, K1, Hq, Hkv, max_pages, window, pl.nwg, pl.c_floor, pl.GK1,
                       pl.rows_wg);
  }
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
  SPEC_REQUIRE((long long)B * K1 * Hq <= 0x7fffffffLL, SPEC_EUNSUPPORTED,
               "spec_verify_attn: B*K1*Hq output rows exceed one grid");
  SPEC_REQUIRE(D == 64 || D == 128 || D == 256 || D == 512, SPEC_EUNSUPPORTED,
               "spec_verify_attn: head dim %d not in {64, 128, 256, 512}", D);
  SPEC_REQUIRE(page_size == kPage, SPEC_EUNSUPPORTED, "spec_verify_attn: page_size=%d, only 16", page_size);
  SPEC_REQUIRE((long)max_pages <= (long)(kMaxPiecesPerUnit - 2) * kMaxPagesPerPiece, SPEC_EUNSUPPORTED,
               "spec_verify_attn: max_pages_per_seq=%d exceeds %d", max_pages,
               (kMaxPiecesPerUnit - 2) * kMaxPagesPerPiece);
  return SPEC_OK;
}

}  // namespace

extern "C" size_t spec_verify_attn_workspace(int B, int K1, int Hq, int Hkv, int D,
                                             int page_size, int max_pages_per_seq, int window) {
  spec::clear_error();
  if (check_shape(B, K1, Hq, Hkv, D, page_size, max_pages_per_seq, window) != SPEC_OK) return 0;
  // the grid (and with it the workspace) depends on the element type; size for either
  return max(plan(B, K1, Hq, Hkv, D, max_pages_per_seq, window, true).bytes,
             plan(B, K1, Hq, Hkv, D, max_pages_per_seq, window, false).bytes);
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
  const AttnPlan pl = plan(B, K1, Hq, Hkv, D, max_pages_per_seq, window, dtype == SPEC_BF16);
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
