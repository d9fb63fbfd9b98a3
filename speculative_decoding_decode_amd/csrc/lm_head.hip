// lm-head of the verify step: logits = hidden W^T for the R = B*K1 verify rows, and the
// target's row distributions p = softmax(logits / T).
//
// The pages single out this contraction: with a 256k vocabulary the final logit projection is
// a major cost (butteryoon "Gemma 4 MTP 서빙 가이드 해설", section 1; damoang's text of the
// MTP announcement, drafter internals section), and decoding is bound by streaming weights
// from memory (same guide, introduction).  At R = 3..96 rows the kernel is a stream over the
// V x H table: every table element is read once from HBM and used R times.
//
// Design (gfx950).  Two contraction kernels share one softmax finalize; which one runs was
// set by timing both on MI355X at 1..8 rows and two table widths:
//  * up to 5 rows (batch-1 verification): a bandwidth-bound GEMV.  Each wave owns 64 table
//    rows and walks the hidden dimension in 128-byte chunks, eight rows per load instruction,
//    with nontemporal loads (the table is used once per call); every lane accumulates its slot
//    of eight rows in fp32 with v_dot2_f32_bf16 (fp32 tables: FMAs) and a three-step DPP
//    reduction inside each 8-lane group gives each row's logit; wave priorities that fall with
//    each wave's progress keep a CU's workgroups level.  About 6.7 TB/s in the step.
//  * every other R: MFMA (v_mfma_f32_16x16x32_bf16; fp32 tables: four v_mfma_f32_16x16x4_f32).
//    One workgroup = 512 vocab rows against up to 96 hidden rows per pass; chunks of 128 bytes
//    of every row are loaded as 128-byte contiguous runs per row and transposed into MFMA
//    fragments through bank-conflict-free LDS tiles; p leaves with nontemporal stores.
//  * Every epilogue turns a 256-row vocab block into per-block softmax statistics (max, sum of
//    exp, first argmax) and writes exp(logit - block max) into p; lm_head_finalize merges the
//    statistics of all blocks and rescales p in place (or writes the greedy one-hot rows).
#include <math.h>

#include <mutex>

#include "common.hpp"
#include "softmax_stats.hpp"

namespace {

using spec::kWave;
using spec::wave_argmax;
using spec::wave_sum;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));   // one 16-byte slot

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;          // 4
constexpr int kBlockRows = 256;                   // vocab rows per statistics block
constexpr int kFinChunk = 4096;                   // vocab entries per finalize workgroup
constexpr long kFinWideWGs = 2048;                // above this many, 4x larger chunks
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxRows = 65535;                   // rows per call (grid y of the finalize)

template <typename T> struct Mma;
template <> struct Mma<uint16_t> {  // bf16 table: one 16x16x32 MFMA per 16-byte fragment
  static constexpr int kEPL = 8;             // elements per lane per fragment
  static constexpr int kStep = 4 * kEPL;     // hidden elements per K-step (4 lane groups)
  __device__ static __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {  // fp32 table: four 16x16x4 MFMAs, one per fragment element
  static constexpr int kEPL = 4;
  static constexpr int kStep = 4 * kEPL;
  __device__ static __forceinline__ f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[1]), __uint_as_float(b[1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[2]), __uint_as_float(b[2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[3]), __uint_as_float(b[3]), c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ u32x4_t load_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

__device__ __forceinline__ bool better(float m, int a, float om, int oa) {
  return spec::first_max_better(m, a, om, oa);
}

// Contraction + per-block statistics for every R the GEMV does not take.  512 threads, two
// waves per SIMD; a workgroup owns 512 vocab rows (two statistics blocks) and NH <= 6 tiles of
// 16 hidden rows.
// Grid: (ceil(V / 512), ceil(R / (16 NH))).  Wave w multiplies vocab rows 64 w + [0, 64) of the
// workgroup (four MFMA tiles, the A operand) by all NH hidden-row tiles (the B operand).  The
// workgroup walks the hidden dimension in chunks of 128 bytes of every row.
//  * Loads: 8 consecutive lanes read the 128 bytes of one row, so each instruction takes 128
//    contiguous bytes from each of 8 rows (table loads nontemporal: it is read once per call).
//    MFMA fragments need one row per lane instead, so every chunk (512 table rows and 16 NH
//    hidden rows) passes through LDS: rows 128 bytes apart with the 16-byte slots XOR-swizzled
//    by row pair, so neither the writes nor the fragment reads conflict on a bank.  The hidden
//    rows are re-read for every chunk by every workgroup, so the workgroup is made as tall as
//    the LDS allows (their bytes per table byte are 16 NH / 512).
//  * Pipeline: per chunk, one workgroup barrier, the multiplies of chunk c out of one LDS
//    buffer, then chunk c + 1 (loaded into registers during chunk c - 1) is written to the
//    other buffer and the registers refilled with chunk c + 2.  (Two chunks in registers were
//    measured 1-2% slower.)  Fetches past the last chunk read one shared address; slots past H
//    are zeroed on both operands when they are written to LDS.
// Accumulator lane l of tile (vt, n) holds the logits of vocab rows 16 vt + 4 (l / 16) + e
// (e = 0..3) of the wave's 64 for hidden row 16 n + l % 16.
constexpr int kMmaThreads = 512;
constexpr int kMmaWaves = kMmaThreads / kWave;                // 8
constexpr int kMmaRowsW = 64;                                 // vocab rows per wave
constexpr int kMmaVT = kMmaRowsW / 16;                        // 4 vocab tiles per wave
constexpr int kMmaRows = kMmaWaves * kMmaRowsW;               // 512 vocab rows per workgroup
constexpr int kMmaSlots = 8;                                  // 16-byte slots per row per chunk
constexpr int kMmaWL = kMmaRows * kMmaSlots / kMmaThreads;    // 8 table loads per thread per chunk
constexpr int kMmaWBuf = kMmaRows * kMmaSlots * 16;           // 64 KB: one chunk of the table rows
constexpr int kMaxNH = 6;                                     // hidden-row tiles per pass

template <int NH>
struct MmaShape {
  static constexpr int kXBuf = NH * 16 * kMmaSlots * 16;      // one chunk of the hidden rows
  static constexpr size_t kLds = 2 * (size_t)(kMmaWBuf + kXBuf);
  static_assert(kMmaRows % kBlockRows == 0 && NH <= kMaxNH, "workgroup = whole statistics blocks");
};

__device__ __forceinline__ u32x4_t mask16(u32x4_t v, bool keep) {
  const uint32_t m = keep ? 0xffffffffu : 0u;
  return u32x4_t{v[0] & m, v[1] & m, v[2] & m, v[3] & m};
}

// Byte offset of 16-byte slot `slot` of row `row` in a [rows][8 slots] LDS tile.
__device__ __forceinline__ int swz(int row, int slot) { return row * 128 + ((slot ^ (row >> 1)) & 7) * 16; }

// Epilogue of the MFMA contractions: per 256-row statistics block and hidden row, the block
// max / first argmax and the sum of exp, written to `so`; exp((z - block max) / T) into p (the
// finalize rescales it); logits stored when asked for.  The p and logit stores are nontemporal
// and issued as soon as each tile (pair) is done, so they drain while the sums are reduced:
// every workgroup of a round reaches its epilogue at about the same time, and stores that
// allocate in the cache took about 15 us longer per call at 40-48 rows on MI355X (p is read
// once, by the finalize or the accept, after the whole table has streamed past the cache).
// acc[vt][n]: lane l holds the logits of vocab rows vw + 16 vt + 4 (l / 16) + e for hidden row
// r0 + 16 n + l % 16.  smem: at least 3 * kMmaWaves * kMaxNH * 16 words of LDS no longer in use.
template <int NH>
__device__ __forceinline__ void mfma_epilogue(f32x4_t (&acc)[kMmaVT][NH], unsigned char *smem,
                                              int wave, int lr, int lq, int vb, int vw, int r0,
                                              const float *__restrict__ temp,
                                              float *__restrict__ logits, float *__restrict__ probs,
                                              const spec::StatsOut &so, int R, int V) {
  // block max / first argmax, then sum of exp, per hidden row.  Hidden row
  // slot c = n * 16 + lr of the wave is row r0 + 16 n + lr; the four 64-row slices
  // of a statistics block (waves g0 + q) are merged in slice order.
  static_assert(kMmaVT % 2 == 0, "p is stored by pairs of vocab tiles");
  const int g0 = wave & ~3;                     // first wave of this wave's block
  typedef float RowF[kMaxNH * 16];
  typedef int RowI[kMaxNH * 16];
  RowF *red_m = reinterpret_cast<RowF *>(smem);
  RowF *red_s = red_m + kMmaWaves;
  RowI *red_i = reinterpret_cast<RowI *>(red_s + kMmaWaves);
  const int sb = vb / kBlockRows + wave / 4;    // statistics block
#pragma unroll
  for (int n = 0; n < NH; ++n) {
    float mx = -INFINITY;
    int ax = 0x7fffffff;
#pragma unroll
    for (int vt = 0; vt < kMmaVT; ++vt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {   // increasing v within the lane: the first maximum stays
        const int v = vw + vt * 16 + lq * 4 + e;
        const float z = acc[vt][n][e];
        if (v < V && z > mx) { mx = z; ax = v; }
      }
#pragma unroll
    for (int off = 16; off < kWave; off <<= 1) {
      const float om = __shfl_xor(mx, off);
      const int oa = __shfl_xor(ax, off);
      if (better(mx, ax, om, oa)) { mx = om; ax = oa; }
    }
    if (lq == 0) { red_m[wave][n * 16 + lr] = mx; red_i[wave][n * 16 + lr] = ax; }
  }
  __syncthreads();
  float cexp[NH];
  bool live[NH];
#pragma unroll
  for (int n = 0; n < NH; ++n) {
    const int c = n * 16 + lr;
    float m = red_m[g0][c];
#pragma unroll
    for (int q = 1; q < 4; ++q) m = fmaxf(m, red_m[g0 + q][c]);
    const int r = r0 + n * 16 + lr;
    live[n] = r < R;
    const float tr = live[n] ? temp[r] : 1.f;
    cexp[n] = tr > 0.f ? kLog2e / tr : 0.f;   // 0: greedy row, p is written by the finalize
    float sacc = 0.f;
#pragma unroll
    for (int vt = 0; vt < kMmaVT; ++vt) {
      const int v0 = vw + vt * 16 + lq * 4;
      if (live[n] && logits != nullptr) {
        float *dst = logits + (size_t)r * V + v0;
        if (v0 + 3 < V && (V & 3) == 0) {
          __builtin_nontemporal_store(acc[vt][n], reinterpret_cast<f32x4_t *>(dst));
        } else {
          for (int e = 0; e < 4; ++e)
            if (v0 + e < V) __builtin_nontemporal_store(acc[vt][n][e], dst + e);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ex = (v0 + e < V) ? exp2f((acc[vt][n][e] - m) * cexp[n]) : 0.f;
        acc[vt][n][e] = ex;
        sacc += ex;
      }
      if (vt & 1) {
        // p of tiles vt - 1 and vt (32 entries, one 128-byte line of each of the 16 rows) in two
        // stores of whole lines: lanes lr and lr ^ 8 swap one tile (DPP row_ror:8), so that
        // the first store writes rows 0..7 and the second rows 8..15 of the tile pair.  Stores
        // of the 64-byte halves, one per tile, reached HBM as 1.4x the bytes written.
        const bool lo = lr < 8;
        const f32x4_t a = acc[vt - 1][n], b = acc[vt][n];
        f32x4_t pa, pb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pa[e] = spec::dpp_move<0x128>(a[e]);
          pb[e] = spec::dpp_move<0x128>(b[e]);
        }
        const int wo = (live[n] && cexp[n] != 0.f) ? 1 : 0;
        const int wp = spec::dpp_move<0x128>(wo);
        const int col = v0 - 16 + (lo ? 0 : 16);
        auto put = [&](int row, const f32x4_t &x, bool ok) __attribute__((always_inline)) {
          if (!ok) return;
          float *dst = probs + (size_t)row * V + col;
          if (col + 3 < V && (V & 3) == 0) {
            __builtin_nontemporal_store(x, reinterpret_cast<f32x4_t *>(dst));
          } else {
            for (int e = 0; e < 4; ++e)
              if (col + e < V) __builtin_nontemporal_store(x[e], dst + e);
          }
        };
        put(lo ? r : r - 8, lo ? a : pb, lo ? wo != 0 : wp != 0);
        put(lo ? r + 8 : r, lo ? pa : b, lo ? wp != 0 : wo != 0);
      }
    }
#pragma unroll
    for (int off = 16; off < kWave; off <<= 1) sacc += __shfl_xor(sacc, off);
    if (lq == 0) red_s[wave][c] = sacc;
  }
  __syncthreads();
  if ((wave & 3) == 0 && lq == 0 && sb * kBlockRows < V) {
#pragma unroll
    for (int n = 0; n < NH; ++n) {
      const int c = n * 16 + lr, r = r0 + n * 16 + lr;
      if (r >= R) continue;
      float m = red_m[g0][c];
      int a = red_i[g0][c];
#pragma unroll
      for (int q = 1; q < 4; ++q)
        if (better(m, a, red_m[g0 + q][c], red_i[g0 + q][c])) {
          m = red_m[g0 + q][c];
          a = red_i[g0 + q][c];
        }
      const float sum = ((red_s[g0][c] + red_s[g0 + 1][c]) + red_s[g0 + 2][c]) +
                        red_s[g0 + 3][c];
      so.stats[(size_t)sb * R + r] = make_float2(m, sum);
      so.amax[(size_t)sb * R + r] = a;
    }
  }
}

template <typename T, int NH>
__global__ __launch_bounds__(kMmaThreads, 1) void lm_head_mfma(
    const T *__restrict__ X, const T *__restrict__ W, const float *__restrict__ temp,
    float *__restrict__ logits, float *__restrict__ probs, spec::StatsOut so, int R, int H,
    int V) {
  using M = Mma<T>;
  using S = MmaShape<NH>;
  constexpr int NT = NH;
  constexpr int EPL = M::kEPL;                    // elements per 16-byte slot
  constexpr int KC = kMmaSlots * EPL;             // elements per chunk (two MFMA K-steps)
  constexpr int XS = NT * 16 * kMmaSlots;         // hidden-row slots per chunk
  constexpr int XL = (XS + kMmaThreads - 1) / kMmaThreads;   // of them per thread
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int lr = lane & 15, lq = lane >> 4;           // fragment row / K group
  const int ls = tid & 7;                             // load slot
  const int blk = blockIdx.x;
  const int r0 = blockIdx.y * NT * 16;
  const int vb = blk * kMmaRows;
  const int vw = vb + wave * kMmaRowsW;
  const int nch = (H + KC - 1) / KC;
  unsigned char *wl = smem;                             // [2][512 rows][128 B]
  unsigned char *xl = smem + 2 * (size_t)kMmaWBuf;      // [2][NH * 16 rows][128 B]

  struct Chunk {
    u32x4_t w[kMmaWL];
    u32x4_t x[XL];
  };
  auto fetch = [&](Chunk &ch, int c) __attribute__((always_inline)) {
    const size_t live = c < nch ? ~(size_t)0 : 0;   // uniform; past the end: offset 0
    const int kk = min(c * KC + ls * EPL, H - EPL);
#pragma unroll
    for (int i = 0; i < kMmaWL; ++i) {
      const size_t off = (size_t)min(vb + (tid + i * kMmaThreads) / kMmaSlots, V - 1) * H + kk;
      ch.w[i] = load_stream(W + (off & live));
    }
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int e = min(tid + j * kMmaThreads, XS - 1);
      const int row = min(r0 + e / kMmaSlots, R - 1);
      const size_t off = (size_t)row * H + min(c * KC + (e % kMmaSlots) * EPL, H - EPL);
      ch.x[j] = *reinterpret_cast<const u32x4_t *>(X + (off & live));
    }
  };
  // chunk c (the oldest in the ring) into LDS buffer c & 1; slots past H become zero
  auto stage = [&](const Chunk &ch, int c) __attribute__((always_inline)) {
    const int buf = c & 1;
    const bool in = c * KC + ls * EPL < H;
#pragma unroll
    for (int i = 0; i < kMmaWL; ++i)
      *reinterpret_cast<u32x4_t *>(wl + buf * kMmaWBuf + swz((tid + i * kMmaThreads) / kMmaSlots, ls)) =
          mask16(ch.w[i], in);
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int e = min(tid + j * kMmaThreads, XS - 1);   // duplicates write the same bytes
      *reinterpret_cast<u32x4_t *>(xl + buf * S::kXBuf + swz(e / kMmaSlots, e % kMmaSlots)) =
          mask16(ch.x[j], c * KC + (e % kMmaSlots) * EPL < H);
    }
  };
  f32x4_t acc[kMmaVT][NH];
#pragma unroll
  for (int vt = 0; vt < kMmaVT; ++vt)
#pragma unroll
    for (int n = 0; n < NH; ++n) acc[vt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int c) __attribute__((always_inline)) {
    const int buf = c & 1;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t a[kMmaVT], bx[NH];
#pragma unroll
      for (int vt = 0; vt < kMmaVT; ++vt)
        a[vt] = *reinterpret_cast<const u32x4_t *>(
            wl + buf * kMmaWBuf + swz(wave * kMmaRowsW + vt * 16 + lr, s * 4 + lq));
#pragma unroll
      for (int n = 0; n < NH; ++n)
        bx[n] = *reinterpret_cast<const u32x4_t *>(
            xl + buf * S::kXBuf + swz(n * 16 + lr, s * 4 + lq));
#pragma unroll
      for (int vt = 0; vt < kMmaVT; ++vt)
#pragma unroll
        for (int n = 0; n < NH; ++n) acc[vt][n] = M::run(a[vt], bx[n], acc[vt][n]);
    }
  };

  Chunk ring;
  fetch(ring, 0);
  stage(ring, 0);
  fetch(ring, 1);
  // Scheduling barriers keep each phase where it is written, so the wait before a stage is
  // for the chunk that stage writes and the next chunk's loads stay in flight.
  for (int c = 0; c < nch; ++c) {
    __syncthreads();          // chunk c is in LDS; every wave is done with chunk c - 1
    __builtin_amdgcn_sched_barrier(0);
    compute(c);
    __builtin_amdgcn_sched_barrier(0);
    stage(ring, c + 1);
    fetch(ring, c + 2);
    __builtin_amdgcn_sched_barrier(0);
  }

  __syncthreads();   // the chunk buffers are free: they hold the reduction arrays now
  mfma_epilogue<NH>(acc, smem, wave, lr, lq, vb, vw, r0, temp, logits, probs, so, R, V);
}

// ------------------------------------------------------------------------- small-R GEMV path
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Rows up to which the GEMV serves a call of hidden width H; above it the MFMA contraction
// streams faster.  The GEMV's time grows with every row (one more dot product per table
// element), the MFMA contraction's stays flat up to 16 rows.  Timed on MI355X inside the
// verify step's call at 1..8 rows and 2560 / 5376 wide, the GEMV is faster up to five rows at
// both widths (at 5376 wide the two tie at five and six rows) and the MFMA contraction from
// six.  A build may fix the limit (SPEC_GEMV_MAX_ROWS) to time one kernel against the other.
constexpr int kGemvMaxInstR = 8;     // GEMV instantiations: 1..8 rows
#ifdef SPEC_GEMV_MAX_ROWS
static_assert(SPEC_GEMV_MAX_ROWS >= 0 && SPEC_GEMV_MAX_ROWS <= kGemvMaxInstR,
              "GEMV rows within its instantiations");
constexpr int gemv_max_rows(int) { return SPEC_GEMV_MAX_ROWS; }
#else
constexpr int gemv_max_rows(int) { return 5; }
#endif
constexpr int kRowsPerWave = 64;     // one table row per lane in the epilogue

template <typename T> struct Dot;
template <> struct Dot<uint16_t> {
  static constexpr int kEPL = 8;
  __device__ static __forceinline__ float run(const uint4 &w, const uint4 &x, float s) {
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x.x), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x.w), s, false);
    return s;
  }
};
template <> struct Dot<float> {
  static constexpr int kEPL = 4;
  __device__ static __forceinline__ float run(const uint4 &w, const uint4 &x, float s) {
    s = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), s);
    s = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), s);
    s = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), s);
    s = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), s);
    return s;
  }
};

// GEMV epilogue: lane l holds the logits keep[r] of vocab row v0 + l.  Per 256-row block and
// hidden row: (max, sum of exp) and the first argmax into stats / amax; exp((z - block max) / T)
// into probs (the finalize rescales it); logits stored when asked for.
template <int RT>
__device__ __forceinline__ void gemv_epilogue(const float (&keep)[RT], int v0, int lane, int wave,
                                              int blk, const float *__restrict__ temp,
                                              float *__restrict__ logits, float *__restrict__ probs,
                                              const spec::StatsOut &so, int V) {
  __shared__ float red_m[kWaves][RT];
  __shared__ float red_s[kWaves][RT];
  __shared__ int red_i[kWaves][RT];
  const int v = v0 + lane;
  const bool vok = v < V;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    float mx = vok ? keep[r] : -INFINITY;
    int ax = vok ? v : 0x7fffffff;
    wave_argmax(mx, ax);
    if (lane == 0) { red_m[wave][r] = mx; red_i[wave][r] = ax; }
  }
  __syncthreads();
  float ex[RT];
  bool greedy[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    float m = red_m[0][r];
    for (int w2 = 1; w2 < kWaves; ++w2) m = fmaxf(m, red_m[w2][r]);
    const float tr = temp[r];
    greedy[r] = !(tr > 0.f);
    const float c = greedy[r] ? 0.f : kLog2e / tr;
    ex[r] = vok ? exp2f((keep[r] - m) * c) : 0.f;
    const float sw = wave_sum(ex[r]);
    if (lane == 0) red_s[wave][r] = sw;
    if (vok && logits != nullptr) logits[(size_t)r * V + v] = keep[r];
  }
  __syncthreads();
  if (wave == 0 && lane < RT) {
    const int r = lane;
    float m = red_m[0][r];
    int a = red_i[0][r];
    for (int w2 = 1; w2 < kWaves; ++w2)
      if (better(m, a, red_m[w2][r], red_i[w2][r])) { m = red_m[w2][r]; a = red_i[w2][r]; }
    const float sum = ((red_s[0][r] + red_s[1][r]) + red_s[2][r]) + red_s[3][r];
    so.stats[(size_t)blk * RT + r] = make_float2(m, sum);
    so.amax[(size_t)blk * RT + r] = a;
  }
#pragma unroll
  for (int r = 0; r < RT; ++r)
    if (vok && !greedy[r]) probs[(size_t)r * V + v] = ex[r];
}

// Grid: ceil(V / 256).  The GEMV for R <= gemv_max_rows(H) rows.  A wave owns 64 table rows and
// walks the hidden dimension in chunks of 128 bytes: one load instruction covers 8 rows x 128
// contiguous bytes (lane 8 g + s reads 16-byte slot s of row t + 8 g of the wave's 64, for
// load t = 0..7), so a chunk of the wave's 64 rows is eight nontemporal loads and the same
// 16-byte slot of the R hidden rows (read by every wave, cache-resident).  Every lane keeps
// 8 x R partial dot products (v_dot2_f32_bf16; fp32 tables: FMAs) across all chunks, so the
// only cross-lane work is one three-step DPP reduction inside each 8-lane group at the end
// (quad swaps and the half-row mirror), after which lane 8 g + t holds row t + 8 g's logits.
// Two chunks are in flight per wave; a fetch past the last chunk reads one valid 16-byte
// location, and slots past H are zeroed on both operands.  Registers grow by 16 VGPRs per row
// (97 at one row, 177 at six), so four, three or two workgroups fit per CU.
template <typename T, int RT>
__global__ __launch_bounds__(kThreads, RT <= 2 ? 4 : RT == 3 ? 3 : 2) void lm_head_gemv(
    const T *__restrict__ X, const T *__restrict__ W, const float *__restrict__ temp,
    float *__restrict__ logits, float *__restrict__ probs, spec::StatsOut so, int H, int V) {
  using Dt = Dot<T>;
  constexpr int EPL = Dt::kEPL;
  constexpr int CE = 8 * EPL;                       // elements per 128-byte chunk
  constexpr int kRowsPerLoad = 8;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane >> 3, sl = lane & 7;
  const int blk = blockIdx.x;
  const int v0 = blk * kBlockRows + wave * kRowsPerWave;
  // Element offsets from the wave's first row (below 64 H: 32 bits); rows past V are clamped
  // to the last row (their sums are never used).
  const T *wbase = W + (size_t)v0 * H;
  int off[kRowsPerLoad];
#pragma unroll
  for (int t = 0; t < kRowsPerLoad; ++t) off[t] = (min(v0 + t + 8 * g, V - 1) - v0) * H;
  const int off_end = (min(v0, V - 1) - v0) * H;    // the location read past the last chunk
  const int nch = (H + CE - 1) / CE;

  float acc[kRowsPerLoad][RT];
#pragma unroll
  for (int t = 0; t < kRowsPerLoad; ++t)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[t][r] = 0.f;
  struct Chunk {
    u32x4_t w[kRowsPerLoad];
    u32x4_t x[RT];
  };
  auto fetch = [&](Chunk &ch, int c) __attribute__((always_inline)) {
    const bool live = c < nch;   // uniform
    const int col = min(c * CE + sl * EPL, H - EPL);
#pragma unroll
    for (int t = 0; t < kRowsPerLoad; ++t)
      ch.w[t] = load_stream(wbase + (live ? off[t] + col : off_end));
#pragma unroll
    for (int r = 0; r < RT; ++r)
      ch.x[r] = *reinterpret_cast<const u32x4_t *>(X + (live ? r * H + col : 0));
  };
  auto compute = [&](const Chunk &ch, int c) __attribute__((always_inline)) {
    const bool in = c * CE + sl * EPL < H;           // false for every slot of a chunk past the end
    uint4 xv[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) xv[r] = __builtin_bit_cast(uint4, mask16(ch.x[r], in));
#pragma unroll
    for (int t = 0; t < kRowsPerLoad; ++t) {
      const uint4 wv = __builtin_bit_cast(uint4, mask16(ch.w[t], in));
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[t][r] = Dt::run(wv, xv[r], acc[t][r]);
    }
  };
  // The scheduling barriers keep each phase where it is written, so the wait before a compute
  // is for that chunk only and the other chunk's loads stay in flight.
  // Wave priority falls as the wave gets through its rows (3 for the first eighth of the
  // chunks, then 2, 1 from three eighths, 0 from five eighths).  The waves of a CU's three
  // workgroups otherwise share its issue slots oldest first: on MI355X the first-dispatched
  // workgroup of a CU finished its rows in 68 us, the second in 115, the third in 157, and the
  // workgroup started in the first one's place at ~70 us ran on with few neighbours to the end
  // of the call.  Letting the waves that are behind go first evens their progress out and
  // took the 3-row call at 2560 wide from 200.8 to 198.9 us.
  Chunk ca, cb;
  fetch(ca, 0);
  fetch(cb, 1);
  __builtin_amdgcn_s_setprio(3);
  const int q1 = nch / 8, q2 = 3 * nch / 8, q3 = 5 * nch / 8;
  for (int c = 0; c < nch; c += 2) {
    if (c == (q1 & ~1)) __builtin_amdgcn_s_setprio(2);
    if (c == (q2 & ~1)) __builtin_amdgcn_s_setprio(1);
    if (c == (q3 & ~1)) __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    compute(ca, c);
    __builtin_amdgcn_sched_barrier(0);
    fetch(ca, c + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(cb, c + 1);
    __builtin_amdgcn_sched_barrier(0);
    fetch(cb, c + 3);
  }
  float keep[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) keep[r] = 0.f;
#pragma unroll
  for (int t = 0; t < kRowsPerLoad; ++t)
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float v = acc[t][r];
      v += spec::dpp_move<0xb1>(v);    // quad_perm [1, 0, 3, 2]
      v += spec::dpp_move<0x4e>(v);    // quad_perm [2, 3, 0, 1]
      v += spec::dpp_move<0x141>(v);   // row_half_mirror: the other quad of the 8 lanes
      if (sl == t) keep[r] = v;        // lane 8 g + t: row t + 8 g = v0 + lane
    }
  gemv_epilogue<RT>(keep, v0, lane, wave, blk, temp, logits, probs, so, V);
}

template <typename T, int RT>
int launch_gemv(const void *X, const void *W, const float *temp, float *logits, float *probs,
                const spec::StatsOut &so, int H, int V, hipStream_t st) {
  hipLaunchKernelGGL((lm_head_gemv<T, RT>), dim3(spec::ceil_div(V, kBlockRows)), dim3(kThreads),
                     0, st, static_cast<const T *>(X), static_cast<const T *>(W), temp, logits,
                     probs, so, H, V);
  return spec::launched("lm_head_gemv");
}

template <typename T>
int launch_gemv_r(int R, const void *X, const void *W, const float *temp, float *logits,
                  float *probs, const spec::StatsOut &so, int H, int V, hipStream_t st) {
  switch (R) {
    case 1: return launch_gemv<T, 1>(X, W, temp, logits, probs, so, H, V, st);
    case 2: return launch_gemv<T, 2>(X, W, temp, logits, probs, so, H, V, st);
    case 3: return launch_gemv<T, 3>(X, W, temp, logits, probs, so, H, V, st);
    case 4: return launch_gemv<T, 4>(X, W, temp, logits, probs, so, H, V, st);
    case 5: return launch_gemv<T, 5>(X, W, temp, logits, probs, so, H, V, st);
    case 6: return launch_gemv<T, 6>(X, W, temp, logits, probs, so, H, V, st);
    case 7: return launch_gemv<T, 7>(X, W, temp, logits, probs, so, H, V, st);
    default: return launch_gemv<T, 8>(X, W, temp, logits, probs, so, H, V, st);
  }
}

// Merge the block statistics of row blockIdx.y and normalise its chunk of p in place.
// Grid: (ceil(V / CH), R), CH = 4096 or 16384 vocabulary entries per workgroup (the larger
// chunk when there are enough rows to fill the GPU, so fewer workgroups repeat the row's
// statistics reduction and each thread streams more entries).  Every load the workgroup needs
// (the row's block statistics, its p entries) is issued before the first wait, so the kernel
// costs one memory round trip plus two exchanges through LDS.
template <int CH>
__global__ __launch_bounds__(kThreads) void lm_head_finalize(
    float *__restrict__ probs, const float2 *__restrict__ stats, const int *__restrict__ amax,
    const float *__restrict__ temp, int R, int V, int nblk) {
  constexpr int kPer = CH / kThreads;             // p entries per thread
  constexpr int kBlocks = CH / kBlockRows;        // statistics blocks per chunk
  __shared__ float fac[kBlocks];
  __shared__ float sm[kWaves], ss[kWaves];
  __shared__ int si[kWaves];
  const int r = blockIdx.y, tid = threadIdx.x;
  const float c = spec::stat_scale(temp[r]);
  const bool greedy = c == 0.f;
  const int v0 = blockIdx.x * CH;
  const int blk0 = v0 / kBlockRows;
  float *row = probs + (size_t)r * V;
  const bool vec = (V & 3) == 0;

  // p entries of this chunk: kPer / 4 float4 per thread (vector path)
  float4 pv[kPer / 4];
  if (!greedy && vec) {
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
      const int v = v0 + (tid + i * kThreads) * 4;
      pv[i] = v < V ? *reinterpret_cast<const float4 *>(row + v) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  // maxima of the chunk's own blocks (for the rescale factors)
  const float own_m = (tid < kBlocks && blk0 + tid < nblk) ? stats[(size_t)(blk0 + tid) * R + r].x : 0.f;
  const spec::RowStat rs = spec::row_stat_wg<kThreads>(stats, amax, R, r, nblk, c, sm, ss, si);
  if (greedy) {
    for (int v = v0 + tid; v < min(V, v0 + CH); v += kThreads) row[v] = (v == rs.a) ? 1.f : 0.f;
    return;
  }
  if (tid < kBlocks) fac[tid] = spec::stat_factor(own_m, rs);
  __syncthreads();
  if (vec) {
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
      const int v = v0 + (tid + i * kThreads) * 4;
      if (v < V) {
        const float f = fac[(v - v0) / kBlockRows];
        float4 x = pv[i];
        x.x *= f; x.y *= f; x.z *= f; x.w *= f;
        *reinterpret_cast<float4 *>(row + v) = x;
      }
    }
  } else {
    for (int v = v0 + tid; v < min(V, v0 + CH); v += kThreads) row[v] *= fac[(v - v0) / kBlockRows];
  }
}

// Grid: R.  The statistics of row blockIdx.x (the reduction of the finalize, once per row)
// into rows[r], for the fused lm-head + accept call.
__global__ __launch_bounds__(kThreads) void lm_row_stats(const float2 *__restrict__ stats,
                                                         const int *__restrict__ amax,
                                                         const float *__restrict__ temp,
                                                         spec::RowStat *__restrict__ rows, int R,
                                                         int nblk) {
  __shared__ float sm[kWaves], ss[kWaves];
  __shared__ int si[kWaves];
  const int r = blockIdx.x;
  const spec::RowStat rs =
      spec::row_stat_wg<kThreads>(stats, amax, R, r, nblk, spec::stat_scale(temp[r]), sm, ss, si);
  if (threadIdx.x == 0) rows[r] = rs;
}

template <typename T, int NH>
int launch_nh(const void *X, const void *W, const float *temp, float *logits, float *probs,
              const spec::StatsOut &so, int R, int H, int V, hipStream_t st) {
  using S = MmaShape<NH>;
  static std::atomic<uint64_t> lds_set{0};   // per instantiation: one bit per device
  const int rc = spec::ensure_dynamic_lds(reinterpret_cast<const void *>(&lm_head_mfma<T, NH>),
                                          S::kLds, lds_set, "spec_lm_head");
  if (rc != SPEC_OK) return rc;
  dim3 grid(spec::ceil_div(V, kMmaRows), spec::ceil_div(R, NH * 16));
  hipLaunchKernelGGL((lm_head_mfma<T, NH>), grid, dim3(kMmaThreads), S::kLds, st,
                     static_cast<const T *>(X), static_cast<const T *>(W), temp, logits, probs,
                     so, R, H, V);
  return spec::launched("lm_head_mfma");
}

// One pass over the table covers up to 96 hidden rows; more rows take further passes.
template <typename T>
int launch(int R, const void *X, const void *W, const float *temp, float *logits, float *probs,
           const spec::StatsOut &so, int H, int V, hipStream_t st) {
  switch (min(kMaxNH, spec::ceil_div(R, 16))) {
    case 1: return launch_nh<T, 1>(X, W, temp, logits, probs, so, R, H, V, st);
    case 2: return launch_nh<T, 2>(X, W, temp, logits, probs, so, R, H, V, st);
    case 3: return launch_nh<T, 3>(X, W, temp, logits, probs, so, R, H, V, st);
    case 4: return launch_nh<T, 4>(X, W, temp, logits, probs, so, R, H, V, st);
    case 5: return launch_nh<T, 5>(X, W, temp, logits, probs, so, R, H, V, st);
    default: return launch_nh<T, 6>(X, W, temp, logits, probs, so, R, H, V, st);
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

}  // namespace

extern "C" int spec_profile_lm_head(void *start_event, void *stop_event) {
  g_prof_start = static_cast<hipEvent_t>(start_event);
  g_prof_stop = static_cast<hipEvent_t>(stop_event);
  return SPEC_OK;
}

static_assert(kBlockRows == spec::kStatBlock, "statistics blocks of the kernels and the reductions");

namespace spec {

LmLayout lm_layout(int R, int V) {
  LmLayout l;
  l.nblk = ceil_div(V, kBlockRows);
  size_t o = 0;
  l.off_stats = o; o += align_up((size_t)l.nblk * R * sizeof(float2), 256);
  l.off_amax = o;  o += align_up((size_t)l.nblk * R * sizeof(int), 256);
  l.off_rows = o;  o += align_up((size_t)R * sizeof(RowStat), 256);
  l.bytes = o;
  return l;
}

StatsOut lm_stats_out(const LmLayout &l, void *ws) {
  char *b = static_cast<char *>(ws);
  return StatsOut{reinterpret_cast<float2 *>(b + l.off_stats), reinterpret_cast<int *>(b + l.off_amax),
                  l.nblk};
}

int lm_row_stats_launch(const StatsOut &so, const float *temperature, RowStat *rows, int R,
                        hipStream_t st) {
  hipLaunchKernelGGL(lm_row_stats, dim3(R), dim3(kThreads), 0, st, so.stats, so.amax,
                     temperature, rows, R, so.nblk);
  return launched("lm_row_stats");
}

int lm_head_check(const void *hidden, const void *weight, const float *temperature,
                  const float *probs, const float *logits, int R, int H, int V, spec_dtype dtype,
                  const char *who) {
  SPEC_REQUIRE(hidden && weight && temperature && probs, SPEC_EINVAL,
               "%s: hidden, weight, temperature and probs must be non-null", who);
  SPEC_REQUIRE(R > 0 && H > 0 && V > 0, SPEC_EINVAL, "%s: R=%d H=%d V=%d must be positive", who,
               R, H, V);
  SPEC_REQUIRE(dtype == SPEC_F32 || dtype == SPEC_BF16, SPEC_EUNSUPPORTED,
               "%s: unsupported dtype %d", who, (int)dtype);
  SPEC_REQUIRE(H % 8 == 0, SPEC_EUNSUPPORTED, "%s: H=%d must be a multiple of 8", who, H);
  SPEC_REQUIRE(R <= kMaxRows, SPEC_EUNSUPPORTED,
               "%s: R=%d rows exceed %d (one grid row of the softmax finalize per row)", who, R,
               kMaxRows);
  SPEC_REQUIRE(aligned16(hidden) && aligned16(weight) && aligned16(probs) &&
                   (logits == nullptr || aligned16(logits)),
               SPEC_EINVAL, "%s: hidden, weight, probs and logits need 16-byte alignment", who);
  return SPEC_OK;
}

int lm_head_contract(const void *hidden, const void *weight, const float *temperature,
                     float *logits, float *probs, const StatsOut &so, int R, int H, int V,
                     spec_dtype dtype, hipStream_t st) {
  hipEvent_t ev0 = g_prof_start, ev1 = g_prof_stop;
  g_prof_start = g_prof_stop = nullptr;
  if (ev0 != nullptr && hipEventRecord(ev0, st) != hipSuccess)
    return fail(SPEC_EHIP, "spec_lm_head: hipEventRecord(start) failed");
  int rc;
  if (R <= gemv_max_rows(H))
    rc = dtype == SPEC_BF16
             ? launch_gemv_r<uint16_t>(R, hidden, weight, temperature, logits, probs, so, H, V, st)
             : launch_gemv_r<float>(R, hidden, weight, temperature, logits, probs, so, H, V, st);
  else
    rc = dtype == SPEC_BF16
             ? launch<uint16_t>(R, hidden, weight, temperature, logits, probs, so, H, V, st)
             : launch<float>(R, hidden, weight, temperature, logits, probs, so, H, V, st);
  if (rc != SPEC_OK) return rc;
  if (ev1 != nullptr && hipEventRecord(ev1, st) != hipSuccess)
    return fail(SPEC_EHIP, "spec_lm_head: hipEventRecord(stop) failed");
  return SPEC_OK;
}

}  // namespace spec

namespace {

int lm_head_finalize_launch(float *probs, const spec::StatsOut &so, const float *temperature,
                            int R, int V, hipStream_t st) {
  if ((long)R * spec::ceil_div(V, kFinChunk) > kFinWideWGs) {
    hipLaunchKernelGGL(lm_head_finalize<4 * kFinChunk>, dim3(spec::ceil_div(V, 4 * kFinChunk), R),
                       dim3(kThreads), 0, st, probs, so.stats, so.amax, temperature, R, V, so.nblk);
  } else {
    hipLaunchKernelGGL(lm_head_finalize<kFinChunk>, dim3(spec::ceil_div(V, kFinChunk), R),
                       dim3(kThreads), 0, st, probs, so.stats, so.amax, temperature, R, V, so.nblk);
  }
  return spec::launched("lm_head_finalize");
}

// Shared by spec_lm_head and spec_lm_head_noalloc: contraction + finalize with the statistics
// in `workspace` (at least spec::lm_layout(R, V).bytes).
int lm_head_run(const void *hidden, const void *weight, const float *temperature, float *logits,
                float *probs, int R, int H, int V, spec_dtype dtype, void *workspace,
                hipStream_t st) {
  const spec::StatsOut so = spec::lm_stats_out(spec::lm_layout(R, V), workspace);
  const int rc = spec::lm_head_contract(hidden, weight, temperature, logits, probs, so, R, H, V,
                                        dtype, st);
  if (rc != SPEC_OK) return rc;
  return lm_head_finalize_launch(probs, so, temperature, R, V, st);
}

}  // namespace

extern "C" size_t spec_lm_head_workspace(int R, int H, int V) {
  if (R <= 0 || H <= 0 || V <= 0) {
    spec::fail(SPEC_EINVAL, "spec_lm_head_workspace: R=%d H=%d V=%d must be positive", R, H, V);
    return 0;
  }
  return spec::lm_layout(R, V).bytes;
}

extern "C" int spec_lm_head(const void *hidden, const void *weight, const float *temperature,
                            float *logits, float *probs, int R, int H, int V, spec_dtype dtype,
                            void *workspace, size_t workspace_bytes, void *stream) {
  spec::clear_error();
  int rc = spec::lm_head_check(hidden, weight, temperature, probs, logits, R, H, V, dtype,
                               "spec_lm_head");
  if (rc != SPEC_OK) return rc;
  const size_t need = spec::lm_layout(R, V).bytes;
  SPEC_REQUIRE(workspace != nullptr && workspace_bytes >= need, SPEC_EWORKSPACE,
               "spec_lm_head: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  return lm_head_run(hidden, weight, temperature, logits, probs, R, H, V, dtype, workspace,
                     static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ allocation-free variant
// For callers that cannot allocate (code under HIP graph capture, serving loops that forbid
// allocation): the per-block statistics of spec_lm_head live in a file-scope device array
// instead of a caller workspace.  Every GPU the library runs on holds its own copy of the
// array, at its own address, until the process ends.  In host code the array's name is only a
// stand-in for the symbol: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address reaches a kernel.
// The statistics are fully rewritten by every call before they are read, so nothing has to
// be cleared between calls; calls that overlap on one GPU share the array and race.
static __device__ __align__(256) unsigned char scratch[SPEC_LM_HEAD_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`.
int static_scratch(void **out, const char *who) {
  int dev = 0;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) return spec::fail(SPEC_EHIP, "%s: hipGetDevice: %s", who, hipGetErrorString(ge));
  SPEC_REQUIRE(dev >= 0 && dev < kMaxDevices, SPEC_EUNSUPPORTED,
               "%s: device id %d beyond the %d devices the static array is tracked for", who,
               dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return spec::fail(SPEC_EHIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", who,
                        dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}

}  // namespace

extern "C" int spec_lm_head_noalloc(const void *hidden, const void *weight,
                                    const float *temperature, float *logits, float *probs, int R,
                                    int H, int V, spec_dtype dtype, void *stream) {
  spec::clear_error();
  int rc = spec::lm_head_check(hidden, weight, temperature, probs, logits, R, H, V, dtype,
                               "spec_lm_head_noalloc");
  if (rc != SPEC_OK) return rc;
  const size_t need = spec::lm_layout(R, V).bytes;
  SPEC_REQUIRE(need <= (size_t)SPEC_LM_HEAD_STATIC_SCRATCH_BYTES, SPEC_EUNSUPPORTED,
               "spec_lm_head_noalloc: R=%d rows over V=%d need %zu bytes of statistics, the "
               "static array holds %zu (use spec_lm_head with a workspace)",
               R, V, need, (size_t)SPEC_LM_HEAD_STATIC_SCRATCH_BYTES);
  void *ws = nullptr;
  rc = static_scratch(&ws, "spec_lm_head_noalloc");
  if (rc != SPEC_OK) return rc;
  return lm_head_run(hidden, weight, temperature, logits, probs, R, H, V, dtype, ws,
                     static_cast<hipStream_t>(stream));
}
