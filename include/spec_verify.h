/*
 * spec_verify.h -- C ABI of the speculative-decoding verify step on AMD MI355X (gfx950).
 *
 * One verify step scores the k drafted tokens of every sequence plus one bonus position in a
 * single target forward, then accepts or rejects the drafts without changing the target's
 * output distribution.  The pages this follows:
 *   - llm-wiki.hwlabs.dev, "Gemma 4 MTP: 드래프터가 초안을 쓰고 타깃이 검증하는 추론 가속 구조",
 *     section "투기적 디코딩(Speculative Decoding)의 기본 구조": the target checks the k
 *     proposed tokens in one forward, confirms them up to the first wrong one and generates
 *     the token there itself, which keeps the output distribution unchanged;
 *   - butteryoon.github.io, "Gemma 4 MTP 서빙 가이드 해설", section 4 execution flow
 *     (parallel verification against the target's own distribution, then accept/reject with
 *     the drafts after the first rejection discarded), section 1 table (the drafter and the
 *     target share one KV-cache pool; a 256k vocabulary), section 7 settings table (local
 *     attention heads of dim 256, global heads of dim 512);
 *   - news.hada.io topic 29214, "Gemma 4 가속하기 : 다중 토큰 예측 drafter로 더 빠른 추론",
 *     section "MTP가 동작하는 방식": when the target agrees with the whole draft it accepts it
 *     and generates one extra token in the same forward.
 * The acceptance rule is the one of Leviathan et al. (2022), which the pages cite.
 *
 * Conventions for every call:
 *   - Pointers are device pointers owned by the caller (except where noted).  The library
 *     allocates nothing; scratch memory is the caller's `workspace`, at least as large as the
 *     matching *_workspace() query says, with no required contents (every call writes what it
 *     reads).  Its only state is per host thread: the message of
 *     the last error (spec_last_error) and the one-shot profiling bracket armed by
 *     spec_profile_lm_head; every call is otherwise independent of earlier calls and may be
 *     made from any thread.
 *   - Calls run on the calling thread's current HIP device: `stream` (a hipStream_t, NULL
 *     for the null stream) and every pointer must belong to it, and spec_verify_attn_workspace
 *     sizes for its compute units.  Calls only enqueue kernels on the stream and return;
 *     results are valid once the stream has reached that point.  They enqueue no memset, copy
 *     or synchronisation, so a sequence of calls can be captured in a HIP graph and replayed
 *     (the inputs read at replay time are whatever the captured buffers then hold).
 *   - Return value: SPEC_OK (0) or a negative spec_status.  Host-checkable argument errors are
 *     reported before anything is enqueued; spec_last_error() then describes the failure (a
 *     thread-local string, valid until the next call on the same thread).
 *   - Preconditions on device-resident data are documented per call and not checked on the
 *     host; where a violation could make a kernel read out of bounds the kernel clamps or
 *     masks instead (stated per call), so no input makes a kernel fault.
 *   - All tensors are dense, row-major, with the shapes given; "b-major" means sequence
 *     index outermost.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_OK = 0,
  SPEC_EINVAL = -1,        /* a null pointer, a non-positive size, inconsistent shapes */
  SPEC_EUNSUPPORTED = -2,  /* a shape or dtype outside what the kernels implement */
  SPEC_EWORKSPACE = -3,    /* workspace smaller than the *_workspace() query returns */
  SPEC_EHIP = -4           /* the HIP runtime rejected a launch; message from hipGetErrorString */
} spec_status;

typedef enum {
  SPEC_F32 = 0,            /* IEEE binary32 */
  SPEC_BF16 = 1            /* bfloat16 (upper 16 bits of a binary32) */
} spec_dtype;

/* Version of this interface, (major << 16) | minor. */
int spec_version(void);

/* Message describing the last failing call on this thread ("" if none). */
const char *spec_last_error(void);

/* ------------------------------------------------------------------------------------------
 * (i) Verify attention: K1 = k + 1 causal queries per sequence over a paged KV cache, one
 *     layer per call, grouped-query heads.
 *
 * Passages: the target scores all k drafts in one forward pass (llm-wiki "Gemma 4 MTP ...",
 * section "투기적 디코딩(Speculative Decoding)의 기본 구조"; butteryoon guide, section 4
 * "실행 흐름", parallel verification step); over the KV cache the drafter shares with it
 * (same guide, section 1 table, KV-cache row); with local heads of dim 256 and global heads of
 * dim 512 (same guide, section 7 settings table).
 *
 * The K1 verified positions are the last K1 tokens of each sequence's cache (their K/V are
 * already written).  Query i of sequence b sits at position t = ctx_lens[b] - K1 + i and sees
 * the key positions s with lo <= s <= t, lo = 0 for a global layer (window == 0) and
 * lo = max(0, t - window + 1) for a sliding-window layer.  Query head h reads KV head
 * h / (Hq / Hkv).  out = softmax(scale * q k^T) v over the visible keys, accumulated in fp32.
 *
 *   q           [B, K1, Hq, D]               dtype
 *   k_pool      [num_pages, Hkv, page_size, D] dtype   key position s of sequence b is at page
 *   v_pool      [num_pages, Hkv, page_size, D] dtype   page_table[b][s / page_size], slot
 *                                                       s % page_size
 *   page_table  [B, max_pages_per_seq] int32  physical page ids
 *   ctx_lens    [B] int32                     tokens in each cache, the K1 new ones included
 *   out         [B, K1, Hq, D] fp32
 *   D in {64, 128, 256, 512}; page_size == 16; Hq % Hkv == 0; K1 in [1, 64];
 *   B * K1 * Hq < 2^31 (SPEC_EUNSUPPORTED otherwise).
 *
 * Device-data preconditions: K1 <= ctx_lens[b] <= max_pages_per_seq * page_size.  ctx_lens
 * beyond that bound are clamped to it (the verified positions then sit at the clamped length
 * - K1 + i); a page id outside [0, num_pages) hides the keys on that page; a query with no
 * visible key gets a zero output row.
 * ---------------------------------------------------------------------------------------- */
size_t spec_verify_attn_workspace(int B, int K1, int Hq, int Hkv, int D, int page_size,
                                  int max_pages_per_seq, int window);

int spec_verify_attn(const void *q, const void *k_pool, const void *v_pool,
                     const int32_t *page_table, const int32_t *ctx_lens, float *out,
                     int B, int K1, int Hq, int Hkv, int D, int page_size, int num_pages,
                     int max_pages_per_seq, int window, float scale, spec_dtype dtype,
                     void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------------
 * (ii) lm-head: logits = hidden W^T over the R = B * K1 verify rows, then the target's row
 *      distributions p = softmax(logits / T) (temperature per row; T <= 0 gives the one-hot
 *      vector at the first maximal logit, i.e. greedy).
 *
 * Passages: every verified position is compared with the target's own distribution
 * (butteryoon guide, section 4 "실행 흐름"); the projection onto the 256k vocabulary is a large
 * part of the cost (same guide, section 1; damoang's text of the MTP announcement, section on
 * the drafters' internals: the final logit computation is a major bottleneck).
 *
 *   hidden       [R, H]  dtype  (rows b-major: row b*K1 + i is query position i of sequence b)
 *   weight       [V, H]  dtype  vocab x hidden table, row-major
 *   temperature  [R] fp32 (device)
 *   logits       [R, V] fp32, or NULL when the raw logits are not wanted
 *   probs        [R, V] fp32  p, rows summing to 1
 *   H % 8 == 0 (16-byte rows for bf16); R <= 65535.  Accumulation is fp32 (dot products in
 *   the GEMV, which serves up to five rows; MFMA otherwise).
 *   Workspace: per 256-row vocabulary block and row the softmax statistics.
 * ---------------------------------------------------------------------------------------- */
size_t spec_lm_head_workspace(int R, int H, int V);

int spec_lm_head(const void *hidden, const void *weight, const float *temperature,
                 float *logits, float *probs, int R, int H, int V, spec_dtype dtype,
                 void *workspace, size_t workspace_bytes, void *stream);

/* (ii) without a workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops or harnesses that forbid hipMalloc).  Same arguments, results
 * and errors as spec_lm_head, minus the workspace: the scratch it needs (the per-256-row
 * vocabulary block softmax statistics) lives in a static device array of
 * SPEC_LM_HEAD_STATIC_SCRATCH_BYTES that every GPU the library runs on holds until the process
 * ends.  Usable whenever spec_lm_head_workspace(R, H, V) <= SPEC_LM_HEAD_STATIC_SCRATCH_BYTES
 * (about R * ceil(V / 256) * 12 bytes: at V = 262144 up to 681 rows); larger problems return
 * SPEC_EUNSUPPORTED before anything is enqueued.  Allocates nothing.  Every call on one
 * GPU uses that GPU's one array: calls that overlap on a GPU (concurrent streams, threads)
 * race and must be serialised by the caller. */
#define SPEC_LM_HEAD_STATIC_SCRATCH_BYTES (8u << 20)

int spec_lm_head_noalloc(const void *hidden, const void *weight, const float *temperature,
                         float *logits, float *probs, int R, int H, int V, spec_dtype dtype,
                         void *stream);

/* Profiling aid for (ii), and the library's one piece of state besides the error message:
 * arms a one-shot bracket, held per host thread, around the contraction kernel of the next
 * spec_lm_head call on this thread.  `start_event` / `stop_event` are hipEvent_t handles
 * created by the caller (either may be NULL); the call records them on its stream right
 * before and right after the contraction kernel (not around the softmax finalize), then
 * disarms.  Returns SPEC_OK.  Not part of the verify step itself: a benchmark uses it to time
 * the dominant kernel on the stream it runs on. */
int spec_profile_lm_head(void *start_event, void *stop_event);

/* ------------------------------------------------------------------------------------------
 * (iii) Accept / reject (Leviathan et al.), with the correction or bonus token.
 *
 * Passages: drafts are confirmed up to the first wrong one, where the target generates the
 * token itself, leaving the output distribution unchanged (llm-wiki "Gemma 4 MTP ...",
 * section "투기적 디코딩(Speculative Decoding)의 기본 구조"; butteryoon guide, section 4,
 * accept/reject step); when the whole draft is accepted the same forward yields one extra
 * token (GeekNews "Gemma 4 가속하기 : 다중 토큰 예측 drafter로 더 빠른 추론", section "MTP가
 * 동작하는 방식"; damoang's text of the MTP announcement, section "추측적 해독은 어떻게
 * 작동하는가", which cites Leviathan et al. for the rule).
 *
 * For each sequence b and i < k: draft i is accepted iff u[b][i] * q[b][i][d] < p[b][i][d]
 * with d = draft[b][i], evaluated exactly (fp64 product of fp32 values); acceptance stops at
 * the first rejection, n = number accepted.  Then one token y is drawn with u[b][k]:
 * n < k: from max(0, p[b][n] - q[b][n]) (correction); n == k: from p[b][k] (bonus).  The draw
 * is an inverse CDF over integer weights floor(x * 2^38) (order-independent sums; if every
 * correction weight is 0 the weights of p[b][n] are used): with W the weight total and
 * m = floor(u[b][k] * 2^24), y is the smallest index whose running weight sum exceeds
 * floor(m * W / 2^24).
 *
 *   draft       [B, k]     int32
 *   q           [B, k, V]  fp32  drafter distributions (may be NULL when k == 0)
 *   p           [B, K1, V] fp32  target distributions, K1 = k + 1
 *   uniforms    [B, K1]    fp32  in [0, 1): k acceptance tests, then the one draw
 *   n_accepted  [B] int32  (out) 0..k
 *   tokens      [B, K1] int32 (out) d_0 .. d_{n-1}, y, then -1 padding
 *   k in [0, 63]; B <= 65535.
 *
 * Device-data preconditions: p and q rows are distributions (non-negative, summing to 1).  A
 * draft id outside [0, V) is rejected without being read.  A p row whose weights are all 0
 * draws index 0.
 * Workspace: per sequence the weight sums of its vocabulary chunks and the count n.
 * ---------------------------------------------------------------------------------------- */
size_t spec_accept_workspace(int B, int k, int V);

int spec_accept(const int32_t *draft, const float *q, const float *p, const float *uniforms,
                int32_t *n_accepted, int32_t *tokens, int B, int k, int V,
                void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------------
 * (iii) with the uniforms drawn on the GPU: the same accept / reject and draw as spec_accept,
 * with u[b][i] generated in the kernels by the counter-based generator Philox4x32-10 (Salmon,
 * Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) instead of read
 * from an array, so a decode loop needs no host-side random numbers:
 *
 *   u[b][i] = (word (i mod 4) of Philox4x32-10 at counter (i div 4, b, offset mod 2^32,
 *              offset div 2^32) with key (seed mod 2^32, seed div 2^32)) >> 8, times 2^-24.
 *
 * A caller advances `offset` (e.g. by one per verify step) to get fresh draws under one seed.
 * uniforms_out [B, K1] fp32, if not NULL, receives the values used; given those values
 * spec_accept returns the same n_accepted and tokens.  Other arguments, workspace (the size
 * spec_accept_workspace returns) and errors as for spec_accept.
 * ---------------------------------------------------------------------------------------- */
int spec_accept_philox(const int32_t *draft, const float *q, const float *p, uint64_t seed,
                       uint64_t offset, float *uniforms_out, int32_t *n_accepted,
                       int32_t *tokens, int B, int k, int V, void *workspace,
                       size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------------
 * (ii) + (iii) in one call: the lm-head contraction of the R = B * K1 verify rows, then the
 * accept / reject and the correction or bonus draw, without the softmax finalize pass over p.
 * The accept kernel forms the values of p it needs (at the drafts, and the chunks of row n it
 * sums and draws from) from the contraction's per-block exp values and statistics, with the
 * operations of spec_lm_head's finalize, so n_accepted and tokens equal those of spec_lm_head
 * followed by spec_accept (or spec_accept_philox) on the same arguments, bit for bit.  Four
 * launches (contraction, row statistics once per row, accept chunks, draw) and no pass over p:
 * the softmax finalize that reads and rewrites all of p [R, V] (100 MB at 96 rows over a 256k
 * vocabulary) is not run, and each row's statistics are reduced once instead of by every
 * finalize workgroup of the row; p itself is not returned.
 *
 * Passages: the verify forward compares every drafted position with the target's own
 * distribution and accepts or rejects in the same step (butteryoon guide, section 4 "실행
 * 흐름"); the serving guide runs sampling on a dedicated GPU backend (section 7 settings
 * table); the bonus token comes out of the same forward (GeekNews "Gemma 4 가속하기 : 다중
 * 토큰 예측 drafter로 더 빠른 추론", section "MTP가 동작하는 방식").
 *
 *   hidden, weight, temperature   as spec_lm_head (R = B * (k + 1) rows, b-major)
 *   draft, q                      as spec_accept
 *   uniforms    [B, K1] fp32, or NULL: then u[b][i] is Philox4x32-10 at (seed, offset) as in
 *               spec_accept_philox, and uniforms_out (if not NULL) receives the values used
 *   n_accepted, tokens            as spec_accept
 *   Limits of both calls apply (R <= 65535, k <= 63, H % 8 == 0).  Workspace: the
 *   contraction's exp values [R, V] fp32, its block and row statistics, the accept step's
 *   chunk sums.
 * ---------------------------------------------------------------------------------------- */
size_t spec_lm_head_accept_workspace(int B, int k, int H, int V);

int spec_lm_head_accept(const void *hidden, const void *weight, const float *temperature,
                        const int32_t *draft, const float *q, const float *uniforms,
                        uint64_t seed, uint64_t offset, float *uniforms_out,
                        int32_t *n_accepted, int32_t *tokens, int B, int k, int H, int V,
                        spec_dtype dtype, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------------
 * KV-cache bookkeeping around the verify step.  Drafts from the first rejected one on are
 * discarded and the target generates the token there (butteryoon "Gemma 4 MTP 서빙 가이드
 * 해설", section 4 accept/reject step; llm-wiki "Gemma 4 MTP ...", section "투기적 디코딩의
 * 기본 구조").  The verify forward's K1 input positions are the last committed token and the k
 * drafts; their K/V go into the cache before spec_verify_attn reads it:
 *
 *   spec_kv_append  writes k_new / v_new [B, K1, Hkv, D] (dtype) to positions
 *                   ctx_lens[b] - K1 + i of each sequence's pages (ctx_lens already counts
 *                   them, as in spec_verify_attn).  Positions outside the page table or on a
 *                   page id outside [0, num_pages) are skipped.  D * element size must be a
 *                   multiple of 16 bytes; B * K1 * Hkv < 2^31.
 *   spec_kv_commit  after spec_accept: ctx_lens[b] -= K1 - 1 - n_accepted[b] (n clamped to
 *                   [0, K1 - 1]), keeping the last committed token and the n accepted drafts;
 *                   the rejected slots are overwritten by the next append, and the correction
 *                   or bonus token's K/V arrive with the next step.
 * Both are asynchronous on `stream` and allocate nothing.
 * ---------------------------------------------------------------------------------------- */
int spec_kv_append(const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                   const int32_t *page_table, const int32_t *ctx_lens, int B, int K1, int Hkv,
                   int D, int page_size, int num_pages, int max_pages_per_seq, spec_dtype dtype,
                   void *stream);

int spec_kv_commit(int32_t *ctx_lens, const int32_t *n_accepted, int B, int K1, void *stream);

/* ------------------------------------------------------------------------------------------
 * Measurement aid, not part of the verify step: the HBM ceilings its streaming kernels are
 * compared with on the same GPU (decoding is bound by streaming weights from memory,
 * butteryoon guide, introduction).  Both probes use 16-byte nontemporal loads, 1 KB contiguous
 * per wave instruction, a grid of spec_hbm_probe_grid() workgroups striding over the buffer.
 *   mode 0  read `bytes` of src; dst receives 4 * spec_hbm_probe_grid() uint32 words whose
 *           XOR equals the XOR of every 32-bit word of src (so no load is dead);
 *   mode 1  copy `bytes` from src to dst (nontemporal stores); the buffers must not overlap.
 * bytes a positive multiple of 16; src and dst 16-byte aligned.  Asynchronous on `stream`.
 * ---------------------------------------------------------------------------------------- */
int spec_hbm_probe_grid(void);

int spec_hbm_probe(int mode, const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
