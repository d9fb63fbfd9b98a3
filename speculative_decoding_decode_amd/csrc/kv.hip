// KV-cache bookkeeping around the verify step: append the K/V of the verified positions, then
// keep the accepted ones.
//
// The pages: drafts from the first rejected one on are discarded and the target generates the
// token at that position (butteryoon "Gemma 4 MTP 서빙 가이드 해설", section 4, accept/reject
// step; llm-wiki "Gemma 4 MTP ...", section "투기적 디코딩의 기본 구조": confirm up to the wrong
// position).  In cache terms: the verify forward writes K/V for its K1 input positions (the last
// committed token and the k drafts); after acceptance of n drafts, the last committed token and
// the n accepted drafts stay, the k - n rejected drafts are dropped, and the correction (or bonus)
// token's K/V arrive with the next step.  Dropping is a length update: the next append simply
// overwrites the rejected slots.
#include "common.hpp"

namespace {

constexpr int kPage = 16;

// Grid: (B * K1 * Hkv), block: D / EPG threads, each copying one 16-byte group of K and of V.
template <typename T>
__global__ void kv_append(const T *__restrict__ k_new, const T *__restrict__ v_new,
                          T *__restrict__ k_pool, T *__restrict__ v_pool,
                          const int32_t *__restrict__ table, const int32_t *__restrict__ ctx_lens,
                          int K1, int Hkv, int D, int num_pages, int max_pages) {
  constexpr int EPG = 16 / (int)sizeof(T);
  const int id = blockIdx.x;
  const int g = id % Hkv, i = (id / Hkv) % K1, b = id / (Hkv * K1);
  const int pos = ctx_lens[b] - K1 + i;
  if (pos < 0 || pos >= max_pages * kPage) return;
  const int page = table[(size_t)b * max_pages + pos / kPage];
  if (page < 0 || page >= num_pages) return;
  const int e = threadIdx.x * EPG;
  if (e >= D) return;
  const size_t src = (((size_t)b * K1 + i) * Hkv + g) * D + e;
  const size_t dst = (((size_t)page * Hkv + g) * kPage + pos % kPage) * D + e;
  *reinterpret_cast<uint4 *>(k_pool + dst) = *reinterpret_cast<const uint4 *>(k_new + src);
  *reinterpret_cast<uint4 *>(v_pool + dst) = *reinterpret_cast<const uint4 *>(v_new + src);
}

__global__ void kv_commit(int32_t *__restrict__ ctx_lens, const int32_t *__restrict__ n_accepted,
                          int B, int K1) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int n = n_accepted[b];
  n = n < 0 ? 0 : (n > K1 - 1 ? K1 - 1 : n);
  ctx_lens[b] -= K1 - 1 - n;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int spec_kv_append(const void *k_new, const void *v_new, void *k_pool, void *v_pool,
                              const int32_t *page_table, const int32_t *ctx_lens, int B, int K1,
                              int Hkv, int D, int page_size, int num_pages, int max_pages_per_seq,
                              spec_dtype dtype, void *stream) {
  spec::clear_error();
  SPEC_REQUIRE(k_new && v_new && k_pool && v_pool && page_table && ctx_lens, SPEC_EINVAL,
               "spec_kv_append: null pointer argument");
  SPEC_REQUIRE(B > 0 && K1 > 0 && Hkv > 0 && D > 0 && num_pages > 0 && max_pages_per_seq > 0,
               SPEC_EINVAL, "spec_kv_append: sizes must be positive");
  SPEC_REQUIRE(page_size == kPage, SPEC_EUNSUPPORTED, "spec_kv_append: page_size=%d, only 16", page_size);
  SPEC_REQUIRE((long long)B * K1 * Hkv <= 0x7fffffffLL, SPEC_EUNSUPPORTED,
               "spec_kv_append: B*K1*Hkv rows exceed one grid");
  SPEC_REQUIRE(dtype == SPEC_F32 || dtype == SPEC_BF16, SPEC_EUNSUPPORTED,
               "spec_kv_append: unsupported dtype %d", (int)dtype);
  const int epg = dtype == SPEC_BF16 ? 8 : 4;
  SPEC_REQUIRE(D % epg == 0 && D / epg <= 1024, SPEC_EUNSUPPORTED,
               "spec_kv_append: head dim %d must be a multiple of %d (16-byte rows)", D, epg);
  SPEC_REQUIRE(aligned16(k_new) && aligned16(v_new) && aligned16(k_pool) && aligned16(v_pool),
               SPEC_EINVAL, "spec_kv_append: tensors need 16-byte alignment");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int threads = ((D / epg + 63) / 64) * 64;
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL(kv_append<uint16_t>, dim3(B * K1 * Hkv), dim3(threads), 0, st,
                       static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new),
                       static_cast<uint16_t *>(k_pool), static_cast<uint16_t *>(v_pool),
                       page_table, ctx_lens, K1, Hkv, D, num_pages, max_pages_per_seq);
  else
    hipLaunchKernelGGL(kv_append<float>, dim3(B * K1 * Hkv), dim3(threads), 0, st,
                       static_cast<const float *>(k_new), static_cast<const float *>(v_new),
                       static_cast<float *>(k_pool), static_cast<float *>(v_pool), page_table,
                       ctx_lens, K1, Hkv, D, num_pages, max_pages_per_seq);
  return spec::launched("kv_append");
}

extern "C" int spec_kv_commit(int32_t *ctx_lens, const int32_t *n_accepted, int B, int K1,
                              void *stream) {
  spec::clear_error();
  SPEC_REQUIRE(ctx_lens && n_accepted, SPEC_EINVAL, "spec_kv_commit: null pointer argument");
  SPEC_REQUIRE(B > 0 && K1 > 0, SPEC_EINVAL, "spec_kv_commit: B=%d K1=%d must be positive", B, K1);
  hipLaunchKernelGGL(kv_commit, dim3((B + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                     ctx_lens, n_accepted, B, K1);
  return spec::launched("kv_commit");
}
