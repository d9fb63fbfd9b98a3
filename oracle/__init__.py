"""fp64 CPU oracle of the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or executes this
package: only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py use it.  It
shares no code with the HIP library (speculative_decoding_decode_amd); the two meet only in
the seeded input generators of workloads/, which hold no arithmetic of the method.

Every value is computed in float64 from inputs converted exactly (bf16 and fp32 values are
exactly representable in float64), with plain numpy, in the order the method states it.

Pages this oracle follows (cited below by the short name in brackets):
  [wiki]     llm-wiki.hwlabs.dev, "Gemma 4 MTP: 드래프터가 초안을 쓰고 타깃이 검증하는 추론
             가속 구조" (sections "투기적 디코딩(Speculative Decoding)의 기본 구조",
             "드래프터 내부 아키텍처")
  [geeknews] news.hada.io topic 29214, "Gemma 4 가속하기 : 다중 토큰 예측 drafter로 더 빠른
             추론" (section "MTP가 동작하는 방식")
  [damoang]  damoang.net free/6230569, Korean text of Google's MTP drafter announcement
             (section "추측적 해독은 어떻게 작동하는가")
  [guide]    butteryoon.github.io, "Gemma 4 MTP 서빙 가이드 해설 — 페어드 드래프터·MIG
             슬라이싱·vLLM 설정" (section 4 "실행 흐름", section 7 settings table)

The pages state the verify step in words and cite Leviathan et al. (2022), "Fast Inference from
Transformers via Speculative Decoding", for the acceptance rule; that published rule is what
accept.py restates.  Readings of points the pages leave open are listed in each module.

Parity pins: every function here is checked by tests/test_oracle_*.py against values the pages
or the mathematics fix (closed forms, brute-force enumeration, library routines on special
cases, invariants).  No function is "parity unpinned".
"""
from .attention import verify_attention, visible_range  # noqa: F401
from .lm_head import logits, probabilities  # noqa: F401
from .accept import (accept_mask, first_rejection, integer_weights, sample_index,  # noqa: F401
                     verify_accept, FIXED_BITS, UNIFORM_BITS)
from .philox import philox4x32_10, uniforms as philox_uniforms  # noqa: F401
