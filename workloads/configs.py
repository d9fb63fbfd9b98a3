"""Shapes of the verify-step workloads.

Each workload is one verify step of speculative decoding: a batch of B sequences, k drafted
tokens each, so K1 = k + 1 query positions per sequence (the k drafts plus the bonus
position) are scored by the target in one pass, then accepted or rejected.

The attention shapes follow the hybrid layout the serving guide describes for Gemma 4
(butteryoon "Gemma 4 MTP 서빙 가이드 해설", section 7, settings table: local heads of dim 256,
global heads of dim 512) and the 3 sliding + 1 global pattern of the drafter block
(llm-wiki "Gemma 4 MTP ...", section "드래프터 내부 아키텍처").  The 256k vocabulary comes from
the same guide's section 1 table.  Everything here is a shape or a recipe constant; no value
of the method is computed in this module.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import json
import os


@dataclass(frozen=True)
class Layer:
    """One attention layer of the verify forward.

    kind: "sliding" (keys within `window` positions of the query, self included) or
    "global" (all earlier keys).
    """
    kind: str
    hq: int
    hkv: int
    head_dim: int
    window: int = 0  # 0 means global

    @property
    def group(self) -> int:
        return self.hq // self.hkv


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    k: int
    layers: tuple
    ctx: str                 # "fixed:<n>", "uniform:<lo>:<hi>", "loguniform:<lo>:<hi>"
    hidden: int
    vocab: int
    dtype: str               # "f32" or "bf16" for Q/K/V, hidden states and the lm-head table
    logit_recipe: str        # "gauss" (drafter N(0,1), target = drafter + noise) or "zipf"
    noise_key: str           # key into the tuned noise table, or a literal "sigma:<x>"
    temperatures: tuple      # per-sequence temperature pattern, cycled over the batch
    paged: bool = True       # False: identity page table (a contiguous cache)
    page_size: int = 16
    seed: int = 0
    description: str = field(default="", compare=False)

    @property
    def k1(self) -> int:
        return self.k + 1

    @property
    def rows(self) -> int:
        """Rows of the lm-head contraction: every query position of every sequence."""
        return self.batch * self.k1

    def temperature_of(self, b: int) -> float:
        return float(self.temperatures[b % len(self.temperatures)])


SLIDING_256 = dict(kind="sliding", head_dim=256, window=1024)
GLOBAL_512 = dict(kind="global", head_dim=512, window=0)

WORKLOADS = {
    # Tiny fp32 case the oracle finishes instantly: one global layer, contiguous cache.
    "tiny_fp32_b1_k2": Workload(
        name="tiny_fp32_b1_k2", batch=1, k=2,
        layers=(Layer("global", 8, 2, 64, 0),),
        ctx="fixed:512", hidden=256, vocab=4096, dtype="f32",
        logit_recipe="gauss", noise_key="sigma:0.7", temperatures=(1.0,), paged=False, seed=0,
        description="batch 1, k=2, 1 global layer 8q/2kv hd64, 512-token contiguous cache, "
                    "hidden 256, vocab 4096, fp32"),
    # Batch-1 decode at 8K context: the throughput headline.
    "b1_k2_sliding256_8k": Workload(
        name="b1_k2_sliding256_8k", batch=1, k=2,
        layers=(Layer(hq=8, hkv=2, **SLIDING_256),),
        ctx="fixed:8192", hidden=2560, vocab=262144, dtype="bf16",
        logit_recipe="gauss", noise_key="pos0_047", temperatures=(1.0,), seed=1,
        description="batch 1, k=2, sliding hd256 window 1024, 8q/2kv, paged 16-token pages "
                    "over 8192 tokens, lm-head 2560 x 262144 bf16"),
    "b1_k4_global512_32k": Workload(
        name="b1_k4_global512_32k", batch=1, k=4,
        layers=(Layer(hq=16, hkv=4, **GLOBAL_512),),
        ctx="fixed:32768", hidden=5376, vocab=262144, dtype="bf16",
        logit_recipe="zipf", noise_key="sigma:0.5", temperatures=(1.0,), seed=2,
        description="batch 1, k=4, global hd512 16q/4kv, paged over 32768 tokens, "
                    "lm-head 5376 x 262144 bf16, Zipf(1.1) base logits"),
    "b8_ragged_k5_hybrid": Workload(
        name="b8_ragged_k5_hybrid", batch=8, k=5,
        layers=(Layer(hq=8, hkv=2, **SLIDING_256), Layer(hq=8, hkv=2, **SLIDING_256),
                Layer(hq=8, hkv=2, **SLIDING_256), Layer(hq=8, hkv=2, **GLOBAL_512)),
        ctx="uniform:1024:16384", hidden=2560, vocab=262144, dtype="bf16",
        logit_recipe="gauss", noise_key="pos0_047", temperatures=(0.0, 0.7, 1.0), seed=3,
        description="batch 8 ragged, k=5, layers [S,S,S,G] (S: hd256 window 1024, G: hd512), "
                    "8q/2kv, shared page pool, lm-head 2560 x 262144"),
    "b32_k2_mixed_16k": Workload(
        name="b32_k2_mixed_16k", batch=32, k=2,
        layers=(Layer(hq=16, hkv=4, **GLOBAL_512), Layer(hq=16, hkv=4, **SLIDING_256)),
        ctx="loguniform:512:16384", hidden=5376, vocab=262144, dtype="bf16",
        logit_recipe="gauss", noise_key="overall_035", temperatures=(1.0,), seed=4,
        description="batch 32, k=2, layers [G hd512, S hd256 window 1024], 16q/4kv, "
                    "log-uniform context 512..16384, lm-head 5376 x 262144"),
}

# Order in which the workloads are listed: the tiny case first, then the headline.
ORDER = ("tiny_fp32_b1_k2", "b1_k2_sliding256_8k", "b1_k4_global512_32k",
         "b8_ragged_k5_hybrid", "b32_k2_mixed_16k")

_NOISE_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "noise_sigma.json")


def noise_sigma(w: Workload) -> float:
    """Standard deviation of the logit noise between drafter and target for `w`.

    A literal "sigma:<x>" is the value the workload states.  The tuned entries
    ("pos0_047": acceptance at the first position about 47%; "overall_035": about 35% overall
    acceptance at k=2) are read from noise_sigma.json, which oracle/tune_noise.py writes by
    bisecting the closed-form acceptance of the oracle.
    """
    if w.noise_key.startswith("sigma:"):
        return float(w.noise_key.split(":", 1)[1])
    with open(_NOISE_FILE) as f:
        table = json.load(f)
    return float(table[w.noise_key]["sigma"])
