"""Acceptance telemetry computed from the accept counts the verify step returns.

The four signals and their thresholds are the ones the Gemma 4 MTP serving guide recommends
watching (butteryoon "Gemma 4 MTP 서빙 가이드 해설", section 6 monitoring table; the G4
measurements of section 2):

  overall acceptance    accepted drafts / drafted tokens; reference 34-36%, alarm below 25%
  mean accepted length  tokens emitted per verify step (accepted drafts + the correction or
                        bonus token), "MAL"; about 1.70-1.72 at k = 2
  per-position decay    fraction of steps whose draft at position i was accepted
                        (unconditional); pos0 about 47%, pos1 about 24%; pos1 below 15% while
                        pos0 is normal means k should drop to 1
  net TPOT/ITL gain     measured outside this module

k tuning (the guide's operating loop: raise k while the tokens per step still grow, and the
G4 result that k = 2 was optimal with k >= 3 wasted, section 2): choose_k combines the
tokens-per-step curve with the measured verify-step time at every k.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

OVERALL_ALARM = 0.25      # sustained overall acceptance below this: drafter drift
POS1_ALARM = 0.15         # pos1 below this with a normal pos0: reduce k to 1
NO_GAIN = 0.20            # below this the verify cost is paid with no speed-up


@dataclass
class AcceptStats:
    k: int
    steps: int
    mean_accepted_length: float
    overall_acceptance: float
    per_position: list
    alarms: list = field(default_factory=list)


def accept_stats(n_accepted, k: int, pos0_normal: float = 0.40) -> AcceptStats:
    """Telemetry of a set of verify steps; n_accepted holds one accept count (0..k) per
    sequence per step."""
    n = np.asarray(n_accepted).reshape(-1)
    if n.size == 0:
        raise ValueError("no steps")
    if k <= 0:
        return AcceptStats(k, int(n.size), 1.0, 0.0, [])
    per_pos = [float(np.mean(n > i)) for i in range(k)]
    overall = float(np.mean(n)) / k
    mal = float(np.mean(n + 1))
    alarms = []
    if overall < NO_GAIN:
        alarms.append("acceptance below 20%: speculative decoding gives no net gain")
    elif overall < OVERALL_ALARM:
        alarms.append("acceptance below 25%: drafter drift, realign the drafter")
    if k >= 2 and per_pos[0] >= pos0_normal and per_pos[1] < POS1_ALARM:
        alarms.append("pos1 below 15% with a normal pos0: reduce k to 1")
    return AcceptStats(k, int(n.size), mal, overall, per_pos, alarms)


def expected_tokens_per_step(per_position_acceptance: float, k: int) -> float:
    """E[n + 1] when every position is accepted with the same probability a (given the
    previous ones): 1 + a + ... + a^k."""
    a = float(per_position_acceptance)
    return float(sum(a ** i for i in range(k + 1)))


def mal_from_positions(per_position, k: int) -> float:
    """Tokens per verify step at k drafts from unconditional per-position acceptance rates
    P(n > i) measured with at least k drafts: 1 + sum over i < k.  (Whether position i is
    accepted does not depend on the drafts after it, so rates measured at a larger k hold.)"""
    if k > len(per_position):
        raise ValueError(f"rates for {len(per_position)} positions, k = {k}")
    return 1.0 + float(sum(per_position[:k]))


@dataclass
class KChoice:
    best_k: int                   # highest verified tokens per second
    plateau_k: int                # smallest k after which one more draft adds < min_gain tokens
    tokens_per_step: dict
    tokens_per_second: dict


def choose_k(tokens_per_step: dict, step_seconds: dict, min_gain: float = 0.05) -> KChoice:
    """Pick k from the tokens-per-step curve and the verify-step time at each k (both keyed
    by k; k = 0 is plain decoding).  best_k maximises tokens per second (ties: smaller k);
    plateau_k is the first k whose next draft adds less than min_gain tokens per step."""
    ks = sorted(set(tokens_per_step) & set(step_seconds))
    if not ks:
        raise ValueError("no k with both a tokens-per-step value and a step time")
    tps = {k: tokens_per_step[k] / step_seconds[k] for k in ks}
    best = max(ks, key=lambda k: (tps[k], -k))
    plateau = ks[-1]
    for a, b in zip(ks, ks[1:]):
        if tokens_per_step[b] - tokens_per_step[a] < min_gain:
            plateau = a
            break
    return KChoice(best, plateau, {k: tokens_per_step[k] for k in ks}, tps)
