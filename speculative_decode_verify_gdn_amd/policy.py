"""Draft-length policy for speculative rounds (host side, no kernels).

Two rules from the pages, applied to measured round times:

* Choosing N.  A round that verifies N drafted tokens commits the accepted
  prefix plus one correction token.  With independent per-position acceptance
  alpha, the expected number committed is sum_{k=0..N} alpha**k (the
  closed form behind the X article's 1.6x / 2x figures, Exps. 5-6), and
  the round costs t_round(N).  The verify-cost analysis of "Speculative
  Decoding on GDN Hybrid Architectures" (s2.2) models that cost as growing
  with N because the recurrent layers are sequential; here t_round(N) is the
  measured time of the whole round instead of the modelled one.  The policy
  picks the N with the most committed tokens per second, and N = 0 (no
  drafting, one token per step) when a plain step is faster.
* Adaptive disable.  colibri "MTP speculative decoding and prefetch" s4.1:
  once at least 24 drafts have been proposed, drafting stops if fewer than
  one in ten was accepted.

alpha is estimated from the accepted-prefix lengths: each round contributes
n accepted positions and, when n < N, one rejection, so the maximum-likelihood
estimate of a truncated geometric law is sum(n) / (sum(n) + rejections).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

GUARD_MIN_PROPOSED = 24   # colibri s4.1: proposals before the guard may fire


def expected_committed(alpha: float, n: int) -> float:
    """E[accepted prefix + correction token] for n drafts at acceptance alpha."""
    if n <= 0:
        return 1.0
    if alpha == 1.0:
        return float(n + 1)
    return (1.0 - alpha ** (n + 1)) / (1.0 - alpha)


@dataclass
class AcceptanceStats:
    """Running counts of proposed drafts, accepted drafts and rejections."""
    proposed: int = 0
    accepted: int = 0
    rejections: int = 0

    def update(self, n_keep, n_drafts: int) -> None:
        """Add one round: n_keep holds each sequence's accepted length (a host
        array or a device tensor, read once here)."""
        n = np.asarray(n_keep.cpu() if hasattr(n_keep, "cpu") else n_keep, dtype=np.int64)
        if n.size and (n.min() < 0 or n.max() > n_drafts):
            raise ValueError("accepted lengths outside [0, %d]" % n_drafts)
        self.proposed += int(n.size) * int(n_drafts)
        self.accepted += int(n.sum())
        self.rejections += int(np.count_nonzero(n < n_drafts))

    def alpha(self) -> Optional[float]:
        """Maximum-likelihood per-position acceptance, or None before any data."""
        seen = self.accepted + self.rejections
        if seen == 0:
            return None
        return self.accepted / seen

    def guard_disables(self) -> bool:
        """colibri s4.1: at least 24 proposals and accepted * 10 < proposed."""
        return self.proposed >= GUARD_MIN_PROPOSED and self.accepted * 10 < self.proposed


def choose_draft_length(alpha: float, t_round_us: Dict[int, float],
                        t_plain_us: Optional[float] = None) -> int:
    """The N (a key of t_round_us, or 0 for a plain step costing t_plain_us)
    with the highest expected committed tokens per microsecond; ties go to
    the smaller N."""
    best_n, best = 0, (1.0 / t_plain_us) if t_plain_us else -1.0
    for n in sorted(t_round_us):
        rate = expected_committed(alpha, n) / t_round_us[n]
        if rate > best * (1 + 1e-12):
            best_n, best = n, rate
    return best_n


@dataclass
class DraftPolicy:
    """Picks the draft length for the next round from measured round times
    and the acceptance seen so far; `prior_alpha` is used before any round."""
    t_round_us: Dict[int, float]
    t_plain_us: Optional[float] = None
    prior_alpha: float = 0.5
    stats: AcceptanceStats = field(default_factory=AcceptanceStats)

    def record(self, n_keep, n_drafts: int) -> None:
        self.stats.update(n_keep, n_drafts)

    def next_draft_length(self) -> int:
        if self.stats.guard_disables():
            return 0
        a = self.stats.alpha()
        return choose_draft_length(self.prior_alpha if a is None else a, self.t_round_us,
                                   self.t_plain_us)
