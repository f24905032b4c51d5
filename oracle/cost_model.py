"""Closed forms the pages give for the verify-cost model and acceptance statistics.

TEST INFRASTRUCTURE ONLY (part of the oracle): the benchmark prints these
beside its measurements as a sanity check; nothing on the GPU path uses them.

Sources:
  "Speculative Decoding on GDN Hybrid Architectures: A 31-Experiment
  Investigation", s2.2 (verify-cost floor): in a hybrid of 25% attention
  layers (parallel over N tokens) and 75% GDN layers (sequential), verifying N
  tokens costs 0.25 + 0.75*N single-token units, so the best speedup at 100%
  acceptance is N / (0.25 + 0.75*N), which tends to 4/3 as N grows.  The page
  prints the ceiling as 1/(0.25 + 0.75/N); that expression tends to 4, not to
  the stated 1.33, and contradicts the stated cost, so the consistent form is
  used and the printed one is only reported beside it.
  Same page, s3 (Exp. 7-8 and Exp. 15): the chance that all N drafts match at
  per-position acceptance alpha is alpha**N (27% at 85%/8, 1.7% at 36%/4,
  0.05% at 15%/4).
  Curated X article by Tom Turney (easyvibecoding), Exp. 5-6: 36% acceptance
  with N=4 drafts gives about 1.6x on a pure-attention model, and 50% is needed
  for 2x; both equal the expected committed tokens per round,
  sum_{k=0..N} alpha**k = (1 - alpha**(N+1)) / (1 - alpha).

Parity: the printed numbers pin these functions (tests/golden/); the page's
0.6x effective speedup at 36%/N=4 for the GDN hybrid and the "weighted 3.2x"
have no derivation on the pages and stay unpinned.
"""
from __future__ import annotations


def verify_cost_units(n: int, attn_frac: float = 0.25) -> float:
    """Cost of verifying n tokens in single-token units: attention is paid once,
    the recurrent (GDN) share is paid per token."""
    return attn_frac + (1.0 - attn_frac) * n


def verify_ceiling(n: int, attn_frac: float = 0.25) -> float:
    """Best speedup at 100% acceptance: n tokens per verify of cost verify_cost_units(n)."""
    return n / verify_cost_units(n, attn_frac)


def verify_ceiling_as_printed(n: int) -> float:
    """The page's printed expression 1/(0.25 + 0.75/n) (reported only)."""
    return 1.0 / (0.25 + 0.75 / n)


def p_all_match(alpha: float, n: int) -> float:
    """Probability that all n drafts are accepted with independent per-position acceptance alpha."""
    return alpha ** n


def p_accept_exactly(alpha: float, n: int, k: int) -> float:
    """P(accepted prefix length == k) for k in 0..n (geometric, truncated at n)."""
    if k < 0 or k > n:
        return 0.0
    if k == n:
        return alpha ** n
    return alpha ** k * (1.0 - alpha)


def expected_committed_per_round(alpha: float, n: int) -> float:
    """E[accepted + 1 correction token] = sum_{k=0..n} alpha**k."""
    return sum(alpha ** k for k in range(n + 1))


def expected_accepted(alpha: float, n: int) -> float:
    """E[accepted prefix length] = sum_{k=1..n} alpha**k."""
    return sum(alpha ** k for k in range(1, n + 1))
