"""Host-side draft-length policy (speculative_decode_verify_gdn_amd.policy).

Pinned against the pages' printed figures (tests/golden), the oracle's
independent cost-model functions, the statistics of simulated acceptance,
and colibri's guard rule (s4.1: acc * 10 < proposed after >= 24 proposals).
"""
import json
import os

import numpy as np
import pytest

import oracle.cost_model as cm
from speculative_decode_verify_gdn_amd import policy as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_closed_forms.json")


def test_expected_committed_matches_pages_and_oracle():
    """The X article's 1.6x (36%, N=4) and 2x (50%, N=4) are expected committed
    tokens per round; the closed form agrees with the oracle's sum."""
    entries = {e["id"]: e for e in json.load(open(GOLDEN))["entries"]}
    for key in ("pure_attn_036_n4", "pure_attn_050_n4"):
        e = entries[key]
        assert abs(P.expected_committed(*e["args"]) - e["printed"]) <= e["tol"], key
    for a in (0.0, 0.15, 0.36, 0.5, 0.85, 0.999, 1.0):
        for n in range(0, 17):
            assert P.expected_committed(a, n) == pytest.approx(cm.expected_committed_per_round(a, n),
                                                               rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("alpha,n", [(0.36, 8), (0.85, 16), (0.15, 4), (0.97, 4)])
def test_alpha_estimate_recovers_the_law(alpha, n):
    """Accepted lengths drawn from the truncated geometric law of the pages'
    Bernoulli acceptance give back alpha (maximum likelihood)."""
    rng = np.random.default_rng(int(alpha * 1000) + n)
    st = P.AcceptanceStats()
    for _ in range(400):
        match = rng.random((64, n)) < alpha
        keep = np.where(match.all(1), n, np.argmin(match, 1))
        st.update(keep, n)
    assert abs(st.alpha() - alpha) < 0.01
    assert st.proposed == 400 * 64 * n


def test_alpha_edge_cases_and_validation():
    st = P.AcceptanceStats()
    assert st.alpha() is None
    st.update([4, 4, 4], 4)           # nothing rejected
    assert st.alpha() == 1.0
    st2 = P.AcceptanceStats()
    st2.update([0, 0], 8)             # every first draft rejected
    assert st2.alpha() == 0.0
    with pytest.raises(ValueError):
        st2.update([9], 8)


def test_guard_follows_colibri_rule():
    st = P.AcceptanceStats()
    st.update([0] * 5 + [2], 4)       # 24 proposed, 2 accepted: 20 < 24
    assert st.proposed == 24 and st.guard_disables()
    st = P.AcceptanceStats()
    st.update([0] * 23, 1)            # 23 proposed: too early to judge
    assert not st.guard_disables()
    st = P.AcceptanceStats()
    st.update([1, 1, 1] + [0] * 27, 1)  # 30 proposed, 3 accepted: 30 < 30 is false
    assert not st.guard_disables()


def test_choose_draft_length():
    # constant round cost (pure attention): more drafts always help
    flat = {n: 100.0 for n in (1, 2, 4, 8, 16)}
    assert P.choose_draft_length(0.36, flat) == 16
    # nothing is ever accepted: the cheapest option wins, a plain step if given
    lin = {n: 100.0 + 10.0 * n for n in (1, 2, 4, 8, 16)}
    assert P.choose_draft_length(0.0, lin) == 1
    assert P.choose_draft_length(0.0, lin, t_plain_us=90.0) == 0
    # GDN-like cost growing with N: a moderate N at 36%, a long one at 97%
    gdn = {n: 0.25 + 0.75 * (n + 1) for n in range(1, 17)}
    n36 = P.choose_draft_length(0.36, gdn, t_plain_us=1.0)
    n97 = P.choose_draft_length(0.97, gdn, t_plain_us=1.0)
    assert n36 == 0                   # sequential GDN cost: drafting loses at 36%
    assert n97 > 1
    # the chosen N maximises committed tokens per unit time over the table
    for a in (0.2, 0.5, 0.8, 0.95):
        nb = P.choose_draft_length(a, lin)
        rates = {n: cm.expected_committed_per_round(a, n) / t for n, t in lin.items()}
        assert rates[nb] == max(rates.values())


def test_policy_prior_then_guard():
    pol = P.DraftPolicy(t_round_us={n: 100.0 + 5.0 * n for n in (1, 2, 4, 8)}, t_plain_us=95.0,
                        prior_alpha=0.8)
    first = pol.next_draft_length()
    assert first > 0
    for _ in range(10):
        pol.record(np.zeros(8, dtype=np.int32), first)
    assert pol.next_draft_length() == 0
