"""Pin the cost-model and acceptance closed forms to the numbers the pages print."""
import json
import os

import numpy as np
import pytest

from oracle import cost_model as cm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_closed_forms.json")


def _entries():
    with open(GOLDEN) as f:
        return json.load(f)["entries"]


@pytest.mark.parametrize("e", _entries(), ids=lambda e: e["id"])
def test_printed_values(e):
    val = getattr(cm, e["fn"])(*e["args"])
    assert abs(val - e["printed"]) <= e["tol"], (e["id"], val, e["cite"])


def test_ceiling_consistent_form():
    # cost 0.25 + 0.75 N and "pure attention -> N x": the ceiling must be
    # increasing in N, bounded by 4/3, and equal 1 at N = 1.
    vals = [cm.verify_ceiling(n) for n in range(1, 65)]
    assert abs(vals[0] - 1.0) < 1e-15
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert max(vals) < 4.0 / 3.0
    assert abs(cm.verify_ceiling(4) - 16.0 / 13.0) < 1e-15
    # pure attention (attn_frac = 1) has ceiling N
    assert cm.verify_ceiling(8, attn_frac=1.0) == 8.0
    # the printed expression tends to 4, which contradicts the stated 1.33x limit
    assert abs(cm.verify_ceiling_as_printed(10 ** 9) - 4.0) < 1e-6


def test_geometric_law_sums_to_one():
    for a in (0.15, 0.36, 0.85):
        for n in (4, 8, 16):
            ps = [cm.p_accept_exactly(a, n, k) for k in range(n + 1)]
            assert abs(sum(ps) - 1.0) < 1e-12
            ek = sum(k * p for k, p in enumerate(ps))
            assert abs(ek - cm.expected_accepted(a, n)) < 1e-12
            assert abs(cm.expected_committed_per_round(a, n) - (1 - a ** (n + 1)) / (1 - a)) < 1e-12
