"""Pins of the oracle's rejection-sampling acceptance (oracle.accept_sample).

Rule: colibri "MTP speculative decoding and prefetch" s5 -- a point-mass
draft token d is kept with probability p(d); after a rejection the output
token is drawn from p with d removed and renormalised, which makes the output
distribution exactly p.  Each pin below fails for a plausible mistake: a
reversed acceptance test, a missing removal of the rejected token, a missing
renormalisation, a wrong row, a temperature applied the wrong way.
"""
import math

import numpy as np
import pytest

import oracle


def _grid(n):
    return (np.arange(n) + 0.5) / n


def _first_token_distribution(logits, draft, tau, n):
    """Distribution of the first emitted token over an n x n midpoint grid of
    (u_0, u_T): the draft token if kept, else the drawn token.  T = 1."""
    V = logits.shape[-1]
    u0, u1 = np.meshgrid(_grid(n), _grid(n), indexing="ij")
    B = n * n
    uni = np.stack([u0.ravel(), u1.ravel()], 1)
    lg = np.broadcast_to(logits, (B, 2, V))
    dr = np.full((B, 1), draft)
    nk, _, tok = oracle.accept_sample(dr, lg, tau, uni)
    first = np.where(nk >= 1, draft, tok)
    return np.bincount(first, minlength=V) / B


@pytest.mark.parametrize("draft,tau", [(0, 1.0), (3, 1.0), (1, 0.7), (4, 2.5)])
def test_first_output_token_has_distribution_p(draft, tau):
    """The page's lossless claim, by quadrature over the two uniforms: the
    first emitted token is distributed exactly as p = softmax(logits / tau).
    Grid error per cell edge is at most 1/n per dimension."""
    rng = np.random.default_rng(11)
    logits = np.zeros((2, 5))
    logits[0] = rng.normal(size=5) * 1.5
    p = np.exp(logits[0] / tau - (logits[0] / tau).max())
    p /= p.sum()
    n = 240
    freq = _first_token_distribution(logits, draft, tau, n)
    assert np.max(np.abs(freq - p)) <= 2.5 / n, (freq, p)


def test_hand_computed_case():
    """p = (1/6, 2/6, 3/6) at temperature 1 (logits 0, ln 2, ln 3)."""
    lg = np.array([[[0.0, math.log(2), math.log(3)], [0.0, 0.0, 0.0]]])
    # draft 2 (p = 1/2): u = 0.4 keeps it, the bonus row is uniform over 3
    nk, path, tok = oracle.accept_sample([[2]], lg, 1.0, [[0.4, 0.5]])
    assert nk[0] == 1 and path[0, 0] == 0 and tok[0] == 1   # 0.5 * 3 = 1.5 -> index 1
    # u = 0.6 rejects it; q = (1/6, 2/6, 0): threshold 0.3 * 1/2 = 0.15 < 1/6 -> 0
    nk, path, tok = oracle.accept_sample([[2]], lg, 1.0, [[0.6, 0.3]])
    assert nk[0] == 0 and path[0, 0] == -1 and tok[0] == 0
    # threshold 0.5 * 1/2 = 0.25 > 1/6 -> 1; never the rejected token
    nk, _, tok = oracle.accept_sample([[2]], lg, 1.0, [[0.6, 0.5]])
    assert nk[0] == 0 and tok[0] == 1
    nk, _, tok = oracle.accept_sample([[2]], lg, 1.0, [[0.6, 0.999]])
    assert tok[0] == 1
    # temperature 2 flattens: p(2) = sqrt3 / (1 + sqrt2 + sqrt3) = 0.4185
    nk, _, _ = oracle.accept_sample([[2]], lg, 2.0, [[0.41, 0.0]])
    assert nk[0] == 1
    nk, _, _ = oracle.accept_sample([[2]], lg, 2.0, [[0.42, 0.0]])
    assert nk[0] == 0


def test_low_temperature_is_the_greedy_accept():
    """As temperature -> 0, p becomes the point mass on the argmax: the kept
    prefix and the output token equal the (independent, C) greedy oracle's
    n_keep and bonus, whenever the top two logits are separated."""
    rng = np.random.default_rng(5)
    B, T, V = 40, 6, 50
    logits = rng.normal(size=(B, T + 1, V))
    star = logits.argmax(-1)
    logits[np.arange(B)[:, None], np.arange(T + 1)[None, :], star] += 1.0  # gap >= 1
    n_true = rng.integers(0, T + 1, size=B)
    draft = star[:, :T].copy()
    for b in range(B):
        if n_true[b] < T:
            draft[b, n_true[b]] = (star[b, n_true[b]] + 1 + rng.integers(0, V - 1)) % V
            draft[b, n_true[b] + 1:] = rng.integers(0, V, size=T - n_true[b] - 1)
    uni = rng.uniform(0.0, 0.999, size=(B, T + 1))
    nk_s, path_s, tok_s = oracle.accept_sample(draft, logits, 0.01, uni)
    nk_g, path_g, bonus_g = oracle.accept(draft, logits)
    np.testing.assert_array_equal(nk_s, nk_g)
    np.testing.assert_array_equal(path_s, path_g)
    np.testing.assert_array_equal(tok_s, bonus_g)


def test_uniform_extremes_and_invalid_tokens():
    rng = np.random.default_rng(9)
    B, T, V = 6, 5, 30
    logits = rng.normal(size=(B, T + 1, V))
    draft = rng.integers(0, V, size=(B, T))
    # u = 0 keeps every draft of positive probability; the draw takes index 0
    nk, _, tok = oracle.accept_sample(draft, logits, 1.0, np.zeros((B, T + 1)))
    assert (nk == T).all() and (tok == 0).all()
    # a draft outside [0, V) is never kept and removes nothing
    bad = draft.copy()
    bad[:, 2] = V + 3
    nk, _, tok, pd = oracle.accept_sample(bad, logits, 1.0, np.zeros((B, T + 1)), detail=True)
    assert (nk == 2).all() and (tok == 0).all() and (pd[:, 2] == 0).all()
    # u just below 1 rejects the first draft unless it holds all the mass;
    # the draw then takes the last index of positive mass other than it
    nk, _, tok = oracle.accept_sample(draft, logits, 1.0, np.full((B, T + 1), 1 - 1e-12))
    assert (nk == 0).all()
    for b in range(B):
        assert tok[b] == (V - 1 if draft[b, 0] != V - 1 else V - 2)


def test_draws_follow_the_residual_cdf():
    """Every draw satisfies the inverse-CDF definition on its row."""
    rng = np.random.default_rng(3)
    B, T, V = 30, 4, 97
    logits = rng.normal(size=(B, T + 1, V)) * 2
    draft = rng.integers(0, V, size=(B, T))
    uni = rng.uniform(size=(B, T + 1))
    nk, _, tok, pd = oracle.accept_sample(draft, logits, 0.8, uni, detail=True)
    for b in range(B):
        n = nk[b]
        for j in range(n):
            assert uni[b, j] < pd[b, j]
        if n < T:
            assert uni[b, n] >= pd[b, n]
        ban = int(draft[b, n]) if n < T else -1
        c = oracle.sample_cdf(logits[b, n], 0.8, ban)
        i = tok[b]
        target = uni[b, T] * c[-1]
        assert c[i] > target and (i == 0 or c[i - 1] <= target)
        assert i != ban
