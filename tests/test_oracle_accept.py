"""Pins of the oracle's greedy acceptance (chain and tree).

Brute force enumerates prefixes / root paths on tiny inputs; hand cases follow
the accept loop of xserv "Phase 25" s2 (longest matching prefix, correction =
target argmax at the stop position); ties go to the lowest token index.
"""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_verify_gdn_amd import workload as W


def brute_chain(draft, logits):
    T = len(draft)
    best = 0
    for m in range(T + 1):  # every prefix length; keep the longest fully matching
        if all(draft[j] == int(np.argmax(logits[j])) for j in range(m)):
            best = m
    return best, int(np.argmax(logits[best]))


def brute_tree(parent, draft, logits):
    """All maximal root paths whose every step matches the argmax of the row
    before it; the lexicographically smallest node sequence is the answer."""
    T = len(draft)
    children = {v: [c for c in range(T) if parent[c] == v] for v in range(-1, T)}

    def valid_paths(cur, acc):
        row = logits[cur + 1]
        star = int(np.argmax(row))
        ext = [c for c in children[cur] if draft[c] == star]
        if not ext:
            return [(acc, star)]
        out = []
        for c in ext:
            out += valid_paths(c, acc + [c])
        return out

    paths = valid_paths(-1, [])
    paths.sort(key=lambda p: p[0])
    return paths[0]


def test_hand_cases():
    V = 6
    lg = np.zeros((1, 4, V))
    for r, t in enumerate([2, 4, 1, 5]):
        lg[0, r, t] = 1.0
    cases = [([2, 4, 1], 3, 5), ([2, 4, 0], 2, 1), ([3, 4, 1], 0, 2), ([2, 0, 1], 1, 4)]
    for dr, n, bonus in cases:
        nk, path, bo = oracle.accept(np.array([dr]), lg)
        assert nk[0] == n and bo[0] == bonus
        assert list(path[0]) == list(range(n)) + [-1] * (3 - n)


def test_ties_take_lowest_index():
    lg = np.zeros((1, 2, 8))
    lg[0, 0, [5, 2, 7]] = 3.0
    lg[0, 1, [1, 6]] = 2.0
    nk, _, bo = oracle.accept(np.array([[2]]), lg)
    assert nk[0] == 1 and bo[0] == 1
    nk, _, bo = oracle.accept(np.array([[5]]), lg)
    assert nk[0] == 0 and bo[0] == 2


@pytest.mark.parametrize("seed", range(6))
def test_chain_bruteforce(seed):
    rng = np.random.default_rng(seed)
    B, T, V = 40, 5, 4
    logits = rng.integers(-2, 3, size=(B, T + 1, V)).astype(np.float64)  # many ties
    draft = rng.integers(0, V, size=(B, T))
    nk, path, bo = oracle.accept(draft, logits)
    for b in range(B):
        n, bonus = brute_chain(draft[b], logits[b])
        assert nk[b] == n and bo[b] == bonus
        assert list(path[b, :n]) == list(range(n)) and np.all(path[b, n:] == -1)


@pytest.mark.parametrize("seed", range(6))
def test_tree_bruteforce_with_duplicate_siblings(seed):
    rng = np.random.default_rng(100 + seed)
    B, T, V = 30, 12, 3
    parent = np.stack([W.random_tree(rng, T, 4, 5) for _ in range(B)])
    logits = rng.integers(-1, 2, size=(B, T + 1, V)).astype(np.float64)
    draft = rng.integers(0, V, size=(B, T))  # duplicates among siblings on purpose
    nk, path, bo = oracle.accept(draft, logits, parent)
    for b in range(B):
        p, bonus = brute_tree(parent[b], draft[b], logits[b])
        assert nk[b] == len(p) and bo[b] == bonus
        assert list(path[b, :nk[b]]) == p and np.all(path[b, nk[b]:] == -1)


def test_chain_equals_tree_with_chain_parents():
    rng = np.random.default_rng(9)
    B, T, V = 50, 7, 5
    logits = rng.standard_normal((B, T + 1, V))
    tg = logits.argmax(-1)
    draft = np.where(rng.random((B, T)) < 0.7, tg[:, :T], rng.integers(0, V, (B, T)))
    par = np.tile(np.arange(T) - 1, (B, 1))
    a = oracle.accept(draft, logits)
    b = oracle.accept(draft, logits, par)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("law", ["uniform", "bernoulli"])
def test_generator_plants_requested_chain_lengths(law):
    cfg = W.CONFIGS[3].with_(law=law, B=64, V=1000)
    d = W.chain_accept_inputs(cfg, rnd=3)
    nk, path, bo = oracle.accept(d["draft"].numpy(), W.to_f64(d["logits"]))
    np.testing.assert_array_equal(nk, d["n_planted"])
    np.testing.assert_array_equal(bo, d["targets"][np.arange(cfg.B), nk])


def test_generator_plants_requested_tree_paths():
    cfg = W.CONFIGS[5].with_(B=16, V=2000)
    d = W.tree_accept_inputs(cfg, rnd=1)
    nk, path, bo = oracle.accept(d["draft"].numpy(), W.to_f64(d["logits"]), d["parent"].numpy())
    np.testing.assert_array_equal(nk, d["n_planted"])
    np.testing.assert_array_equal(path, d["planted_path"])


def _nan_rule_argmax(row):
    """numpy's NaN-skipping first-maximum; a row with no number gives 0."""
    row = np.asarray(row, dtype=np.float64)
    return 0 if np.all(np.isnan(row)) else int(np.nanargmax(row))


@pytest.mark.parametrize("tree", [False, True])
def test_infinite_and_nan_logits(tree):
    """Rows of -inf, -inf padding, +inf entries and NaN entries: the argmax is
    numpy's NaN-skipping first maximum (np.nanargmax), -inf rows give 0, a row
    of NaN gives 0; the walk then follows the same rule as for finite rows."""
    rng = np.random.default_rng(21 if tree else 20)
    B, T, V = 40, 6, 9
    logits = rng.integers(-2, 3, size=(B, T + 1, V)).astype(np.float64)
    kinds = rng.integers(0, 6, size=(B, T + 1))
    for b in range(B):
        for r in range(T + 1):
            k = kinds[b, r]
            if k == 1:
                logits[b, r, :] = -np.inf
            elif k == 2:
                logits[b, r, rng.integers(1, V):] = -np.inf   # -inf padded tail
            elif k == 3:
                logits[b, r, rng.integers(0, V, size=3)] = np.nan
            elif k == 4:
                logits[b, r, :] = np.nan
            elif k == 5:
                logits[b, r, rng.integers(0, V, size=2)] = np.inf
    star = np.array([[_nan_rule_argmax(logits[b, r]) for r in range(T + 1)] for b in range(B)])
    draft = np.where(rng.random((B, T)) < 0.8, star[:, :T], rng.integers(0, V, (B, T)))
    parent = np.stack([W.random_tree(rng, T, 3, 4) for _ in range(B)]) if tree else None
    nk, path, bo = oracle.accept(draft, logits, parent)
    nanfree = np.where(np.isnan(logits), -np.inf, logits)  # NaN never wins
    for b in range(B):
        assert all(star[b, r] == (0 if np.all(np.isnan(logits[b, r]))
                                  else int(np.argmax(nanfree[b, r])))
                   for r in range(T + 1))
        if tree:
            # the brute-force walk with the same argmax rule
            lg = np.where(np.isnan(logits[b]), -np.inf, logits[b])
            p, bonus = brute_tree(parent[b], draft[b], lg)
        else:
            m = 0
            while m < T and draft[b, m] == star[b, m]:
                m += 1
            p, bonus = list(range(m)), star[b, m]
        assert nk[b] == len(p) and bo[b] == bonus
        assert list(path[b, :nk[b]]) == list(p)
    assert oracle.accept(np.zeros((1, 1), np.int32), np.full((1, 2, 5), -np.inf))[2][0] == 0
    assert oracle.accept(np.zeros((1, 1), np.int32), np.full((1, 2, 5), np.nan))[2][0] == 0
