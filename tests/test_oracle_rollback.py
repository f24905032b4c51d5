"""Pins of the oracle's tape replay and conv-state rollback.

The invariants: replaying n accepted tape entries onto the snapshot equals a
fresh verify over those n tokens; the closed-form rank-n sum agrees; n = 0 is
the identity; the conv window equals the last K-1 accepted raw rows; and a
speculative round followed by rollback continues exactly like plain decoding
of the accepted tokens.  The two failure modes of the pages' Exp. 7 (keeping
the post-verify state, restoring without replay) are shown to diverge.
"""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_verify_gdn_amd import workload as W

from test_oracle_delta import inputs_f64, shape_of, tiny_cfg


def rel_fro(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("n", [0, 1, 3, 7])
def test_replay_equals_fresh_recompute(oracle_mod, n):
    cfg = tiny_cfg(T=7)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    full = oracle.verify_chunk(sh, **inp)
    Sn = oracle.tape_rollback(sh, inp["S0"], full["u"], full["k"], full["g"],
                              np.full(cfg.B, n, np.int32))
    if n == 0:
        np.testing.assert_array_equal(Sn, inp["S0"])
        return
    sub = dict(inp)
    for key in ("x", "a", "b"):
        sub[key] = inp[key][:, :, :n]
    fresh = oracle.verify_chunk(sh, **sub)
    np.testing.assert_array_equal(Sn, fresh["S_final"])
    if n == cfg.T:
        np.testing.assert_array_equal(Sn, full["S_final"])


def test_replay_per_sequence_lengths(oracle_mod):
    cfg = tiny_cfg(T=6, B=3)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    full = oracle.verify_chunk(sh, **inp)
    n = np.array([0, 4, 6], np.int32)
    Sn = oracle.tape_rollback(sh, inp["S0"], full["u"], full["k"], full["g"], n)
    for b in range(cfg.B):
        if n[b] == 0:
            np.testing.assert_array_equal(Sn[:, b], inp["S0"][:, b])
            continue
        sub = {key: (v[:, b:b + 1] if key != "conv_w" else v) for key, v in inp.items()}
        for key in ("x", "a", "b"):
            sub[key] = sub[key][:, :, :n[b]]
        fresh = oracle.verify_chunk(shape_of(cfg, B=1), **sub)
        np.testing.assert_array_equal(Sn[:, b], fresh["S_final"][:, 0])


def test_replay_closed_form(oracle_mod):
    """S_n = (prod_{j<n} a_j) S0 + sum_{i<n} (prod_{i<j<n} a_j) u_i k_i^T."""
    cfg = tiny_cfg(T=8)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    full = oracle.verify_chunk(sh, **inp)
    hk = np.arange(cfg.Hv) * cfg.Hk // cfg.Hv
    for n in range(1, cfg.T + 1):
        Sn = oracle.tape_rollback(sh, inp["S0"], full["u"], full["k"], full["g"],
                                  np.full(cfg.B, n, np.int32))
        a = inp["a"]
        ref = np.prod(a[:, :, :n], axis=2)[..., None, None] * inp["S0"]
        for i in range(n):
            w = np.prod(a[:, :, i + 1:n], axis=2)  # [L,B,Hv]
            ref = ref + w[..., None, None] * np.einsum(
                "lbhi,lbhj->lbhij", full["u"][:, :, i], full["k"][:, :, i][:, :, hk])
        np.testing.assert_allclose(Sn, ref, rtol=1e-12, atol=1e-14)


def test_tree_path_replay_equals_node_state(oracle_mod):
    cfg = tiny_cfg(T=20, L=1, B=2)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    rng = np.random.default_rng(23)
    par = np.stack([W.random_tree(rng, cfg.T, 4, 8) for _ in range(cfg.B)])
    tr = oracle.tree_verify(sh, par, **inp, want_node_states=True)
    leaf = [cfg.T - 1, int(np.flatnonzero(par[1] >= 0)[-1])]
    path = np.full((cfg.B, cfg.T), -1, np.int32)
    n = np.zeros(cfg.B, np.int32)
    for b in range(cfg.B):
        chain = []
        cur = leaf[b]
        while cur >= 0:
            chain.append(cur)
            cur = par[b][cur]
        chain.reverse()
        path[b, :len(chain)] = chain
        n[b] = len(chain)
    Sn = oracle.tape_rollback(sh, inp["S0"], tr["u"], tr["k"], tr["g"], n, path)
    for b in range(cfg.B):
        np.testing.assert_allclose(Sn[:, b], tr["S_nodes"][:, b, leaf[b]], rtol=1e-13, atol=1e-15)


def test_exp7_failure_modes_diverge(oracle_mod):
    """Keeping the post-verify state (no rollback) or restoring the snapshot
    without replay both leave a state far from the correct S_n."""
    cfg = tiny_cfg(T=4, B=1, L=1, Hk=1, Hv=2, Dk=16, Dv=16, dtype=torch.bfloat16)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    full = oracle.verify_chunk(sh, **inp)
    n = np.array([2], np.int32)
    Sn = oracle.tape_rollback(sh, inp["S0"], full["u"], full["k"], full["g"], n)
    assert rel_fro(full["S_final"], Sn) > 1e-2     # v1: rejected tokens leak in
    assert rel_fro(inp["S0"], Sn) > 1e-2           # v3: accepted tokens lost


@pytest.mark.parametrize("n", [0, 1, 2, 3, 5, 6])
def test_conv_rollback_chain(oracle_mod, n):
    cfg = tiny_cfg(T=6, K=4)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    cs, win = oracle.conv_rollback(sh, inp["conv_state"], inp["x"], np.full(cfg.B, n, np.int32))
    K = cfg.K
    for l in range(cfg.L):
        for b in range(cfg.B):
            xt = np.concatenate([inp["conv_state"][l, b], inp["x"][l, b, :n]], axis=0)
            np.testing.assert_array_equal(cs[l, b], xt[-(K - 1):])
    for b in range(cfg.B):
        assert list(win[b]) == [n + j - (K - 1) for j in range(K - 1)]


def test_conv_rollback_path(oracle_mod):
    cfg = tiny_cfg(T=12, K=4, B=2)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    path = np.full((cfg.B, cfg.T), -1, np.int32)
    path[0, :1] = [5]
    path[1, :4] = [0, 3, 7, 11]
    n = np.array([1, 4], np.int32)
    cs, win = oracle.conv_rollback(sh, inp["conv_state"], inp["x"], n, path)
    for b in range(cfg.B):
        ext = list(range(-(cfg.K - 1), 0)) + list(path[b, :n[b]])
        assert list(win[b]) == ext[-(cfg.K - 1):]
        for l in range(cfg.L):
            xt = np.concatenate([inp["conv_state"][l, b], inp["x"][l, b, path[b, :n[b]]]], axis=0)
            np.testing.assert_array_equal(cs[l, b], xt[-(cfg.K - 1):])


@pytest.mark.parametrize("n", [0, 2, 5])
def test_round_with_rollback_continues_like_plain_decoding(oracle_mod, n):
    """verify(T1) -> rollback(n) -> verify(T2) == verify over x1[:n] ++ x2."""
    cfg = tiny_cfg(T=5)
    sh = shape_of(cfg)
    r1 = inputs_f64(cfg, rnd=1)
    r2 = inputs_f64(cfg, rnd=2)
    v1 = oracle.verify_chunk(sh, **r1)
    nk = np.full(cfg.B, n, np.int32)
    S = oracle.tape_rollback(sh, r1["S0"], v1["u"], v1["k"], v1["g"], nk)
    cs, _ = oracle.conv_rollback(sh, r1["conv_state"], r1["x"], nk)
    nxt = dict(r2, S0=S, conv_state=cs, conv_w=r1["conv_w"])
    v2 = oracle.verify_chunk(sh, **nxt)
    cat = dict(r1)
    for key in ("x", "a", "b"):
        cat[key] = np.concatenate([r1[key][:, :, :n], r2[key]], axis=2)
    ref = oracle.verify_chunk(sh, **cat)
    np.testing.assert_allclose(v2["o"], ref["o"][:, :, n:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(v2["S_final"], ref["S_final"], rtol=1e-12, atol=1e-14)


def test_rollback_rejects_bad_lengths(oracle_mod):
    cfg = tiny_cfg(T=4, B=1)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    full = oracle.verify_chunk(sh, **inp)
    with pytest.raises(ValueError):
        oracle.tape_rollback(sh, inp["S0"], full["u"], full["k"], full["g"],
                             np.array([5], np.int32))
    with pytest.raises(ValueError):
        oracle.conv_rollback(sh, inp["conv_state"], inp["x"], np.array([-1], np.int32))
