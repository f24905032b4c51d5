"""Pins of the oracle's per-key-channel decay form (verify_chunk_vg,
tape_rollback_vg): the [B,T,Hv,Dk] decay tape of the GDN page, s4, under
which the state decays column by column, S <- S diag(a_t) + u_t k_t^T with
u_t = b_t (v_t - S diag(a_t) k_t).

Each pin fails for a plausible mistake: decaying rows instead of columns, a
transposed gate, the decay applied after the update, a missing b, the tape
replayed in the wrong order."""
import numpy as np
import pytest

import oracle

SH = oracle.Shape(L=2, B=2, Hk=2, Hv=4, Dk=8, Dv=6, K=3, silu=True, eps=1e-6)


def _inputs(sh, T, seed, gate_lo=0.3):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(sh.L, sh.B, T, sh.C))
    cs = rng.normal(size=(sh.L, sh.B, sh.K - 1, sh.C))
    w = rng.normal(size=(sh.L, sh.C, sh.K)) / np.sqrt(sh.K)
    a = rng.uniform(gate_lo, 1.0, size=(sh.L, sh.B, T, sh.Hv, sh.Dk))
    b = rng.uniform(0.1, 1.0, size=(sh.L, sh.B, T, sh.Hv))
    S0 = rng.normal(size=(sh.L, sh.B, sh.Hv, sh.Dv, sh.Dk)) * 0.1
    return x, cs, w, a, b, S0


def test_equal_channel_gates_reduce_to_the_scalar_form():
    x, cs, w, a, b, S0 = _inputs(SH, 7, 1)
    a_s = a[..., 0]
    a_v = np.repeat(a_s[..., None], SH.Dk, axis=-1)
    vg = oracle.verify_chunk_vg(SH, x, cs, w, a_v, b, S0)
    sc = oracle.verify_chunk(SH, x, cs, w, a_s, b, S0, want_final=True)
    for key in ("o", "u", "k"):
        np.testing.assert_allclose(vg[key], sc[key], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(vg["S_final"], sc["S_final"], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(vg["g"], a_v)


def test_matrix_form_of_the_recurrence():
    """S_t = S_{t-1} diag(a_t) (I - b_t k_t k_t^T) + b_t v_t k_t^T, written
    with numpy matrices from the oracle's own conv/norm outputs (k, and q, v
    recovered from the chunk oracle's post-conv stream)."""
    sh = oracle.Shape(L=1, B=1, Hk=1, Hv=2, Dk=5, Dv=4, K=2)
    T = 6
    x, cs, w, a, b, S0 = _inputs(sh, T, 2)
    vg = oracle.verify_chunk_vg(sh, x, cs, w, a, b, S0)
    post = oracle.verify_chunk(sh, x, cs, w, a[..., 0], b, S0, want_final=False,
                               want_qkv_post=True)["qkv_post"]
    for hv in range(sh.Hv):
        S = S0[0, 0, hv].copy()
        for t in range(T):
            y = post[0, 0, t]
            q = y[:sh.Dk] / np.sqrt((y[:sh.Dk] ** 2).sum() + sh.eps)
            k = y[sh.Dk:2 * sh.Dk] / np.sqrt((y[sh.Dk:2 * sh.Dk] ** 2).sum() + sh.eps)
            v = y[2 * sh.Dk + hv * sh.Dv:2 * sh.Dk + (hv + 1) * sh.Dv]
            bt = b[0, 0, t, hv]
            S = S @ np.diag(a[0, 0, t, hv]) @ (np.eye(sh.Dk) - bt * np.outer(k, k)) + bt * np.outer(v, k)
            np.testing.assert_allclose(vg["o"][0, 0, t, hv], S @ q, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(vg["S_final"][0, 0, hv], S, rtol=1e-10, atol=1e-12)


def test_zero_gate_erases_its_key_column():
    """a_t[c] = 0 forgets column c of the state before step t: afterwards
    column c holds only u_t k_t[c]."""
    x, cs, w, a, b, S0 = _inputs(SH, 1, 3)
    a[..., 3] = 0.0
    vg = oracle.verify_chunk_vg(SH, x, cs, w, a, b, S0)
    for l in range(SH.L):
        for bb in range(SH.B):
            for hv in range(SH.Hv):
                hk = hv * SH.Hk // SH.Hv
                col = vg["u"][l, bb, 0, hv] * vg["k"][l, bb, 0, hk, 3]
                np.testing.assert_allclose(vg["S_final"][l, bb, hv, :, 3], col, rtol=1e-12,
                                           atol=1e-14)


@pytest.mark.parametrize("n", [0, 1, 4, 9])
def test_replay_equals_recompute_and_full_replay_equals_final(n):
    T = 9
    x, cs, w, a, b, S0 = _inputs(SH, T, 4)
    full = oracle.verify_chunk_vg(SH, x, cs, w, a, b, S0)
    nk = np.full(SH.B, n, np.int32)
    S_rep = oracle.tape_rollback_vg(SH, S0, full["u"], full["k"], full["g"], nk)
    if n == 0:
        np.testing.assert_array_equal(S_rep, S0)
        return
    part = oracle.verify_chunk_vg(SH, x[:, :, :n], cs, w, a[:, :, :n], b[:, :, :n], S0)
    np.testing.assert_allclose(S_rep, part["S_final"], rtol=1e-12, atol=1e-14)
    if n == T:
        np.testing.assert_allclose(S_rep, full["S_final"], rtol=1e-12, atol=1e-14)


def test_rollback_equal_gates_is_the_scalar_rollback():
    T = 5
    x, cs, w, a, b, S0 = _inputs(SH, T, 5)
    sc = oracle.verify_chunk(SH, x, cs, w, a[..., 0], b, S0, want_final=False)
    g_v = np.repeat(sc["g"][..., None], SH.Dk, axis=-1)
    nk = np.array([3, 5], np.int32)
    path = np.array([[0, 1, 2, -1, -1], [0, 1, 2, 3, 4]], np.int32)
    np.testing.assert_allclose(
        oracle.tape_rollback_vg(SH, S0, sc["u"], sc["k"], g_v, nk, path),
        oracle.tape_rollback(SH, S0, sc["u"], sc["k"], sc["g"], nk, path), rtol=1e-13, atol=1e-15)


# ------------------------------------------------- per-key gate over a tree --

def _tree_inputs(sh, T, seed, branching=3, depth=5):
    from speculative_decode_verify_gdn_amd import workload as W
    x, cs, w, a, b, S0 = _inputs(sh, T, seed)
    rng = np.random.default_rng(seed + 100)
    parent = np.stack([W.random_tree(rng, T, branching, depth) for _ in range(sh.B)])
    return parent, x, cs, w, a, b, S0


def test_tree_vg_equal_channel_gates_reduce_to_the_scalar_tree():
    parent, x, cs, w, a, b, S0 = _tree_inputs(SH, 9, 6)
    a_s = a[..., 0]
    a_v = np.repeat(a_s[..., None], SH.Dk, axis=-1)
    vg = oracle.tree_verify_vg(SH, parent, x, cs, w, a_v, b, S0, want_node_states=True)
    sc = oracle.tree_verify(SH, parent, x, cs, w, a_s, b, S0, want_node_states=True)
    for key in ("o", "u", "k", "S_nodes"):
        np.testing.assert_allclose(vg[key], sc[key], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(vg["conv_win"], sc["conv_win"])
    np.testing.assert_array_equal(vg["g"], a_v)


def test_tree_vg_with_chain_parents_is_the_chain():
    T = 8
    x, cs, w, a, b, S0 = _inputs(SH, T, 7)
    parent = np.tile(np.arange(-1, T - 1, dtype=np.int32), (SH.B, 1))
    tr = oracle.tree_verify_vg(SH, parent, x, cs, w, a, b, S0, want_node_states=True)
    ch = oracle.verify_chunk_vg(SH, x, cs, w, a, b, S0)
    for key in ("o", "u", "k", "g"):
        np.testing.assert_array_equal(tr[key], ch[key])
    np.testing.assert_array_equal(tr["S_nodes"][:, :, T - 1], ch["S_final"])


def test_tree_vg_node_states_match_the_matrix_form_along_each_path():
    """S_v = S_p diag(a_v) (I - b_v k_v k_v^T) + b_v v_v k_v^T from S0 along
    v's root path, with q/k/v from the pinned tree conv and numpy norms."""
    sh = oracle.Shape(L=1, B=2, Hk=1, Hv=2, Dk=5, Dv=4, K=3)
    T = 10
    parent, x, cs, w, a, b, S0 = _tree_inputs(sh, T, 8, branching=2, depth=6)
    out = oracle.tree_verify_vg(sh, parent, x, cs, w, a, b, S0, want_node_states=True)
    for bb in range(sh.B):
        y, _ = oracle.conv_tree(parent[bb], cs[0, bb], x[0, bb], w[0], silu=True)
        for hv in range(sh.Hv):
            for v in range(T):
                path = []
                c = v
                while c >= 0:
                    path.append(c)
                    c = parent[bb, c]
                S = S0[0, bb, hv].copy()
                for t in reversed(path):
                    q = y[t, :sh.Dk] / np.sqrt((y[t, :sh.Dk] ** 2).sum() + sh.eps)
                    k = y[t, sh.Dk:2 * sh.Dk] / np.sqrt((y[t, sh.Dk:2 * sh.Dk] ** 2).sum() + sh.eps)
                    vv = y[t, 2 * sh.Dk + hv * sh.Dv:2 * sh.Dk + (hv + 1) * sh.Dv]
                    bt = b[0, bb, t, hv]
                    S = (S @ np.diag(a[0, bb, t, hv]) @ (np.eye(sh.Dk) - bt * np.outer(k, k))
                         + bt * np.outer(vv, k))
                np.testing.assert_allclose(out["S_nodes"][0, bb, v, hv], S, rtol=1e-10, atol=1e-12)
                np.testing.assert_allclose(out["o"][0, bb, v, hv], S @ q, rtol=1e-10, atol=1e-12)


def test_tree_vg_path_replay_gives_each_node_state():
    """tape_rollback_vg along a node's root path, from the tree's own tape,
    rebuilds that node's state (what rollback to an accepted tree path does)."""
    T = 12
    parent, x, cs, w, a, b, S0 = _tree_inputs(SH, T, 9)
    out = oracle.tree_verify_vg(SH, parent, x, cs, w, a, b, S0, want_node_states=True)
    for v in (0, 5, T - 1):
        path = np.full((SH.B, T), -1, np.int32)
        nk = np.zeros(SH.B, np.int32)
        for bb in range(SH.B):
            p, c = [], v
            while c >= 0:
                p.append(c)
                c = parent[bb, c]
            p = p[::-1]
            path[bb, :len(p)] = p
            nk[bb] = len(p)
        S = oracle.tape_rollback_vg(SH, S0, out["u"], out["k"], out["g"], nk, path)
        np.testing.assert_allclose(S, out["S_nodes"][:, :, v], rtol=1e-12, atol=1e-14)
