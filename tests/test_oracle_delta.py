"""Pins of the oracle's conv, normalisation and gated delta-rule verify.

Each check compares the oracle with something other than itself: numpy's
convolution, an algebraically different matrix form of the delta rule, the
chunked WY closed form derived independently, or special cases with a known
answer.  Run on CPU only.
"""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_verify_gdn_amd import workload as W

pytestmark = pytest.mark.filterwarnings("ignore")


def tiny_cfg(**kw):
    base = dict(cfg_id=0, name="tiny", L=2, B=2, Hk=2, Hv=4, Dk=8, Dv=6, K=4, T=7,
                dtype=torch.float32, law="uniform", seed=0x5EED0101)
    base.update(kw)
    return W.Config(**base)


def shape_of(cfg, **kw):
    d = dict(L=cfg.L, B=cfg.B, Hk=cfg.Hk, Hv=cfg.Hv, Dk=cfg.Dk, Dv=cfg.Dv, K=cfg.K,
             silu=cfg.silu, eps=cfg.eps)
    d.update(kw)
    return oracle.Shape(**d)


def inputs_f64(cfg, rnd=0, T=None):
    t = W.layer_inputs(cfg, rnd, "cpu", T=T)
    return {k: W.to_f64(v) for k, v in t.items()}


# ---------------------------------------------------------------- conv -------

@pytest.mark.parametrize("K", [2, 3, 4, 6])
@pytest.mark.parametrize("silu", [False, True])
def test_conv_chain_matches_numpy_convolve(oracle_mod, K, silu):
    rng = np.random.default_rng(K * 10 + silu)
    T, C = 9, 5
    state = rng.standard_normal((K - 1, C))
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, K))
    y = oracle.conv_chain(state, x, w, silu=silu)
    xt = np.concatenate([state, x], axis=0)
    for c in range(C):
        ref = np.convolve(xt[:, c], w[c, ::-1], mode="valid")
        if silu:
            ref = ref / (1.0 + np.exp(-ref))
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-13, atol=1e-13)


def test_conv_impulse_is_identity(oracle_mod):
    rng = np.random.default_rng(1)
    K, T, C = 4, 6, 7
    w = np.zeros((C, K))
    w[:, K - 1] = 1.0
    x = rng.standard_normal((T, C))
    y = oracle.conv_chain(rng.standard_normal((K - 1, C)), x, w, silu=False)
    np.testing.assert_array_equal(y, x)
    # tap 0 reaches back K-1 rows: the first output is the oldest state row
    w2 = np.zeros((C, K))
    w2[:, 0] = 1.0
    st = rng.standard_normal((K - 1, C))
    y2 = oracle.conv_chain(st, x, w2, silu=False)
    np.testing.assert_array_equal(y2[0], st[0])
    np.testing.assert_array_equal(y2[K - 1], x[0])


def test_conv_tree_equals_chain_along_each_path(oracle_mod):
    rng = np.random.default_rng(7)
    K, T, C = 4, 20, 5
    parent = W.random_tree(rng, T, branching=3, max_depth=6)
    state = rng.standard_normal((K - 1, C))
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, K))
    y, win = oracle.conv_tree(parent, state, x, w, silu=True)
    for v in range(T):
        chain = []
        cur = v
        while cur >= 0:
            chain.append(cur)
            cur = parent[cur]
        chain.reverse()
        yc = oracle.conv_chain(state, x[chain], w, silu=True)
        np.testing.assert_array_equal(y[v], yc[-1])
        # window indices: last K entries of [old rows -(K-1)..-1, chain...]
        ext = list(range(-(K - 1), 0)) + chain
        assert list(win[v]) == ext[-K:]


def test_conv_tree_chain_parents_window_closed_form(oracle_mod):
    K, T, C = 4, 9, 3
    parent = np.arange(T) - 1
    rng = np.random.default_rng(3)
    _, win = oracle.conv_tree(parent, rng.standard_normal((K - 1, C)),
                              rng.standard_normal((T, C)), rng.standard_normal((C, K)))
    for v in range(T):
        assert list(win[v]) == [v - (K - 1) + j for j in range(K)]


# -------------------------------------------------- brute-force matrix form --

def numpy_verify(cfg, inp, parent=None):
    """Independent numpy verify: np.convolve conv, explicit norm, and the
    matrix form S_t = a S_{t-1} (I - b k k^T) + b v k^T of the delta rule."""
    L, B, T = inp["x"].shape[:3]
    Hk, Hv, Dk, Dv, K = cfg.Hk, cfg.Hv, cfg.Dk, cfg.Dv, cfg.K
    C = cfg.C
    o = np.zeros((L, B, T, Hv, Dv))
    u = np.zeros((L, B, T, Hv, Dv))
    kk = np.zeros((L, B, T, Hk, Dk))
    Sf = np.zeros((L, B, Hv, Dv, Dk))
    Snodes = np.zeros((L, B, T, Hv, Dv, Dk))
    for l in range(L):
        for b in range(B):
            par = np.arange(T) - 1 if parent is None else parent[b]
            y = np.zeros((T, C))
            for v in range(T):
                chain = []
                cur = v
                while cur >= 0:
                    chain.append(cur)
                    cur = par[cur]
                chain.reverse()
                xt = np.concatenate([inp["conv_state"][l, b], inp["x"][l, b][chain]], axis=0)
                for c in range(C):
                    r = np.convolve(xt[-K:, c], inp["conv_w"][l, c, ::-1], mode="valid")[0]
                    y[v, c] = r / (1.0 + np.exp(-r)) if cfg.silu else r
            q = y[:, :Hk * Dk].reshape(T, Hk, Dk)
            k = y[:, Hk * Dk:2 * Hk * Dk].reshape(T, Hk, Dk)
            vv = y[:, 2 * Hk * Dk:].reshape(T, Hv, Dv)
            q = q / np.sqrt((q * q).sum(-1, keepdims=True) + cfg.eps)
            k = k / np.sqrt((k * k).sum(-1, keepdims=True) + cfg.eps)
            kk[l, b] = k
            for h in range(Hv):
                hk = h * Hk // Hv
                for v in range(T):
                    p = par[v]
                    Sp = inp["S0"][l, b, h] if p < 0 else Snodes[l, b, p, h]
                    a = inp["a"][l, b, v, h]
                    bb = inp["b"][l, b, v, h]
                    kv = k[v, hk][:, None]
                    S = a * Sp @ (np.eye(Dk) - bb * kv @ kv.T) + bb * vv[v, h][:, None] @ kv.T
                    Snodes[l, b, v, h] = S
                    o[l, b, v, h] = S @ q[v, hk]
                    u[l, b, v, h] = bb * (vv[v, h] - a * Sp @ k[v, hk])
                Sf[l, b, h] = Snodes[l, b, T - 1, h]
    return dict(o=o, u=u, k=kk, S_final=Sf, S_nodes=Snodes)


@pytest.mark.parametrize("silu", [True, False])
def test_verify_matches_bruteforce_matrix_form(oracle_mod, silu):
    cfg = tiny_cfg(silu=silu)
    inp = inputs_f64(cfg)
    ref = numpy_verify(cfg, inp)
    out = oracle.verify_chunk(shape_of(cfg), **inp)
    for key in ("o", "u", "k", "S_final"):
        np.testing.assert_allclose(out[key], ref[key], rtol=1e-11, atol=1e-12, err_msg=key)
    np.testing.assert_array_equal(out["g"], inp["a"])


def test_verify_bf16_inputs_bruteforce(oracle_mod):
    cfg = tiny_cfg(dtype=torch.bfloat16, Hk=1, Hv=3, Dk=16, Dv=8, T=5)
    inp = inputs_f64(cfg, rnd=4)
    ref = numpy_verify(cfg, inp)
    out = oracle.verify_chunk(shape_of(cfg), **inp)
    for key in ("o", "u", "S_final"):
        np.testing.assert_allclose(out[key], ref[key], rtol=1e-11, atol=1e-12, err_msg=key)


def test_qk_unit_norm_and_v_passthrough(oracle_mod):
    cfg = tiny_cfg()
    inp = inputs_f64(cfg)
    out = oracle.verify_chunk(shape_of(cfg), **inp, want_qkv_post=True)
    nk = np.linalg.norm(out["k"], axis=-1)
    post = out["qkv_post"][..., cfg.Hk * cfg.Dk:2 * cfg.Hk * cfg.Dk].reshape(nk.shape + (cfg.Dk,))
    ss = (post ** 2).sum(-1)
    np.testing.assert_allclose(nk, np.sqrt(ss / (ss + cfg.eps)), rtol=1e-13)


# ---------------------------------------------------------- special cases ---

def test_b_zero_is_pure_decay(oracle_mod):
    cfg = tiny_cfg()
    inp = inputs_f64(cfg)
    inp["b"] = np.zeros_like(inp["b"])
    out = oracle.verify_chunk(shape_of(cfg), **inp, want_qkv_post=True)
    gamma = np.cumprod(inp["a"], axis=2)  # [L,B,T,Hv]
    np.testing.assert_allclose(out["S_final"], gamma[:, :, -1, :, None, None] * inp["S0"],
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(out["u"], 0.0)
    # o_t = gamma_t S0 q_t with q from the (separately pinned) conv output
    q = out["qkv_post"][..., :cfg.Hk * cfg.Dk].reshape(cfg.L, cfg.B, cfg.T, cfg.Hk, cfg.Dk)
    q = q / np.sqrt((q * q).sum(-1, keepdims=True) + cfg.eps)
    hk = np.arange(cfg.Hv) * cfg.Hk // cfg.Hv
    ref = gamma[..., None] * np.einsum("lbhij,lbthj->lbthi", inp["S0"], q[:, :, :, hk])
    np.testing.assert_allclose(out["o"], ref, rtol=1e-12, atol=1e-14)


def test_b_one_unit_keys_write_v(oracle_mod):
    """b=1 and |k|=1 (eps=0): the delta rule stores v exactly, S_t k_t = v_t."""
    cfg = tiny_cfg(eps=0.0, T=4)
    inp = inputs_f64(cfg)
    inp["b"] = np.ones_like(inp["b"])
    sh = shape_of(cfg)
    par = np.tile(np.arange(cfg.T) - 1, (cfg.B, 1))
    out = oracle.tree_verify(sh, par, **inp, want_node_states=True)
    full = oracle.verify_chunk(sh, **inp, want_qkv_post=True)
    v = full["qkv_post"][..., 2 * cfg.Hk * cfg.Dk:].reshape(cfg.L, cfg.B, cfg.T, cfg.Hv, cfg.Dv)
    hk = np.arange(cfg.Hv) * cfg.Hk // cfg.Hv
    Sk = np.einsum("lbthij,lbthj->lbthi", out["S_nodes"], full["k"][:, :, :, hk])
    np.testing.assert_allclose(Sk, v, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_accumulate_outer_products(oracle_mod):
    """a=b=1, S0=0, identity conv, orthonormal keys: S_T = sum_t v_t k_t^T."""
    cfg = tiny_cfg(L=1, B=1, Hk=1, Hv=2, Dk=8, Dv=5, T=6, silu=False, eps=0.0)
    sh = shape_of(cfg)
    rng = np.random.default_rng(11)
    T, C, K = cfg.T, cfg.C, cfg.K
    x = rng.standard_normal((1, 1, T, C))
    Q, _ = np.linalg.qr(rng.standard_normal((cfg.Dk, cfg.Dk)))
    x[0, 0, :, cfg.Dk:2 * cfg.Dk] = Q[:T] * 3.0  # orthogonal rows, any scale
    w = np.zeros((1, C, K))
    w[..., K - 1] = 1.0
    inp = dict(x=x, conv_state=np.zeros((1, 1, K - 1, C)), conv_w=w,
               a=np.ones((1, 1, T, cfg.Hv)), b=np.ones((1, 1, T, cfg.Hv)),
               S0=np.zeros((1, 1, cfg.Hv, cfg.Dv, cfg.Dk)))
    out = oracle.verify_chunk(sh, **inp)
    kk = Q[:T]
    for h in range(cfg.Hv):
        vv = x[0, 0, :, 2 * cfg.Dk + h * cfg.Dv:2 * cfg.Dk + (h + 1) * cfg.Dv]
        np.testing.assert_allclose(out["S_final"][0, 0, h], vv.T @ kk, atol=1e-13)
        np.testing.assert_allclose(out["u"][0, 0, :, h], vv, atol=1e-13)


def test_rows_are_independent(oracle_mod):
    cfg = tiny_cfg()
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    base = oracle.verify_chunk(sh, **inp)
    inp2 = dict(inp)
    inp2["S0"] = inp["S0"].copy()
    inp2["S0"][:, :, :, 2, :] += 0.5
    pert = oracle.verify_chunk(sh, **inp2)
    rows = [i for i in range(cfg.Dv) if i != 2]
    np.testing.assert_array_equal(pert["S_final"][:, :, :, rows], base["S_final"][:, :, :, rows])
    np.testing.assert_array_equal(pert["o"][..., rows], base["o"][..., rows])
    assert not np.allclose(pert["o"][..., 2], base["o"][..., 2])


def test_contraction_bound(oracle_mod):
    """|S_t|_F <= a_t |S_{t-1}|_F + b_t |v_t| for b in [0,1], |k| <= 1."""
    cfg = tiny_cfg(T=8)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    par = np.tile(np.arange(cfg.T) - 1, (cfg.B, 1))
    out = oracle.tree_verify(sh, par, **inp, want_node_states=True)
    full = oracle.verify_chunk(sh, **inp, want_qkv_post=True)
    v = full["qkv_post"][..., 2 * cfg.Hk * cfg.Dk:].reshape(cfg.L, cfg.B, cfg.T, cfg.Hv, cfg.Dv)
    Sn = out["S_nodes"]
    prev = np.linalg.norm(inp["S0"], axis=(-2, -1))
    for t in range(cfg.T):
        cur = np.linalg.norm(Sn[:, :, t], axis=(-2, -1))
        bound = inp["a"][:, :, t] * prev + inp["b"][:, :, t] * np.linalg.norm(v[:, :, t], axis=-1)
        assert np.all(cur <= bound * (1 + 1e-12))
        prev = cur


# ------------------------------------------------------------ WY closed form -

def wy_numpy(S0, q, k, v, a, b, parent):
    """Chunked (WY / UT-transform) form of the delta rule over a chain or tree,
    derived by unrolling the recurrence along ancestor paths:
        gamma_t = prod of a over the inclusive ancestor path of t
        A[t,i]  = b_t (gamma_t/gamma_i) k_t.k_i   for proper ancestors i
        U = (I + A)^-1 diag(b) (V - diag(gamma) K S0^T)
        O = diag(gamma) Q S0^T + (M o Gamma o Q K^T) U   (M: inclusive ancestors)
    """
    T = len(parent)
    anc = np.zeros((T, T), dtype=bool)
    lg = np.zeros(T)
    for t in range(T):
        p = parent[t]
        if p >= 0:
            anc[t] = anc[p]
            anc[t, p] = True
        lg[t] = (lg[p] if p >= 0 else 0.0) + np.log(a[t])
    Gam = np.exp(lg[:, None] - lg[None, :])
    gam = np.exp(lg)
    A = np.where(anc, b[:, None] * Gam * (k @ k.T), 0.0)
    rhs = b[:, None] * (v - gam[:, None] * (k @ S0.T))
    U = np.linalg.solve(np.eye(T) + A, rhs)
    M = anc | np.eye(T, dtype=bool)
    O = gam[:, None] * (q @ S0.T) + np.where(M, Gam * (q @ k.T), 0.0) @ U
    return U, O


@pytest.mark.parametrize("tree", [False, True])
def test_wy_form_matches_oracle(oracle_mod, tree):
    cfg = tiny_cfg(T=12, Hk=1, Hv=2, Dk=16, Dv=8, L=1, B=2)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    if tree:
        rng = np.random.default_rng(5)
        par = np.stack([W.random_tree(rng, cfg.T, 3, 5) for _ in range(cfg.B)])
        out = oracle.tree_verify(sh, par, **inp)
    else:
        par = np.tile(np.arange(cfg.T) - 1, (cfg.B, 1))
        out = oracle.verify_chunk(sh, **inp)
    post = numpy_verify(cfg, inp, parent=None if not tree else par)  # for q,k,v via conv
    for b in range(cfg.B):
        # q, v from an independent numpy conv on each node's path
        C = cfg.C
        y = np.zeros((cfg.T, C))
        for v_ in range(cfg.T):
            chain = []
            cur = v_
            while cur >= 0:
                chain.append(cur)
                cur = par[b][cur]
            chain.reverse()
            xt = np.concatenate([inp["conv_state"][0, b], inp["x"][0, b][chain]], axis=0)
            r = (xt[-cfg.K:] * inp["conv_w"][0].T).sum(0)
            y[v_] = r / (1 + np.exp(-r))
        q = y[:, :cfg.Dk]
        q = q / np.sqrt((q * q).sum(-1, keepdims=True) + cfg.eps)
        k = post["k"][0, b, :, 0]
        for h in range(cfg.Hv):
            vv = y[:, 2 * cfg.Dk + h * cfg.Dv:2 * cfg.Dk + (h + 1) * cfg.Dv]
            U, O = wy_numpy(inp["S0"][0, b, h], q, k, vv, inp["a"][0, b, :, h],
                            inp["b"][0, b, :, h], par[b])
            np.testing.assert_allclose(out["u"][0, b, :, h], U, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(out["o"][0, b, :, h], O, rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------ tree ----

def test_tree_with_chain_parents_equals_chunk(oracle_mod):
    cfg = tiny_cfg(T=9)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    par = np.tile(np.arange(cfg.T) - 1, (cfg.B, 1))
    tr = oracle.tree_verify(sh, par, **inp)
    ch = oracle.verify_chunk(sh, **inp)
    for key in ("o", "u", "k", "g"):
        np.testing.assert_array_equal(tr[key], ch[key], err_msg=key)


def test_tree_nodes_equal_chunk_along_root_path(oracle_mod):
    cfg = tiny_cfg(T=16, L=1, B=2)
    sh = shape_of(cfg)
    inp = inputs_f64(cfg)
    rng = np.random.default_rng(17)
    par = np.stack([W.random_tree(rng, cfg.T, 4, 8) for _ in range(cfg.B)])
    tr = oracle.tree_verify(sh, par, **inp, want_node_states=True)
    for b in range(cfg.B):
        for v in range(cfg.T):
            chain = []
            cur = v
            while cur >= 0:
                chain.append(cur)
                cur = par[b][cur]
            chain.reverse()
            sub = {key: val[:, b:b + 1] for key, val in inp.items() if key != "conv_w"}
            sub["conv_w"] = inp["conv_w"]
            for key in ("x", "a", "b"):
                sub[key] = sub[key][:, :, chain]
            shb = shape_of(cfg, B=1)
            ch = oracle.verify_chunk(shb, **sub)
            np.testing.assert_allclose(tr["o"][:, b, v], ch["o"][:, 0, -1], rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(tr["u"][:, b, v], ch["u"][:, 0, -1], rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(tr["S_nodes"][:, b, v], ch["S_final"][:, 0], rtol=1e-13,
                                       atol=1e-14)
