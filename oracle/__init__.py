"""fp64 CPU oracle for GDN speculative verification with tape-replay rollback.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library (``speculative_decode_verify_gdn_amd``) and never imports it;
both sides see only the bytes the seeded workload generator produces.

The numeric work lives in ``gdn_oracle.c`` (plain C, double precision, plain
loops); this module only marshals numpy arrays through ctypes.  Every input is
up-cast to float64 exactly (bf16 and fp32 values are exact in fp64).

Parity status of each function (the pins live in ``tests/test_oracle_*.py``):
  conv_chain / conv_tree  pinned: numpy.convolve per channel, impulse weights,
                          tree == chain along each root-to-node path.
  verify_chunk            pinned: brute-force matrix form of the delta rule,
                          b=0 / b=1 / orthonormal-key special cases, row
                          independence, contraction bound, WY closed form.
  tree_verify             pinned: chain parents == verify_chunk; every node ==
                          verify_chunk along its root path.
  accept                  pinned: brute-force enumeration of prefixes / paths.
  verify_chunk_vg         pinned: equal per-channel gates give verify_chunk;
                          the matrix form S diag(a)(I - b k k^T) + b v k^T;
                          a zero gate erases its key column; replay of the
                          whole tape gives S_final.
  tree_verify_vg          pinned: equal gates give tree_verify; chain parents
                          give verify_chunk_vg; every node state and output
                          against the matrix form along its root path; path
                          replay of the tree's tape gives each node state.
  tape_rollback_vg        pinned: replay(n) == fresh recompute over n tokens,
                          equal gates give tape_rollback.
  accept_sample           pinned: the first output token's distribution equals
                          p exactly (quadrature over the uniforms), the
                          low-temperature limit equals the greedy accept,
                          hand-computed cases, uniform extremes.
  tape_rollback           pinned: replay(n) == fresh recompute over n tokens,
                          closed-form rank-n sum, n=0 identity.
  conv_rollback           pinned: numpy concatenation of the accepted rows;
                          window indices against their closed form.
  cost_model              pinned: the pages' printed limits and closed forms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC_PATH = os.path.join(_HERE, "gdn_oracle.c")

_lib = None


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into liboracle.so with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-fPIC",
             "-shared", _SRC_PATH, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _OShape(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int), ("B", ctypes.c_int), ("Hk", ctypes.c_int),
                ("Hv", ctypes.c_int), ("Dk", ctypes.c_int), ("Dv", ctypes.c_int),
                ("K", ctypes.c_int), ("silu", ctypes.c_int), ("eps", ctypes.c_double)]


@dataclass(frozen=True)
class Shape:
    """Layer-stack shape.  C = 2*Hk*Dk + Hv*Dv channels in the qkv stream."""
    L: int
    B: int
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    K: int
    silu: bool = True
    eps: float = 1e-6

    @property
    def C(self) -> int:
        return 2 * self.Hk * self.Dk + self.Hv * self.Dv

    def _c(self) -> _OShape:
        return _OShape(self.L, self.B, self.Hk, self.Hv, self.Dk, self.Dv, self.K,
                       int(self.silu), float(self.eps))


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_conv_chain.argtypes = [I, I, I, I, P, P, P, P]
        lib.oracle_conv_chain.restype = None
        lib.oracle_conv_tree.argtypes = [I, I, I, I, P, P, P, P, P, P]
        lib.oracle_conv_tree.restype = I
        SP = ctypes.POINTER(_OShape)
        lib.oracle_verify_chunk.argtypes = [SP, I] + [P] * 12
        lib.oracle_verify_chunk.restype = I
        lib.oracle_tree_verify.argtypes = [SP, I] + [P] * 13
        lib.oracle_tree_verify.restype = I
        lib.oracle_tree_verify_vg.argtypes = [SP, I] + [P] * 13
        lib.oracle_tree_verify_vg.restype = I
        lib.oracle_accept.argtypes = [I, I, I, P, P, P, P, P, P]
        lib.oracle_accept.restype = I
        lib.oracle_tape_rollback.argtypes = [SP, I, P, P, P, P, P, P]
        lib.oracle_tape_rollback.restype = I
        lib.oracle_verify_chunk_vg.argtypes = [SP, I] + [P] * 11
        lib.oracle_verify_chunk_vg.restype = I
        lib.oracle_tape_rollback_vg.argtypes = [SP, I, P, P, P, P, P, P]
        lib.oracle_tape_rollback_vg.restype = I
        lib.oracle_conv_rollback.argtypes = [SP, I, P, P, P, P, P]
        lib.oracle_conv_rollback.restype = I
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = I
        lib.oracle_set_num_threads.argtypes = [I]
        lib.oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def _f64(a, shape=None) -> np.ndarray:
    out = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and out.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), out.shape))
    return out


def _i32(a, shape=None) -> np.ndarray:
    out = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    if shape is not None and out.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), out.shape))
    return out


def _p(a):
    return None if a is None else a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s failed with code %d" % (what, rc))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Worker threads of later oracle calls (used to time it on one core)."""
    _load().oracle_set_num_threads(int(n))


def conv_chain(state, x, w, silu: bool = True) -> np.ndarray:
    """Depthwise causal conv over [state; x] (per channel), SiLU after if asked.

    state (K-1, C), x (T, C), w (C, K) -> y (T, C)."""
    w = _f64(w)
    C, K = w.shape
    x = _f64(x)
    T = x.shape[0]
    state = _f64(state, (K - 1, C))
    y = np.empty((T, C))
    _load().oracle_conv_chain(K, T, C, int(silu), _p(state), _p(x), _p(w), _p(y))
    return y


def conv_tree(parent, state, x, w, silu: bool = True):
    """Tree conv: node v uses the last K entries of [state, ancestors' x, x_v].

    Returns (y (T, C), win (T, K) int32 window indices)."""
    w = _f64(w)
    C, K = w.shape
    x = _f64(x)
    T = x.shape[0]
    state = _f64(state, (K - 1, C))
    parent = _i32(parent, (T,))
    y = np.empty((T, C))
    win = np.empty((T, K), dtype=np.int32)
    _check(_load().oracle_conv_tree(K, T, C, int(silu), _p(parent), _p(state), _p(x),
                                    _p(w), _p(y), _p(win)), "conv_tree")
    return y, win


def verify_chunk(sh: Shape, x, conv_state, conv_w, a, b, S0, want_final=True,
                 want_qkv_post=False) -> dict:
    """Sequential gated delta-rule verify of T tokens per (layer, sequence).

    Returns a dict with o, u, k, g (the tape), S_final and optionally qkv_post."""
    L, B, C = sh.L, sh.B, sh.C
    x = _f64(x)
    T = x.shape[2]
    x = _f64(x, (L, B, T, C))
    conv_state = _f64(conv_state, (L, B, sh.K - 1, C))
    conv_w = _f64(conv_w, (L, C, sh.K))
    a = _f64(a, (L, B, T, sh.Hv))
    b = _f64(b, (L, B, T, sh.Hv))
    S0 = _f64(S0, (L, B, sh.Hv, sh.Dv, sh.Dk))
    o = np.empty((L, B, T, sh.Hv, sh.Dv))
    u = np.empty((L, B, T, sh.Hv, sh.Dv))
    k = np.empty((L, B, T, sh.Hk, sh.Dk))
    g = np.empty((L, B, T, sh.Hv))
    Sf = np.empty_like(S0) if want_final else None
    qp = np.empty((L, B, T, C)) if want_qkv_post else None
    c = sh._c()
    _check(_load().oracle_verify_chunk(ctypes.byref(c), T, _p(x), _p(conv_state), _p(conv_w),
                                       _p(a), _p(b), _p(S0), _p(o), _p(u), _p(k), _p(g),
                                       _p(Sf), _p(qp)), "verify_chunk")
    out = dict(o=o, u=u, k=k, g=g)
    if want_final:
        out["S_final"] = Sf
    if want_qkv_post:
        out["qkv_post"] = qp
    return out


def verify_chunk_vg(sh: Shape, x, conv_state, conv_w, a, b, S0) -> dict:
    """verify_chunk with a per-key-channel decay gate a (L, B, T, Hv, Dk): per
    token S <- S diag(a_t), u = b (v - S k), S <- S + u k^T, o = S q.
    Returns o, u, k, g (= a, the decay tape) and S_final."""
    L, B, C = sh.L, sh.B, sh.C
    x = _f64(x)
    T = x.shape[2]
    x = _f64(x, (L, B, T, C))
    conv_state = _f64(conv_state, (L, B, sh.K - 1, C))
    conv_w = _f64(conv_w, (L, C, sh.K))
    a = _f64(a, (L, B, T, sh.Hv, sh.Dk))
    b = _f64(b, (L, B, T, sh.Hv))
    S0 = _f64(S0, (L, B, sh.Hv, sh.Dv, sh.Dk))
    o = np.empty((L, B, T, sh.Hv, sh.Dv))
    u = np.empty((L, B, T, sh.Hv, sh.Dv))
    k = np.empty((L, B, T, sh.Hk, sh.Dk))
    g = np.empty((L, B, T, sh.Hv, sh.Dk))
    Sf = np.empty_like(S0)
    c = sh._c()
    _check(_load().oracle_verify_chunk_vg(ctypes.byref(c), T, _p(x), _p(conv_state), _p(conv_w),
                                          _p(a), _p(b), _p(S0), _p(o), _p(u), _p(k), _p(g),
                                          _p(Sf)), "verify_chunk_vg")
    return dict(o=o, u=u, k=k, g=g, S_final=Sf)


def tape_rollback_vg(sh: Shape, S, u, k, g, n_keep, path=None) -> np.ndarray:
    """tape_rollback with the per-key-channel decay tape g (L, B, T, Hv, Dk)."""
    S = _f64(S, (sh.L, sh.B, sh.Hv, sh.Dv, sh.Dk)).copy()
    u = _f64(u)
    T = u.shape[2]
    u = _f64(u, (sh.L, sh.B, T, sh.Hv, sh.Dv))
    k = _f64(k, (sh.L, sh.B, T, sh.Hk, sh.Dk))
    g = _f64(g, (sh.L, sh.B, T, sh.Hv, sh.Dk))
    n_keep = _i32(n_keep, (sh.B,))
    path = None if path is None else _i32(path, (sh.B, T))
    c = sh._c()
    _check(_load().oracle_tape_rollback_vg(ctypes.byref(c), T, _p(S), _p(u), _p(k), _p(g),
                                           _p(path), _p(n_keep)), "tape_rollback_vg")
    return S


def tree_verify(sh: Shape, parent, x, conv_state, conv_w, a, b, S0,
                want_node_states=False) -> dict:
    """Gated delta-rule verify over a draft tree (each node from its parent).

    Returns o, u, k, g, conv_win (B, T, K) and optionally S_nodes."""
    L, B, C = sh.L, sh.B, sh.C
    x = _f64(x)
    T = x.shape[2]
    x = _f64(x, (L, B, T, C))
    parent = _i32(parent, (B, T))
    conv_state = _f64(conv_state, (L, B, sh.K - 1, C))
    conv_w = _f64(conv_w, (L, C, sh.K))
    a = _f64(a, (L, B, T, sh.Hv))
    b = _f64(b, (L, B, T, sh.Hv))
    S0 = _f64(S0, (L, B, sh.Hv, sh.Dv, sh.Dk))
    o = np.empty((L, B, T, sh.Hv, sh.Dv))
    u = np.empty((L, B, T, sh.Hv, sh.Dv))
    k = np.empty((L, B, T, sh.Hk, sh.Dk))
    g = np.empty((L, B, T, sh.Hv))
    win = np.empty((B, T, sh.K), dtype=np.int32)
    Sn = np.empty((L, B, T, sh.Hv, sh.Dv, sh.Dk)) if want_node_states else None
    c = sh._c()
    _check(_load().oracle_tree_verify(ctypes.byref(c), T, _p(parent), _p(x), _p(conv_state),
                                      _p(conv_w), _p(a), _p(b), _p(S0), _p(o), _p(u), _p(k),
                                      _p(g), _p(win), _p(Sn)), "tree_verify")
    out = dict(o=o, u=u, k=k, g=g, conv_win=win)
    if want_node_states:
        out["S_nodes"] = Sn
    return out


def tree_verify_vg(sh: Shape, parent, x, conv_state, conv_w, a, b, S0,
                   want_node_states=False) -> dict:
    """tree_verify with a per-key-channel decay gate a (L, B, T, Hv, Dk):
    node v steps from its parent's state as S <- S diag(a_v), u = b (v - S k),
    S <- S + u k^T, o = S q.  Returns o, u, k, g (= a), conv_win and
    optionally S_nodes."""
    L, B, C = sh.L, sh.B, sh.C
    x = _f64(x)
    T = x.shape[2]
    x = _f64(x, (L, B, T, C))
    parent = _i32(parent, (B, T))
    conv_state = _f64(conv_state, (L, B, sh.K - 1, C))
    conv_w = _f64(conv_w, (L, C, sh.K))
    a = _f64(a, (L, B, T, sh.Hv, sh.Dk))
    b = _f64(b, (L, B, T, sh.Hv))
    S0 = _f64(S0, (L, B, sh.Hv, sh.Dv, sh.Dk))
    o = np.empty((L, B, T, sh.Hv, sh.Dv))
    u = np.empty((L, B, T, sh.Hv, sh.Dv))
    k = np.empty((L, B, T, sh.Hk, sh.Dk))
    g = np.empty((L, B, T, sh.Hv, sh.Dk))
    win = np.empty((B, T, sh.K), dtype=np.int32)
    Sn = np.empty((L, B, T, sh.Hv, sh.Dv, sh.Dk)) if want_node_states else None
    c = sh._c()
    _check(_load().oracle_tree_verify_vg(ctypes.byref(c), T, _p(parent), _p(x), _p(conv_state),
                                         _p(conv_w), _p(a), _p(b), _p(S0), _p(o), _p(u), _p(k),
                                         _p(g), _p(win), _p(Sn)), "tree_verify_vg")
    out = dict(o=o, u=u, k=k, g=g, conv_win=win)
    if want_node_states:
        out["S_nodes"] = Sn
    return out


def accept(draft, logits, parent=None):
    """Greedy acceptance.  draft (B, T), logits (B, T+1, V), parent (B, T) or None.

    Returns (n_keep (B,), path (B, T) -1 padded, bonus (B,))."""
    draft = _i32(draft)
    B, T = draft.shape
    logits = _f64(logits)
    V = logits.shape[2]
    logits = _f64(logits, (B, T + 1, V))
    par = None if parent is None else _i32(parent, (B, T))
    n = np.empty(B, dtype=np.int32)
    path = np.empty((B, T), dtype=np.int32)
    bonus = np.empty(B, dtype=np.int32)
    _check(_load().oracle_accept(B, T, V, _p(par), _p(draft), _p(logits), _p(n), _p(path),
                                 _p(bonus)), "accept")
    return n, path, bonus


def tape_rollback(sh: Shape, S, u, k, g, n_keep, path=None) -> np.ndarray:
    """Replay the accepted tape entries onto the snapshot S; returns the new state."""
    S = _f64(S, (sh.L, sh.B, sh.Hv, sh.Dv, sh.Dk)).copy()
    u = _f64(u)
    T = u.shape[2]
    u = _f64(u, (sh.L, sh.B, T, sh.Hv, sh.Dv))
    k = _f64(k, (sh.L, sh.B, T, sh.Hk, sh.Dk))
    g = _f64(g, (sh.L, sh.B, T, sh.Hv))
    n_keep = _i32(n_keep, (sh.B,))
    path = None if path is None else _i32(path, (sh.B, T))
    c = sh._c()
    _check(_load().oracle_tape_rollback(ctypes.byref(c), T, _p(S), _p(u), _p(k), _p(g),
                                        _p(path), _p(n_keep)), "tape_rollback")
    return S


def conv_rollback(sh: Shape, conv_state, x, n_keep, path=None):
    """Rebuild the conv window from the accepted raw rows.

    Returns (new conv_state (L, B, K-1, C), win_idx (B, K-1))."""
    cs = _f64(conv_state, (sh.L, sh.B, sh.K - 1, sh.C)).copy()
    x = _f64(x)
    T = x.shape[2]
    x = _f64(x, (sh.L, sh.B, T, sh.C))
    n_keep = _i32(n_keep, (sh.B,))
    path = None if path is None else _i32(path, (sh.B, T))
    win = np.empty((sh.B, sh.K - 1), dtype=np.int32)
    c = sh._c()
    _check(_load().oracle_conv_rollback(ctypes.byref(c), T, _p(cs), _p(x), _p(path),
                                        _p(n_keep), _p(win)), "conv_rollback")
    return cs, win


def _softmax64(z: np.ndarray) -> np.ndarray:
    e = np.exp(z - z.max())
    return e / e.sum()


def sample_cdf(logits_row, temperature: float, ban: int = -1) -> np.ndarray:
    """Cumulative mass, in index order, of softmax(logits_row / temperature)
    with token `ban` (if >= 0) set to zero; not renormalised."""
    q = _softmax64(_f64(logits_row) / float(temperature))
    if ban >= 0:
        q[ban] = 0.0
    return np.cumsum(q)


def accept_sample(draft, logits, temperature: float, uniforms, detail: bool = False):
    """Rejection-sampling acceptance of a deterministic draft chain.

    colibri "MTP speculative decoding and prefetch" s5: the draft is a point
    mass, so draft token d at position j is kept with probability p_j(d),
    where p_j = softmax(logits[j] / temperature); at the first rejection the
    output token is drawn from p_j with d removed and the rest renormalised
    (which keeps the output distribution exactly p); if every draft is kept,
    the output token is drawn from p_T.

    draft (B, T) int, logits (B, T+1, V), temperature > 0, uniforms (B, T+1)
    in [0, 1): uniforms[b, j] decides draft j (kept iff u < p_j(d)),
    uniforms[b, T] draws the output token as the smallest index i whose
    cumulative mass (index order, removed token counting zero) exceeds u
    times the total remaining mass.  A draft token outside [0, V) is never
    kept and removes nothing.  All arithmetic in float64.

    Returns (n_keep (B,), path (B, T) -1 padded, token (B,)); with
    detail=True also p_draft (B, T), the probability of each draft token
    (NaN past the first rejection)."""
    draft = _i32(draft)
    B, T = draft.shape
    logits = _f64(logits)
    V = logits.shape[2]
    u = _f64(uniforms, (B, T + 1))
    tau = float(temperature)
    if not tau > 0.0:
        raise ValueError("temperature must be > 0")
    n_keep = np.zeros(B, dtype=np.int32)
    path = np.full((B, T), -1, dtype=np.int32)
    token = np.zeros(B, dtype=np.int32)
    p_draft = np.full((B, T), np.nan)
    for b in range(B):
        n = T
        for j in range(T):
            d = int(draft[b, j])
            pd = _softmax64(logits[b, j] / tau)[d] if 0 <= d < V else 0.0
            p_draft[b, j] = pd
            if not u[b, j] < pd:
                n = j
                break
        ban = int(draft[b, n]) if n < T and 0 <= draft[b, n] < V else -1
        c = sample_cdf(logits[b, n], tau, ban)
        i = int(np.searchsorted(c, u[b, T] * c[-1], side="right"))
        if i >= V:  # no index passes the threshold: the last one with mass
            q = np.diff(np.concatenate([[0.0], c]))
            i = int(np.flatnonzero(q > 0)[-1])
        n_keep[b] = n
        path[b, :n] = np.arange(n)
        token[b] = i
    if detail:
        return n_keep, path, token, p_draft
    return n_keep, path, token
