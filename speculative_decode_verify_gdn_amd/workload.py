"""Seeded synthetic workloads for GDN speculative verification.

This module only draws inputs.  It holds none of the method's arithmetic (no
conv, no normalisation, no recurrence, no acceptance rule) and imports neither
the HIP binding nor the oracle, so both can be fed the same bytes from it.

Shapes follow the pages' target model family: a Qwen3.6-style hybrid whose GDN
layers have 16 q/k heads and 32 v heads of 128 dims (qkv stream of 8192
channels), a conv kernel of 4, and 30 GDN layers in the 40-layer stack
("Speculative Decoding on GDN Hybrid Architectures", s2.1).  The vocabulary is
151,936 entries, the only target-model vocabulary the pages print (xserv
"Phase 25", EAGLE3-Qwen3-8B weight table).  No public dataset is involved:
every tensor is drawn here from a seed.

Value recipe (per tensor, independent draws):
  raw qkv rows x and the old conv window   N(0, 1), rounded to the input dtype
  conv weights w                           N(0, 1) / sqrt(K), fp32
  decay gate a                             exp(-U(0.01, 0.5)), rounded to the input dtype
  write gate b                             sigmoid(N(0, 1)), rounded to the input dtype
  state S0                                 N(0, 0.1**2) (std 0.1), fp32; zeros for the
                                           tiny prefill config, whose conv window also starts at 0
  logits                                   N(0, 1) per row with one planted target token
                                           at (row max + 1), rounded to bf16, so the
                                           target is the unique argmax
  drafts (chain)                           draft[j] = target of row j where position j is
                                           accepted, else a different uniformly drawn token
  trees                                    node v picks its parent uniformly among the
                                           virtual root and the earlier nodes that have
                                           fewer than `branching` children and depth below
                                           `max_depth`; sibling tokens are distinct; one leaf
                                           chosen uniformly is the planted accepted path

Bulk tensors come from ``torch.Generator`` on the requested device, seeded by
a SplitMix64 mix of (base seed, round, tensor id); the host-side structure
(trees, acceptance lengths) comes from ``numpy.random.Generator(PCG64)`` with
the same mixed seeds.  A workload drawn on the GPU is read back to the host
for the oracle, so both always see identical bytes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

VOCAB = 151_936

_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """One SplitMix64 output step (Steele, Lea, Flood 2014)."""
    x = (x + 0x9E3779B97F4A7C15) & _M64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def mix_seed(*keys: int) -> int:
    """Fold integer keys into one 63-bit seed."""
    h = 0x5EED_0000_0000_0000
    for k in keys:
        h = splitmix64(h ^ (int(k) & _M64))
    return h & ((1 << 63) - 1)


# Tensor ids for seed derivation.
_TID = dict(x=1, conv_state=2, conv_w=3, a=4, b=5, S0=6, logits=7, targets=8,
            match=9, other=10, tree=11, tokens=12, n_uniform=13)


@dataclass(frozen=True)
class Config:
    """One workload: shape, chunk length, acceptance law and seed."""
    cfg_id: int
    name: str
    L: int
    B: int
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    K: int
    T: int
    dtype: torch.dtype
    law: str                 # "uniform" | "bernoulli" | "tree"
    p_accept: float = 0.0    # per-position acceptance for "bernoulli"
    seed: int = 0
    zero_init: bool = False  # S0 = 0 and conv window = 0 (prefill from scratch)
    prefill: int = 0         # tokens verified and fully committed before round 0
    branching: int = 4
    max_depth: int = 8
    V: int = VOCAB
    silu: bool = True
    eps: float = 1e-6

    @property
    def C(self) -> int:
        return 2 * self.Hk * self.Dk + self.Hv * self.Dv

    @property
    def is_tree(self) -> bool:
        return self.law == "tree"

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    1: Config(1, "tiny_d32_prefill64_n4", L=1, B=1, Hk=1, Hv=1, Dk=32, Dv=32, K=4, T=4,
              dtype=torch.float32, law="uniform", seed=0x5EED0001, zero_init=True, prefill=64),
    2: Config(2, "one_layer_b1_n4", L=1, B=1, Hk=16, Hv=32, Dk=128, Dv=128, K=4, T=4,
              dtype=torch.bfloat16, law="uniform", seed=0x5EED0002),
    3: Config(3, "stack30_b32_n8_p036", L=30, B=32, Hk=16, Hv=32, Dk=128, Dv=128, K=4, T=8,
              dtype=torch.bfloat16, law="bernoulli", p_accept=0.36, seed=0x5EED0003),
    4: Config(4, "stack30_b256_n16_p085", L=30, B=256, Hk=16, Hv=32, Dk=128, Dv=128, K=4, T=16,
              dtype=torch.bfloat16, law="bernoulli", p_accept=0.85, seed=0x5EED0004),
    5: Config(5, "stack30_b64_tree64", L=30, B=64, Hk=16, Hv=32, Dk=128, Dv=128, K=4, T=64,
              dtype=torch.bfloat16, law="tree", seed=0x5EED0005),
}


def _tgen(device, *keys) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(mix_seed(*keys))
    return g


def _npgen(*keys) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(mix_seed(*keys)))


def layer_inputs(cfg: Config, rnd: int, device="cpu", T: Optional[int] = None,
                 layers: Optional[range] = None) -> dict:
    """Draw x, conv_state, conv_w, a, b, S0 for one round.

    Returns torch tensors on `device`:
      x [L,B,T,C] dtype, conv_state [L,B,K-1,C] dtype, conv_w [L,C,K] fp32,
      a, b [L,B,T,Hv] dtype, S0 [L,B,Hv,Dv,Dk] fp32.
    conv_w and the initial S0 / conv_state do not depend on the round."""
    T = cfg.T if T is None else T
    L, B, C, K, Hv = cfg.L, cfg.B, cfg.C, cfg.K, cfg.Hv
    dt = cfg.dtype
    s = cfg.seed

    def normal(shape, tid, r):
        return torch.randn(shape, generator=_tgen(device, s, r, _TID[tid]), device=device,
                           dtype=torch.float32)

    def uniform(shape, tid, r):
        return torch.rand(shape, generator=_tgen(device, s, r, _TID[tid]), device=device,
                          dtype=torch.float32)

    x = normal((L, B, T, C), "x", rnd).to(dt)
    if cfg.zero_init:
        conv_state = torch.zeros((L, B, K - 1, C), device=device, dtype=dt)
        S0 = torch.zeros((L, B, Hv, cfg.Dv, cfg.Dk), device=device, dtype=torch.float32)
    else:
        conv_state = normal((L, B, K - 1, C), "conv_state", -1).to(dt)
        S0 = normal((L, B, Hv, cfg.Dv, cfg.Dk), "S0", -1) * 0.1
    conv_w = normal((L, C, K), "conv_w", -1) / math.sqrt(K)
    a = torch.exp(-(0.01 + 0.49 * uniform((L, B, T, Hv), "a", rnd))).to(dt)
    b = torch.sigmoid(normal((L, B, T, Hv), "b", rnd)).to(dt)
    return dict(x=x, conv_state=conv_state, conv_w=conv_w.contiguous(), a=a, b=b,
                S0=S0.contiguous())


def _planted_logits(B: int, rows: int, V: int, targets: torch.Tensor, seed_keys, device):
    """N(0,1) logits [B, rows, V] with targets[b, r] planted at row max + 1 (bf16)."""
    lg = torch.randn((B, rows, V), generator=_tgen(device, *seed_keys), device=device,
                     dtype=torch.float32)
    mx = lg.max(dim=-1, keepdim=True).values
    lg.scatter_(-1, targets.to(device=device, dtype=torch.int64).unsqueeze(-1), mx + 1.0)
    return lg.to(torch.bfloat16)


def chain_accept_inputs(cfg: Config, rnd: int, device="cpu", B: Optional[int] = None,
                        T: Optional[int] = None, V: Optional[int] = None,
                        forced_n: Optional[int] = None) -> dict:
    """Drafts and logits realising the config's acceptance law on a chain.

    Returns draft [B,T] int32, logits [B,T+1,V] bf16, n_planted [B] int32 and
    targets [B,T+1] int32 (the planted argmax of every row).  `forced_n` plants
    the same accepted length in every sequence (used for rollback sweeps)."""
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    V = cfg.V if V is None else V
    s = cfg.seed
    rng = _npgen(s, rnd, _TID["targets"])
    targets = rng.integers(0, V, size=(B, T + 1), dtype=np.int64)
    if forced_n is not None:
        n = np.full(B, int(forced_n), dtype=np.int64)
        match = np.arange(T)[None, :] < n[:, None]
    elif cfg.law == "bernoulli":
        match = _npgen(s, rnd, _TID["match"]).random((B, T)) < cfg.p_accept
        n = np.where(match.all(axis=1), T, np.argmin(match, axis=1))
    else:  # uniform over 0..T inclusive
        n = _npgen(s, rnd, _TID["n_uniform"]).integers(0, T + 1, size=B)
        match = np.arange(T)[None, :] < n[:, None]
    other = (targets[:, :T] + 1 + _npgen(s, rnd, _TID["other"]).integers(0, V - 1, size=(B, T))) % V
    draft = np.where(match, targets[:, :T], other)
    logits = _planted_logits(B, T + 1, V, torch.from_numpy(targets), (s, rnd, _TID["logits"]),
                             device)
    return dict(draft=torch.from_numpy(draft.astype(np.int32)).to(device), logits=logits,
                n_planted=n.astype(np.int32), targets=targets.astype(np.int32))


def random_tree(rng: np.random.Generator, T: int, branching: int, max_depth: int) -> np.ndarray:
    """Parent array of a T-node draft tree in topological order (parent < child,
    -1 = virtual root); node v attaches to a uniformly chosen open slot holder."""
    parent = np.empty(T, dtype=np.int32)
    n_child = {-1: 0}
    depth = {-1: 0}
    for v in range(T):
        cands = [u for u in range(-1, v) if n_child[u] < branching and depth[u] < max_depth]
        p = cands[int(rng.integers(0, len(cands)))]
        parent[v] = p
        n_child[p] += 1
        n_child[v] = 0
        depth[v] = depth[p] + 1
    return parent


def tree_accept_inputs(cfg: Config, rnd: int, device="cpu", B: Optional[int] = None,
                       T: Optional[int] = None, V: Optional[int] = None) -> dict:
    """Draft trees, node tokens and logits with one planted root-to-leaf path.

    Returns parent [B,T] int32, draft [B,T] int32, logits [B,T+1,V] bf16,
    planted_path [B,T] int32 (-1 padded) and n_planted [B] int32."""
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    V = cfg.V if V is None else V
    s = cfg.seed
    rng = _npgen(s, rnd, _TID["tree"])
    parents = np.stack([random_tree(rng, T, cfg.branching, cfg.max_depth) for _ in range(B)])
    trng = _npgen(s, rnd, _TID["tokens"])
    tokens = np.empty((B, T), dtype=np.int64)
    targets = trng.integers(0, V, size=(B, T + 1), dtype=np.int64)
    paths = np.full((B, T), -1, dtype=np.int32)
    n = np.zeros(B, dtype=np.int32)
    for bb in range(B):
        par = parents[bb]
        sib = {}
        for v in range(T):
            used = sib.setdefault(int(par[v]), set())
            tok = int(trng.integers(0, V))
            while tok in used:
                tok = int(trng.integers(0, V))
            used.add(tok)
            tokens[bb, v] = tok
        has_child = np.zeros(T, dtype=bool)
        for v in range(T):
            if par[v] >= 0:
                has_child[par[v]] = True
        leaves = np.flatnonzero(~has_child)
        leaf = int(leaves[int(trng.integers(0, len(leaves)))])
        chain = []
        cur = leaf
        while cur >= 0:
            chain.append(cur)
            cur = int(par[cur])
        chain.reverse()
        for i, v in enumerate(chain):
            prev_row = 0 if i == 0 else chain[i - 1] + 1
            targets[bb, prev_row] = tokens[bb, v]
            paths[bb, i] = v
        n[bb] = len(chain)
    logits = _planted_logits(B, T + 1, V, torch.from_numpy(targets), (s, rnd, _TID["logits"]),
                             device)
    return dict(parent=torch.from_numpy(parents.astype(np.int32)).to(device),
                draft=torch.from_numpy(tokens.astype(np.int32)).to(device), logits=logits,
                planted_path=paths, n_planted=n)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact up-cast of a generated tensor to a host float64 array."""
    return t.detach().to("cpu", torch.float64).numpy()
