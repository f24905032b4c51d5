"""Seeded workload generator: reproducibility, distributions and structure."""
import math

import numpy as np
import pytest
import torch

from oracle import cost_model as cm
from speculative_decode_verify_gdn_amd import workload as W


def test_seeds_reproduce_bytes():
    cfg = W.CONFIGS[2]
    a = W.layer_inputs(cfg, 5)
    b = W.layer_inputs(cfg, 5)
    c = W.layer_inputs(cfg, 6)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    assert not torch.equal(a["x"], c["x"])
    assert torch.equal(a["S0"], c["S0"])  # initial state does not depend on the round


def test_value_ranges_and_dtypes():
    cfg = W.CONFIGS[2]
    d = W.layer_inputs(cfg, 0)
    assert d["x"].dtype == torch.bfloat16 and d["S0"].dtype == torch.float32
    a = d["a"].float()
    assert float(a.min()) >= math.exp(-0.5) - 0.01 and float(a.max()) <= math.exp(-0.01) + 0.005
    b = d["b"].float()
    assert 0 < float(b.min()) and float(b.max()) < 1
    assert abs(float(d["S0"].std()) - 0.1) < 0.002
    assert abs(float(d["x"].float().std()) - 1.0) < 0.02
    c1 = W.layer_inputs(W.CONFIGS[1], 0)
    assert float(c1["S0"].abs().max()) == 0.0 and float(c1["conv_state"].abs().max()) == 0.0


@pytest.mark.parametrize("p,T", [(0.36, 8), (0.85, 16)])
def test_bernoulli_prefix_is_geometric(p, T):
    cfg = W.CONFIGS[3].with_(p_accept=p, T=T, B=4000, V=64)
    counts = np.zeros(T + 1)
    for r in range(3):
        d = W.chain_accept_inputs(cfg, r)
        counts += np.bincount(d["n_planted"], minlength=T + 1)
    N = counts.sum()
    for k in range(T + 1):
        pk = cm.p_accept_exactly(p, T, k)
        sd = math.sqrt(N * pk * (1 - pk))
        assert abs(counts[k] - N * pk) <= 4 * sd + 1, (k, counts[k], N * pk)


def test_uniform_law():
    cfg = W.CONFIGS[2].with_(B=6000, V=64)
    d = W.chain_accept_inputs(cfg, 0)
    counts = np.bincount(d["n_planted"], minlength=5)
    N = counts.sum()
    for k in range(5):
        sd = math.sqrt(N * 0.2 * 0.8)
        assert abs(counts[k] - N * 0.2) <= 4 * sd


def test_planted_target_is_unique_bf16_argmax():
    cfg = W.CONFIGS[3].with_(B=8, V=5000)
    d = W.chain_accept_inputs(cfg, 1)
    lg = d["logits"].float()
    mx = lg.max(-1)
    assert torch.equal(mx.indices.int(), torch.from_numpy(d["targets"]))
    assert int((lg == mx.values.unsqueeze(-1)).sum()) == lg.shape[0] * lg.shape[1]


def test_tree_structure_bounds():
    cfg = W.CONFIGS[5].with_(B=64, V=3000)
    d = W.tree_accept_inputs(cfg, 0)
    par = d["parent"].numpy()
    tok = d["draft"].numpy()
    depths = []
    for b in range(cfg.B):
        depth = {-1: 0}
        kids = {}
        for v in range(cfg.T):
            p = int(par[b, v])
            assert -1 <= p < v
            depth[v] = depth[p] + 1
            assert depth[v] <= cfg.max_depth
            kids.setdefault(p, []).append(v)
        for p, ks in kids.items():
            assert len(ks) <= cfg.branching
            assert len(set(tok[b, ks])) == len(ks)  # distinct sibling tokens
        depths.append(d["n_planted"][b])
    assert 1 <= min(depths) and max(depths) <= cfg.max_depth
