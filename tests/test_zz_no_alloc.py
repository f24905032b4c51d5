"""spec_accept_prefix_noalloc (static scratch, no allocation) against
spec_accept_prefix (caller's workspace), through the C ABI: two calls in a
row, the second smaller, each bit-exact with the workspace entry point and the
oracle; and the host-side size limit."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_verify_gdn_amd import binding as gb
from speculative_decode_verify_gdn_amd import workload as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(fn_noalloc, draft, logits, parent):
    B, T = draft.shape
    out = [torch.full((B,), -9, dtype=torch.int32, device=DEV),
           torch.full((B, T), -9, dtype=torch.int32, device=DEV),
           torch.full((B,), -9, dtype=torch.int32, device=DEV)]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    if fn_noalloc:
        gb.spec_accept_prefix_noalloc(draft, logits, *out, parent=parent, dev_err=err)
    else:
        ws = torch.empty(gb.spec_accept_workspace_bytes(B, T, logits.shape[-1]),
                         dtype=torch.uint8, device=DEV)
        gb.spec_accept_prefix(draft, logits, *out, ws, parent=parent, dev_err=err)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out] + [int(err.item())]


def test_noalloc_accept_matches_workspace_entry_point_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.lib()
    cases = [
        # the 32-sequence, 8-draft chain workload at the full vocabulary
        (W.CONFIGS[3], 0, None),
        # then a smaller draft-tree call: 5 trees of 12 nodes, 1001 tokens
        (W.CONFIGS[5].with_(B=5, T=12, V=1001), 3, "tree"),
    ]
    for cfg, rnd, kind in cases:
        acc = (W.tree_accept_inputs(cfg, rnd, DEV) if kind == "tree"
               else W.chain_accept_inputs(cfg, rnd, DEV))
        parent = acc["parent"] if kind == "tree" else None
        print("noalloc accept", cfg.name, cfg.B, cfg.T, cfg.V, flush=True)
        a = _run(True, acc["draft"], acc["logits"], parent)
        b = _run(False, acc["draft"], acc["logits"], parent)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
        n, path, bonus = oracle.accept(acc["draft"].cpu().numpy(), W.to_f64(acc["logits"]),
                                       None if parent is None else parent.cpu().numpy())
        np.testing.assert_array_equal(a[0], n)
        np.testing.assert_array_equal(a[1], path)
        np.testing.assert_array_equal(a[2], bonus)
        np.testing.assert_array_equal(a[0], acc["n_planted"])
        assert a[3] == 0


def test_noalloc_accept_oversize_is_refused():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B, T, V = 2100, 63, 7
    draft = torch.zeros((B, T), dtype=torch.int32, device=DEV)
    logits = torch.zeros((B, T + 1, V), dtype=torch.bfloat16, device=DEV)
    outs = [torch.empty((B,), dtype=torch.int32, device=DEV),
            torch.empty((B, T), dtype=torch.int32, device=DEV),
            torch.empty((B,), dtype=torch.int32, device=DEV)]
    with pytest.raises(gb.GdnError) as e:
        gb.spec_accept_prefix_noalloc(draft, logits, *outs)
    assert e.value.status == gb.GDN_ERR_SCRATCH
