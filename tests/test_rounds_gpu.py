"""GPU tests of the steps around the round: long prefill (T up to 4096, both
gate forms), prefill handing its state and conv window to chained verify
rounds, and rounds whose draft length the host policy picks from measured
round times.  Everything goes through the C ABI and is checked against the
fp64 oracle: indices bit-exact, floats per (layer, seq, head) within 1e-4."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_verify_gdn_amd import binding as gb
from speculative_decode_verify_gdn_amd import policy as pol
from speculative_decode_verify_gdn_amd import spec_round
from speculative_decode_verify_gdn_amd import workload as W

from round_ref import check_units, compare, gpu_outputs, gshape, make_buffers, oracle_round

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.lib()


def _prefill(cfg, inp, gate_per_key=False):
    """gdn_prefill of all cfg.T tokens on fresh device copies; returns (o, S, conv_state)."""
    sh = gb.GdnShape(cfg.L, cfg.B, cfg.Hk, cfg.Hv, cfg.Dk, cfg.Dv, cfg.K, cfg.silu, cfg.eps,
                     cfg.dtype, gate_per_key=gate_per_key)
    d = {k: v.to(DEV) for k, v in inp.items()}
    S, cs = d["S0"].clone(), d["conv_state"].clone()
    o = torch.empty((cfg.L, cfg.B, cfg.T, cfg.Hv, cfg.Dv), device=DEV)
    need = gb.gdn_prefill_workspace_bytes(sh)
    ws = torch.empty((need,), device=DEV, dtype=torch.uint8) if need else None
    err = torch.zeros((1,), device=DEV, dtype=torch.int32)
    gb.gdn_prefill(sh, d["x"], cs, d["conv_w"], d["a"], d["b"], S, o, ws, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return o, S, cs


@pytest.mark.parametrize("T", [1024, 4096])
@pytest.mark.parametrize("gate_per_key", [False, True])
def test_long_prefill(T, gate_per_key):
    """Prefill of 1024 and 4096 tokens (bf16, 128-dim heads: the one-launch
    chunk loop with the state in registers) against the oracle's sequential
    recurrence over every token: all outputs, the final state and the final
    conv window; with the per-v-head gate and with the per-key-channel gate
    drawn U(0.05, 1)."""
    _need_gpu()
    cfg = W.CONFIGS[2].with_(L=1, B=2, Hk=1, Hv=2, T=T)
    inp = W.layer_inputs(cfg, 40 + T, "cpu")
    if gate_per_key:
        gen = torch.Generator().manual_seed(T)
        inp["a"] = (0.05 + 0.95 * torch.rand((cfg.L, cfg.B, T, cfg.Hv, cfg.Dk),
                                             generator=gen)).to(cfg.dtype)
    print("long prefill", T, gate_per_key, flush=True)
    o, S, cs = _prefill(cfg, inp, gate_per_key)
    f = {k: W.to_f64(v) for k, v in inp.items()}
    osh = oracle.Shape(L=cfg.L, B=cfg.B, Hk=cfg.Hk, Hv=cfg.Hv, Dk=cfg.Dk, Dv=cfg.Dv, K=cfg.K,
                       silu=cfg.silu, eps=cfg.eps)
    keys = ("x", "conv_state", "conv_w", "a", "b", "S0")
    if gate_per_key:
        ref = oracle.verify_chunk_vg(osh, *[f[k] for k in keys])
    else:
        ref = oracle.verify_chunk(osh, *[f[k] for k in keys], want_final=True)
    cs_ref, _ = oracle.conv_rollback(osh, f["conv_state"], f["x"], np.full(cfg.B, T, np.int32))
    check_units("o", o, ref["o"], "tok")
    check_units("S", S, ref["S_final"], "state")
    np.testing.assert_array_equal(cs.cpu().double().numpy(), cs_ref)


@pytest.mark.parametrize("cfg_id,L,B,n_pre,rounds", [(1, 1, 1, 64, 20), (3, 2, 3, 100, 5),
                                                       (4, 1, 2, 40, 3)])
def test_prefill_then_chained_rounds(cfg_id, L, B, n_pre, rounds):
    """gdn_prefill commits n_pre tokens, then chained verify rounds (verify,
    greedy accept, tape and conv rollback) go on from the state and window it
    left.  Each side carries its own state; every round matches the oracle's
    plain round.  The first case is the tiny configuration as specified: 64
    prefill tokens from a zero state and window, then rounds of 4 drafts
    (32-dim head: the chunked prefill); the others run the one-launch loop."""
    _need_gpu()
    cfg = W.CONFIGS[cfg_id].with_(L=L, B=B, V=509)
    pre_cfg = cfg.with_(T=n_pre)
    pre = W.layer_inputs(pre_cfg, 1000, "cpu")
    print("prefill then rounds", cfg.name, n_pre, flush=True)
    _, S, cs = _prefill(pre_cfg, pre)
    f = {k: W.to_f64(v) for k, v in pre.items()}
    osh = oracle.Shape(L=L, B=B, Hk=cfg.Hk, Hv=cfg.Hv, Dk=cfg.Dk, Dv=cfg.Dv, K=cfg.K,
                       silu=cfg.silu, eps=cfg.eps)
    ref = oracle.verify_chunk(osh, f["x"], f["conv_state"], f["conv_w"], f["a"], f["b"], f["S0"],
                              want_final=True)
    oS = ref["S_final"]
    ocs, _ = oracle.conv_rollback(osh, f["conv_state"], f["x"], np.full(B, n_pre, np.int32))
    check_units("S after prefill", S, oS, "state")
    np.testing.assert_array_equal(cs.cpu().double().numpy(), ocs)
    kept = 0
    for r in range(rounds):
        inp = W.layer_inputs(cfg, r, "cpu")
        acc = W.chain_accept_inputs(cfg, r, "cpu")
        dev_inp = {k: v.to(DEV) for k, v in inp.items()}
        dev_inp["S0"], dev_inp["conv_state"] = S, cs
        rb = make_buffers(cfg, dev_inp, {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
                                         for k, v in acc.items()})
        spec_round.run_round(rb)
        torch.cuda.synchronize()
        got = gpu_outputs(rb)
        fr = {k: W.to_f64(v) for k, v in inp.items()}
        fr["S0"], fr["conv_state"] = oS, ocs
        r_ref = oracle_round(cfg, fr, acc["draft"].numpy(), W.to_f64(acc["logits"]))
        compare(got, r_ref, tree=False)
        kept += int(r_ref["n_keep"].sum())
        S, cs = rb.S, rb.conv_state
        oS, ocs = r_ref["S_new"], r_ref["cs_new"]
    assert kept > 0


def _round_time_table(cfg, Ns, reps=5):
    """Measured time (us) of one plain round of the stack at each draft length."""
    t = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for n in Ns:
        c = cfg.with_(T=n)
        inp = {k: v.to(DEV) for k, v in W.layer_inputs(c, 0, "cpu").items()}
        acc = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
               for k, v in W.chain_accept_inputs(c, 0, "cpu").items()}
        rb = make_buffers(c, inp, acc)
        spec_round.run_round(rb)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            spec_round.run_round(rb)
        b.record()
        torch.cuda.synchronize()
        t[n] = a.elapsed_time(b) / reps * 1e3
    return t


def test_policy_chooses_draft_length_for_gpu_rounds():
    """Rounds whose draft length DraftPolicy picks before each round from a
    round-time table measured on the GPU and the acceptance seen so far
    (GDN page s2.2: verify cost grows with N; the X article's committed
    tokens per round).  Each round runs through spec_round at the chosen N
    and matches the oracle's plain round.  Then rounds in which every draft
    is rejected: the colibri s4.1 guard disables drafting exactly at the
    first round after which at least 24 drafts were proposed and fewer than
    one in ten accepted."""
    _need_gpu()
    # per-position acceptance 0.85 (as in the 256-sequence block-draft
    # workload), so the guard stays off while the policy picks N
    cfg = W.CONFIGS[3].with_(L=2, B=4, V=611, p_accept=0.85)
    table = _round_time_table(cfg, (1, 2, 4, 8))
    assert all(v > 0 for v in table.values())
    policy = pol.DraftPolicy(t_round_us=table, prior_alpha=0.5)
    inp0 = W.layer_inputs(cfg, 0, "cpu")
    S, cs = inp0["S0"].to(DEV), inp0["conv_state"].to(DEV)
    oS, ocs = W.to_f64(inp0["S0"]), W.to_f64(inp0["conv_state"])
    counts = dict(proposed=0, accepted=0, rej=0)

    def one_round(r, N, forced_n=None):
        nonlocal S, cs, oS, ocs
        c = cfg.with_(T=N)
        inp = W.layer_inputs(c, r, "cpu")
        acc = W.chain_accept_inputs(c, r, "cpu", forced_n=forced_n)
        dev_inp = {k: v.to(DEV) for k, v in inp.items()}
        dev_inp["S0"], dev_inp["conv_state"] = S, cs
        rb = make_buffers(c, dev_inp, {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
                                       for k, v in acc.items()})
        spec_round.run_round(rb)
        torch.cuda.synchronize()
        f = {k: W.to_f64(v) for k, v in inp.items()}
        f["S0"], f["conv_state"] = oS, ocs
        ref = oracle_round(c, f, acc["draft"].numpy(), W.to_f64(acc["logits"]))
        compare(gpu_outputs(rb), ref, tree=False)
        S, cs, oS, ocs = rb.S, rb.conv_state, ref["S_new"], ref["cs_new"]
        policy.record(rb.n_keep, N)
        n = ref["n_keep"]
        counts["proposed"] += n.size * N
        counts["accepted"] += int(n.sum())
        counts["rej"] += int(np.count_nonzero(n < N))

    def guard_rule():
        return counts["proposed"] >= 24 and counts["accepted"] * 10 < counts["proposed"]

    chosen = []
    for r in range(6):
        a = None if counts["accepted"] + counts["rej"] == 0 else \
            counts["accepted"] / (counts["accepted"] + counts["rej"])
        want = 0 if guard_rule() else pol.choose_draft_length(0.5 if a is None else a, table)
        N = policy.next_draft_length()
        assert N == want and N in table, (r, counts, N, want)
        print("policy round", r, "N", N, flush=True)
        chosen.append(N)
        one_round(r, N)
    # every draft rejected from here on: the guard fires exactly when its rule holds
    fired = False
    for r in range(6, 200):
        rule = guard_rule()
        N = policy.next_draft_length()
        assert (N == 0) == rule, (r, counts, N)
        if rule:
            fired = True
            break
        one_round(r, N, forced_n=0)
    assert fired and chosen
