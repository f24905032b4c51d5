"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Indices (accepted lengths, paths, bonus tokens, conv-window indices) must be
bit-exact, the rolled-back conv window byte-exact, the decay tape exact, and
states, outputs and tape entries within relative Frobenius error 1e-4.
Small cases run every output through the oracle; full-size cases run the
round exactly as the benchmark does and check sampled (layer, sequence)
units.
"""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_verify_gdn_amd import binding as gb
from speculative_decode_verify_gdn_amd import spec_round
from speculative_decode_verify_gdn_amd import workload as W

from round_ref import check_units, compare, gpu_outputs, gshape, make_buffers, oracle_round

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.lib()


def host_round_inputs(cfg, rnd, T=None, V=None, forced_n=None):
    """Inputs drawn on the host (exact same bytes go to oracle and GPU)."""
    inp = W.layer_inputs(cfg, rnd, "cpu", T=T)
    if cfg.is_tree:
        acc = W.tree_accept_inputs(cfg, rnd, "cpu", T=T, V=V)
    else:
        acc = W.chain_accept_inputs(cfg, rnd, "cpu", T=T, V=V, forced_n=forced_n)
    return inp, acc


def run_pair(cfg, inp, acc, T=None):
    """One round on GPU and oracle from host tensors; returns (got, ref)."""
    dev_inp = {k: v.to(DEV) for k, v in inp.items()}
    dev_acc = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in acc.items()}
    rb = make_buffers(cfg, dev_inp, dev_acc)
    f64 = {k: W.to_f64(v) for k, v in inp.items()}
    spec_round.run_round(rb)
    torch.cuda.synchronize()
    got = gpu_outputs(rb)
    parent = acc["parent"].numpy() if cfg.is_tree else None
    ref = oracle_round(cfg, f64, acc["draft"].numpy(), W.to_f64(acc["logits"]), parent)
    return got, ref


# ------------------------------------------------ configs 1-2, every round --

def test_cfg1_tiny_prefill_then_chained_rounds():
    _need_gpu()
    cfg = W.CONFIGS[1]
    sh_o = oracle.Shape(1, 1, 1, 1, 32, 32, 4, True, cfg.eps)
    # prefill: verify 64 tokens from zero state and window, commit all of them
    pre = W.layer_inputs(cfg, 1000, "cpu", T=cfg.prefill)
    dev = {k: v.to(DEV) for k, v in pre.items()}
    gsh = gb.GdnShape(1, 1, 1, 1, 32, 32, 4, True, cfg.eps, torch.float32)
    o = torch.empty((1, 1, 64, 1, 32), device=DEV)
    tape = gb.Tape.empty(gsh, 64, DEV)
    gb.gdn_verify_chunk(gsh, dev["x"], dev["conv_state"], dev["conv_w"], dev["a"], dev["b"],
                        dev["S0"], o, tape)
    nk = torch.full((1,), 64, dtype=torch.int32, device=DEV)
    S, cs = dev["S0"].clone(), dev["conv_state"].clone()
    gb.gdn_tape_rollback(gsh, S, tape, nk)
    gb.gdn_conv_state_rollback(gsh, cs, dev["x"], nk)
    f = {k: W.to_f64(v) for k, v in pre.items()}
    ref = oracle.verify_chunk(sh_o, f["x"], f["conv_state"], f["conv_w"], f["a"], f["b"], f["S0"])
    check_units("o", o, ref["o"], "tok")
    check_units("S", S, ref["S_final"], "state")
    oS = ref["S_final"]
    ocs, _ = oracle.conv_rollback(sh_o, f["conv_state"], f["x"], np.array([64], np.int32))
    np.testing.assert_array_equal(cs.cpu().double().numpy(), ocs)
    # chained rounds: each side carries its own state
    worst = 0.0
    for rnd in range(20):
        inp = W.layer_inputs(cfg, rnd, "cpu")
        acc = W.chain_accept_inputs(cfg, rnd, "cpu")
        inp["S0"] = S.cpu()
        inp["conv_state"] = cs.cpu()
        dev_inp = {k: v.to(DEV) for k, v in inp.items()}
        rb = make_buffers(cfg, dev_inp, {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
                                         for k, v in acc.items()})
        spec_round.run_round(rb)
        torch.cuda.synchronize()
        got = gpu_outputs(rb)
        f = {k: W.to_f64(v) for k, v in inp.items()}
        f["S0"], f["conv_state"] = oS, ocs
        r = oracle_round(cfg, f, acc["draft"].numpy(), W.to_f64(acc["logits"]))
        errs = compare(got, r, tree=False)
        worst = max(worst, max(errs.values()))
        S, cs = rb.S, rb.conv_state
        oS, ocs = r["S_new"], r["cs_new"]
    assert worst <= 1e-4


def test_cfg2_one_layer_chained_rounds():
    _need_gpu()
    cfg = W.CONFIGS[2]
    inp0 = W.layer_inputs(cfg, 0, "cpu")
    S, cs = inp0["S0"].to(DEV), inp0["conv_state"].to(DEV)
    oS, ocs = W.to_f64(inp0["S0"]), W.to_f64(inp0["conv_state"])
    for rnd in range(6):
        inp = W.layer_inputs(cfg, rnd, "cpu")
        acc = W.chain_accept_inputs(cfg, rnd, "cpu")
        dev_inp = {k: v.to(DEV) for k, v in inp.items()}
        dev_inp["S0"], dev_inp["conv_state"] = S, cs
        rb = make_buffers(cfg, dev_inp, {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
                                         for k, v in acc.items()})
        spec_round.run_round(rb)
        torch.cuda.synchronize()
        got = gpu_outputs(rb)
        f = {k: W.to_f64(v) for k, v in inp.items()}
        f["S0"], f["conv_state"] = oS, ocs
        r = oracle_round(cfg, f, acc["draft"].numpy(), W.to_f64(acc["logits"]))
        compare(got, r, tree=False)
        oS, ocs = r["S_new"], r["cs_new"]


# -------------------------------------------- configs 3-5 at reduced size --

@pytest.mark.parametrize("cfg_id,L,B", [(3, 2, 5), (4, 2, 3), (5, 2, 3)])
def test_reduced_stack_rounds(cfg_id, L, B):
    _need_gpu()
    cfg = W.CONFIGS[cfg_id].with_(L=L, B=B)
    for rnd in range(2):
        inp, acc = host_round_inputs(cfg, rnd)
        got, ref = run_pair(cfg, inp, acc)
        compare(got, ref, tree=cfg.is_tree)


# ---------------------------------------------- ragged and degenerate cases -

@pytest.mark.parametrize("T", [1, 2, 3, 5, 7, 9, 13, 16, 17, 31, 33, 64])
def test_chain_lengths(T):
    _need_gpu()
    cfg = W.CONFIGS[3].with_(L=1, B=3, Hk=2, Hv=4, T=T, V=1001, law="uniform")
    inp, acc = host_round_inputs(cfg, 7)
    got, ref = run_pair(cfg, inp, acc)
    compare(got, ref, tree=False)


@pytest.mark.parametrize("D,Hk,Hv,K,silu,dtype", [
    (64, 2, 8, 4, True, torch.bfloat16),
    (32, 3, 3, 2, True, torch.float32),
    (128, 1, 4, 3, False, torch.float32),
    (64, 4, 4, 6, True, torch.bfloat16),
    (128, 2, 2, 8, True, torch.bfloat16),
])
def test_shapes_and_dtypes(D, Hk, Hv, K, silu, dtype):
    _need_gpu()
    cfg = W.CONFIGS[3].with_(L=2, B=3, Hk=Hk, Hv=Hv, Dk=D, Dv=D, K=K, silu=silu, dtype=dtype,
                             T=6, V=333)
    inp, acc = host_round_inputs(cfg, 3)
    got, ref = run_pair(cfg, inp, acc)
    compare(got, ref, tree=False)


@pytest.mark.parametrize("D,K,silu,dtype", [
    (128, 8, True, torch.float32),    # 16-token chunk, prologue loads one channel pair at a time
    (128, 3, False, torch.bfloat16),
    (64, 6, True, torch.float32),
    (32, 4, True, torch.bfloat16),
])
def test_sixteen_token_chunks(D, K, silu, dtype):
    """Chains of 16 tokens (the block-draft length) across head sizes, conv
    widths and input types."""
    _need_gpu()
    cfg = W.CONFIGS[4].with_(L=2, B=3, Hk=2, Hv=4, Dk=D, Dv=D, K=K, silu=silu, dtype=dtype,
                             V=257)
    inp, acc = host_round_inputs(cfg, 4)
    got, ref = run_pair(cfg, inp, acc)
    compare(got, ref, tree=False)


@pytest.mark.parametrize("T,K,silu,depth", [(48, 3, False, 8), (64, 8, True, 8), (33, 2, True, 12)])
def test_tree_conv_widths(T, K, silu, depth):
    """Trees of 33..64 nodes with conv widths other than 4 (windows that reach
    past the old rows), SiLU off, and depths past the unrolled path solve."""
    _need_gpu()
    cfg = W.CONFIGS[5].with_(L=1, B=3, Hk=2, Hv=4, T=T, K=K, silu=silu, V=300, max_depth=depth)
    inp, acc = host_round_inputs(cfg, 6)
    got, ref = run_pair(cfg, inp, acc)
    compare(got, ref, tree=True)


@pytest.mark.parametrize("n", [0, "T"])
def test_all_rejected_and_all_accepted(n):
    _need_gpu()
    cfg = W.CONFIGS[3].with_(L=2, B=4, V=500)
    forced = cfg.T if n == "T" else 0
    inp, acc = host_round_inputs(cfg, 2, forced_n=forced)
    got, ref = run_pair(cfg, inp, acc)
    compare(got, ref, tree=False)
    if forced == 0:  # the snapshot must be left bit-identical
        assert torch.equal(got["S_new"], inp["S0"])
        assert torch.equal(got["cs_new"], inp["conv_state"])


@pytest.mark.parametrize("T,branching,depth", [(1, 4, 8), (5, 4, 8), (16, 4, 8), (17, 4, 8),
                                               (24, 2, 12), (32, 4, 8), (37, 4, 8), (64, 4, 8),
                                               (64, 64, 1), (64, 1, 64), (40, 2, 20),
                                               (33, 1, 33), (64, 3, 16)])
def test_tree_shapes(T, branching, depth):
    _need_gpu()
    cfg = W.CONFIGS[5].with_(L=1, B=3, Hk=2, Hv=4, T=T, V=700, branching=branching,
                             max_depth=depth)
    inp, acc = host_round_inputs(cfg, 5)
    got, ref = run_pair(cfg, inp, acc)
    compare(got, ref, tree=True)


def test_tree_with_chain_parents_equals_chunk():
    """A chain is the tree with parent t-1 (GDN page s8: tree-aware verify
    generalises the chunk).  The two calls run different kernels, so the
    results agree up to rounding: within the parity bar, with the gate tape
    (a copy of the input) bit-exact."""
    _need_gpu()
    cfg = W.CONFIGS[3].with_(L=1, B=2, Hk=2, Hv=4, T=9, V=100)
    inp, acc = host_round_inputs(cfg, 1)
    d = {k: v.to(DEV) for k, v in inp.items()}
    sh = gb.GdnShape(1, 2, 2, 4, 128, 128, 4, True, cfg.eps, cfg.dtype)
    outs = []
    for tree in (False, True):
        o = torch.empty((1, 2, 9, 4, 128), device=DEV)
        tape = gb.Tape.empty(sh, 9, DEV)
        if tree:
            par = torch.arange(-1, 8, dtype=torch.int32, device=DEV).repeat(2, 1).contiguous()
            gb.gdn_tree_verify(sh, par, d["x"], d["conv_state"], d["conv_w"], d["a"], d["b"],
                               d["S0"], o, tape)
        else:
            gb.gdn_verify_chunk(sh, d["x"], d["conv_state"], d["conv_w"], d["a"], d["b"],
                                d["S0"], o, tape)
        outs.append((o, tape))
    torch.cuda.synchronize()
    check_units("o", outs[1][0], outs[0][0], "tok")
    check_units("u", outs[1][1].u, outs[0][1].u, "tok")
    check_units("k", outs[1][1].k, outs[0][1].k, "tok")
    assert torch.equal(outs[0][1].g, outs[1][1].g)


@pytest.mark.parametrize("cfg_id,L,B,rounds,forced", [
    (2, 1, 1, 6, None), (3, 2, 5, 5, None), (4, 2, 3, 4, None), (3, 2, 4, 3, "T"),
    (3, 2, 4, 3, 0), (4, 1, 2, 3, "T")])
def test_fused_replay_rounds(cfg_id, L, B, rounds, forced):
    """Rounds whose state rollback is folded into the next round's verify of
    each layer (gdn_verify_chunk_replay, GDN page s4 replay applied one verify
    later) give the oracle's plain rounds: outputs, tape, accepted lengths,
    conv windows every round, and the state after the last accepted prefix."""
    _need_gpu()
    cfg = W.CONFIGS[cfg_id].with_(L=L, B=B, V=601)
    inp0 = W.layer_inputs(cfg, 0, "cpu")
    oS, ocs = W.to_f64(inp0["S0"]), W.to_f64(inp0["conv_state"])
    fr = None
    for r in range(rounds):
        inp = W.layer_inputs(cfg, r, "cpu")
        forced_n = None if forced is None else (cfg.T if forced == "T" else 0)
        acc = W.chain_accept_inputs(cfg, r, "cpu", forced_n=forced_n)
        d = {k: v.to(DEV) for k, v in inp.items()}
        da = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in acc.items()}
        if fr is None:
            d["S0"], d["conv_state"] = inp0["S0"].to(DEV), inp0["conv_state"].to(DEV)
            fr = spec_round.FusedRound(make_buffers(cfg, d, da))
        else:
            rb = fr.rb
            rb.x, rb.a, rb.b, rb.conv_w = d["x"], d["a"], d["b"], d["conv_w"]
            rb.logits, rb.draft = da["logits"], da["draft"]
        fr.round(r, first=(r == 0))
        torch.cuda.synchronize()
        f = {k: W.to_f64(v) for k, v in inp.items()}
        f["S0"], f["conv_state"] = oS, ocs
        ref = oracle_round(cfg, f, acc["draft"].numpy(), W.to_f64(acc["logits"]))
        tape = fr.tapes[r % 2]
        np.testing.assert_array_equal(fr.n_keeps[r % 2].cpu().numpy(), ref["n_keep"])
        np.testing.assert_array_equal(fr.rb.bonus.cpu().numpy(), ref["bonus"])
        np.testing.assert_array_equal(fr.rb.conv_state.cpu().double().numpy(), ref["cs_new"])
        for name, got, want in (("o", fr.rb.o, ref["o"]), ("u", tape.u, ref["u"]),
                                ("k", tape.k, ref["k"])):
            check_units("%s, round %d" % (name, r), got, want, "tok")
        np.testing.assert_array_equal(tape.g.cpu().double().numpy(), ref["g"])
        oS, ocs = ref["S_new"], ref["cs_new"]
    fr.finish(rounds - 1)
    torch.cuda.synchronize()
    check_units("S", fr.rb.S, oS, "state")
    assert int(fr.rb.dev_err.item()) == 0


@pytest.mark.parametrize("L,B,rounds,T", [(2, 3, 4, 64), (1, 2, 3, 40), (1, 2, 3, 24),
                                          (1, 2, 3, 17), (1, 2, 3, 12)])
def test_fused_replay_tree_rounds(L, B, rounds, T):
    """Tree rounds with the rollback folded into the next verify
    (gdn_tree_verify_replay) give the oracle's plain tree rounds every round
    and after finish(); T = 12 runs the library's two-call form."""
    _need_gpu()
    cfg = W.CONFIGS[5].with_(L=L, B=B, T=T, V=311)
    inp0 = W.layer_inputs(cfg, 0, "cpu")
    oS, ocs = W.to_f64(inp0["S0"]), W.to_f64(inp0["conv_state"])
    fr = None
    for r in range(rounds):
        inp = W.layer_inputs(cfg, r, "cpu")
        acc = W.tree_accept_inputs(cfg, r, "cpu")
        d = {k: v.to(DEV) for k, v in inp.items()}
        da = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in acc.items()}
        if fr is None:
            d["S0"], d["conv_state"] = inp0["S0"].to(DEV), inp0["conv_state"].to(DEV)
            fr = spec_round.FusedRound(make_buffers(cfg, d, da))
        else:
            rb = fr.rb
            rb.x, rb.a, rb.b, rb.conv_w = d["x"], d["a"], d["b"], d["conv_w"]
            rb.logits, rb.draft, rb.parent = da["logits"], da["draft"], da["parent"]
        fr.round(r, first=(r == 0))
        torch.cuda.synchronize()
        f = {k: W.to_f64(v) for k, v in inp.items()}
        f["S0"], f["conv_state"] = oS, ocs
        ref = oracle_round(cfg, f, acc["draft"].numpy(), W.to_f64(acc["logits"]),
                           parent=acc["parent"].numpy())
        tape = fr.tapes[r % 2]
        np.testing.assert_array_equal(fr.n_keeps[r % 2].cpu().numpy(), ref["n_keep"])
        np.testing.assert_array_equal(fr.paths[r % 2].cpu().numpy(), ref["path"])
        np.testing.assert_array_equal(fr.rb.bonus.cpu().numpy(), ref["bonus"])
        np.testing.assert_array_equal(fr.rb.conv_win.cpu().numpy(), ref["conv_win"])
        np.testing.assert_array_equal(fr.rb.conv_state.cpu().double().numpy(), ref["cs_new"])
        for name, got, want in (("o", fr.rb.o, ref["o"]), ("u", tape.u, ref["u"]),
                                ("k", tape.k, ref["k"])):
            check_units("%s, round %d" % (name, r), got, want, "tok")
        np.testing.assert_array_equal(tape.g.cpu().double().numpy(), ref["g"])
        oS, ocs = ref["S_new"], ref["cs_new"]
    fr.finish(rounds - 1)
    torch.cuda.synchronize()
    check_units("S", fr.rb.S, oS, "state")
    assert int(fr.rb.dev_err.item()) == 0


def test_fused_tree_replay_bad_inputs_flag():
    """A previous path entry outside [0, prev_T) sets GDN_DEV_ERR_PATH and the
    sequence is verified from its state unchanged; a malformed parent array
    sets GDN_DEV_ERR_PARENT and the replay is still applied."""
    _need_gpu()
    cfg = W.CONFIGS[5].with_(L=1, B=2, T=40, V=97)
    inp = W.layer_inputs(cfg, 0, "cpu")
    acc = W.tree_accept_inputs(cfg, 0, "cpu")
    d = {k: v.to(DEV) for k, v in inp.items()}
    sh = gshape(cfg)
    gen = torch.Generator(device="cpu").manual_seed(7)
    prev = gb.Tape.empty(sh, cfg.T, DEV)
    for t in (prev.u, prev.k):
        t.copy_(torch.randn(t.shape, generator=gen).to(DEV) * 0.1)
    prev.g.fill_(0.9)
    pn = torch.tensor([3, 2], dtype=torch.int32, device=DEV)
    ppath = torch.full((2, cfg.T), -1, dtype=torch.int32, device=DEV)
    ppath[0, :3] = torch.tensor([0, 5, 9], dtype=torch.int32)
    ppath[1, :2] = torch.tensor([1, cfg.T], dtype=torch.int32)  # out of range
    parent = acc["parent"].clone()
    parent[0, 7] = 7  # not an earlier node: malformed
    o = torch.empty((1, 2, cfg.T, cfg.Hv, cfg.Dv), device=DEV)
    cur = gb.Tape.empty(sh, cfg.T, DEV)
    err = torch.zeros((1,), dtype=torch.int32, device=DEV)
    S = d["S0"].clone()
    gb.gdn_tree_verify_replay(sh, parent.to(DEV), d["x"], d["conv_state"], d["conv_w"], d["a"],
                              d["b"], S, o, cur, prev, pn, prev_path=ppath, dev_err=err)
    torch.cuda.synchronize()
    e = int(err.item())
    assert e & gb.DEV_ERR_PATH and e & gb.DEV_ERR_PARENT
    # sequence 1: bad path, state unchanged
    assert torch.equal(S[:, 1], d["S0"][:, 1])
    # sequence 0: replayed exactly as the standalone rollback does it
    S_ref = d["S0"].clone()
    gb.gdn_tape_rollback(sh, S_ref, prev, torch.tensor([3, 0], dtype=torch.int32, device=DEV),
                         path=ppath.clamp(0, cfg.T - 1))
    torch.cuda.synchronize()
    check_units("S", S[:, 0], S_ref[:, 0], "state", 1e-5)


@pytest.mark.parametrize("Hk,Hv,chain", [(2, 4, 24), (2, 4, 25), (2, 4, 40), (2, 2, 25),
                                         (2, 2, 64)])
def test_tree_verify_long_chain_with_branches(Hk, Hv, chain):
    """64-node trees made of a chain of `chain` nodes with the others hung
    at random below it: the deepest path lies on either side of the depth at
    which the packed solve switches from one row per lane to one column per
    lane.  Outputs and tape against the oracle's tree_verify."""
    _need_gpu()
    from round_ref import oshape
    cfg = W.CONFIGS[5].with_(L=1, B=3, Hk=Hk, Hv=Hv, T=64, V=97)
    inp = W.layer_inputs(cfg, 7, "cpu")
    rng = np.random.default_rng(chain)
    parent = torch.tensor([[t - 1 for t in range(chain)] +
                           [int(rng.integers(0, t)) for t in range(chain, cfg.T)]
                           for _ in range(cfg.B)], dtype=torch.int32)
    sh, osh = gshape(cfg), oshape(cfg)
    d = {k: v.to(DEV) for k, v in inp.items()}
    o = torch.empty((1, cfg.B, cfg.T, Hv, cfg.Dv), device=DEV)
    tape = gb.Tape.empty(sh, cfg.T, DEV)
    print("tree long chain", Hk, Hv, chain, flush=True)
    gb.gdn_tree_verify(sh, parent.to(DEV), d["x"], d["conv_state"], d["conv_w"], d["a"], d["b"],
                       d["S0"], o, tape)
    torch.cuda.synchronize()
    f = {k: W.to_f64(v) for k, v in inp.items()}
    ref = oracle.tree_verify(osh, parent.numpy(), f["x"], f["conv_state"], f["conv_w"], f["a"],
                             f["b"], f["S0"])
    for name, got in (("o", o), ("u", tape.u), ("k", tape.k)):
        check_units(name, got, ref[name], "tok")


@pytest.mark.parametrize("Hk,Hv,K,T,branching,depth", [
    (2, 4, 4, 48, 4, 8), (2, 2, 4, 64, 4, 8), (1, 4, 3, 40, 4, 8),
    (2, 4, 4, 64, 1, 64), (2, 4, 4, 48, 2, 20), (1, 4, 4, 64, 1, 64), (2, 4, 4, 20, 4, 8)])
def test_tree_replay_long_previous_paths(Hk, Hv, K, T, branching, depth):
    """gdn_tree_verify_replay with previous paths of 0, 9, 20 and 64 steps
    (beyond the operands preloaded into registers): the state equals the
    oracle's tape_rollback along the path and the outputs its tree_verify from
    that state.  The cases cover two v-heads per workgroup and the one-head
    form (one v-head per k-head; conv width 3), trees deeper than the
    register solve (a 64-node chain and depth 20), and a 20-node tree after
    a 64-entry previous path."""
    _need_gpu()
    from round_ref import oshape
    cfg = W.CONFIGS[5].with_(L=1, B=4, Hk=Hk, Hv=Hv, K=K, T=T, V=97, branching=branching,
                             max_depth=depth)
    inp = W.layer_inputs(cfg, 3, "cpu")
    parent = W.tree_accept_inputs(cfg, 3, "cpu")["parent"]
    sh, osh = gshape(cfg), oshape(cfg)
    pT = 64
    gen = torch.Generator().manual_seed(55 + Hv + K)
    pu = torch.randn((1, cfg.B, pT, Hv, cfg.Dv), generator=gen) * 0.2
    pk = torch.nn.functional.normalize(torch.randn((1, cfg.B, pT, Hk, cfg.Dk), generator=gen),
                                       dim=-1)
    pg = 0.6 + 0.4 * torch.rand((1, cfg.B, pT, Hv), generator=gen)
    nk = torch.tensor([0, 9, 20, 64], dtype=torch.int32)
    path = torch.full((cfg.B, pT), -1, dtype=torch.int32)
    for bb in range(cfg.B):
        path[bb, :int(nk[bb])] = torch.randperm(pT, generator=gen)[:int(nk[bb])].to(torch.int32)
    d = {k: v.to(DEV) for k, v in inp.items()}
    S = d["S0"].clone()
    o = torch.empty((1, cfg.B, T, Hv, cfg.Dv), device=DEV)
    tape = gb.Tape.empty(sh, T, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("tree replay long paths", Hk, Hv, K, T, branching, depth, flush=True)
    gb.gdn_tree_verify_replay(sh, parent.to(DEV), d["x"], d["conv_state"], d["conv_w"], d["a"],
                              d["b"], S, o, tape, gb.Tape(pu.to(DEV), pk.to(DEV), pg.to(DEV)),
                              nk.to(DEV), prev_path=path.to(DEV), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    f = {k: W.to_f64(v) for k, v in inp.items()}
    S_rep = oracle.tape_rollback(osh, f["S0"], pu.double().numpy(), pk.double().numpy(),
                                 pg.double().numpy(), nk.numpy(), path.numpy())
    check_units("S", S, S_rep, "state", 1e-5)
    assert torch.equal(S[:, 0].cpu(), inp["S0"][:, 0])
    ref = oracle.tree_verify(osh, parent.numpy(), f["x"], f["conv_state"], f["conv_w"], f["a"],
                             f["b"], S_rep)
    for name, got in (("o", o), ("u", tape.u), ("k", tape.k)):
        check_units(name, got, ref[name], "tok")


def test_fused_replay_bad_prev_n_keep_flags():
    """An accepted length outside [0, prev_T] sets GDN_DEV_ERR_N_KEEP and
    that sequence is verified from its state unchanged."""
    _need_gpu()
    cfg = W.CONFIGS[3].with_(L=1, B=2, V=97)
    inp = W.layer_inputs(cfg, 0, "cpu")
    d = {k: v.to(DEV) for k, v in inp.items()}
    sh = gshape(cfg)
    prev = gb.Tape.empty(sh, cfg.T, DEV)
    for t in (prev.u, prev.k, prev.g):
        t.fill_(1.0)
    cur = gb.Tape.empty(sh, cfg.T, DEV)
    o = torch.empty((1, 2, cfg.T, cfg.Hv, cfg.Dv), device=DEV)
    pn = torch.tensor([cfg.T + 1, 0], dtype=torch.int32, device=DEV)
    err = torch.zeros((1,), dtype=torch.int32, device=DEV)
    S = d["S0"].clone()
    gb.gdn_verify_chunk_replay(sh, d["x"], d["conv_state"], d["conv_w"], d["a"], d["b"], S, o,
                               cur, prev, pn, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & gb.DEV_ERR_N_KEEP
    assert torch.equal(S, d["S0"])


# -------------------------------------------------------------- accept only -

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V", [7, 1001, 151936])
def test_accept_ties_and_ragged_vocab(dtype, V):
    _need_gpu()
    rng = np.random.default_rng(V)
    B, T = 9, 6
    lg = rng.integers(-3, 4, size=(B, T + 1, V)).astype(np.float32)  # many exact ties
    lg_t = torch.from_numpy(lg).to(dtype)
    star = lg.argmax(-1)
    draft = np.where(rng.random((B, T)) < 0.8, star[:, :T], rng.integers(0, V, (B, T)))
    d = torch.from_numpy(draft.astype(np.int32))
    for parent in (None, np.stack([W.random_tree(rng, T, 2, 4) for _ in range(B)])):
        nk = torch.empty(B, dtype=torch.int32, device=DEV)
        path = torch.empty((B, T), dtype=torch.int32, device=DEV)
        bonus = torch.empty(B, dtype=torch.int32, device=DEV)
        ws = torch.empty(gb.spec_accept_workspace_bytes(B, T, V), dtype=torch.uint8, device=DEV)
        par_t = None if parent is None else torch.from_numpy(parent.astype(np.int32)).to(DEV)
        gb.spec_accept_prefix(d.to(DEV), lg_t.to(DEV), nk, path, bonus, ws, parent=par_t)
        n_ref, p_ref, b_ref = oracle.accept(draft, lg_t.double().numpy(), parent)
        np.testing.assert_array_equal(nk.cpu().numpy(), n_ref)
        np.testing.assert_array_equal(path.cpu().numpy(), p_ref)
        np.testing.assert_array_equal(bonus.cpu().numpy(), b_ref)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V", [9, 4100, 151936])
def test_accept_infinite_and_nan_rows(dtype, V):
    """Rows of -inf (fully masked), -inf-padded rows, rows with +inf entries
    and rows with NaN entries or only NaN: the accepted lengths, paths and
    bonus tokens equal the oracle's (NaN never the argmax, a row with no
    number gives 0), every index stays in [0, V), and GDN_DEV_ERR_NAN is set
    exactly when some row holds a NaN."""
    _need_gpu()
    rng = np.random.default_rng(V + (1 if dtype == torch.float32 else 0))
    B, T = 12, 5
    lg = rng.integers(-3, 4, size=(B, T + 1, V)).astype(np.float32)
    kinds = rng.integers(0, 6, size=(B, T + 1))
    kinds[0, :] = 1   # a sequence of -inf rows only
    kinds[1, 0] = 4   # a row of NaN only
    for bb in range(B):
        for r in range(T + 1):
            k = kinds[bb, r]
            if k == 1:
                lg[bb, r, :] = -np.inf
            elif k == 2:
                lg[bb, r, int(rng.integers(1, V)):] = -np.inf
            elif k == 3:
                lg[bb, r, rng.integers(0, V, size=3)] = np.nan
            elif k == 4:
                lg[bb, r, :] = np.nan
            elif k == 5:
                lg[bb, r, rng.integers(0, V, size=2)] = np.inf
    lg_t = torch.from_numpy(lg).to(dtype)
    lg64 = lg_t.double().numpy()
    clean = np.where(np.isnan(lg64), -np.inf, lg64)
    star = np.where(np.all(np.isnan(lg64), -1), 0, clean.argmax(-1))
    draft = np.where(rng.random((B, T)) < 0.8, star[:, :T], rng.integers(0, V, (B, T)))
    d = torch.from_numpy(draft.astype(np.int32)).to(DEV)
    for parent in (None, np.stack([W.random_tree(rng, T, 2, 4) for _ in range(B)])):
        for with_nan in (True, False):
            x = lg_t if with_nan else torch.from_numpy(np.where(np.isnan(lg), -np.inf, lg)).to(dtype)
            nk = torch.empty(B, dtype=torch.int32, device=DEV)
            path = torch.empty((B, T), dtype=torch.int32, device=DEV)
            bonus = torch.empty(B, dtype=torch.int32, device=DEV)
            err = torch.zeros(1, dtype=torch.int32, device=DEV)
            ws = torch.empty(gb.spec_accept_workspace_bytes(B, T, V), dtype=torch.uint8,
                             device=DEV)
            par_t = None if parent is None else torch.from_numpy(parent.astype(np.int32)).to(DEV)
            print("accept inf/nan", V, dtype, parent is not None, with_nan, flush=True)
            gb.spec_accept_prefix(d, x.to(DEV), nk, path, bonus, ws, parent=par_t, dev_err=err)
            n_ref, p_ref, b_ref = oracle.accept(draft, x.double().numpy(), parent)
            np.testing.assert_array_equal(nk.cpu().numpy(), n_ref)
            np.testing.assert_array_equal(path.cpu().numpy(), p_ref)
            np.testing.assert_array_equal(bonus.cpu().numpy(), b_ref)
            assert ((bonus.cpu().numpy() >= 0) & (bonus.cpu().numpy() < V)).all()
            assert bool(int(err.item()) & gb.DEV_ERR_NAN) == with_nan
            assert int(err.item()) & ~gb.DEV_ERR_NAN == 0


# ------------------------------------------------ one-launch round rollback -

@pytest.mark.parametrize("K,dtype,tree", [(4, torch.bfloat16, False), (4, torch.float32, True),
                                          (3, torch.bfloat16, True)])
def test_round_rollback_equals_the_two_calls(K, dtype, tree):
    """gdn_round_rollback (one launch at conv width 4, the two calls
    otherwise) leaves S, the conv window and win_idx byte-identical to
    gdn_tape_rollback followed by gdn_conv_state_rollback, for accepted
    lengths 0..T on chains or arbitrary paths; both match the oracle."""
    _need_gpu()
    T, B, L, D = 11, 6, 2, 64
    sh = gb.GdnShape(L, B, 2, 4, D, D, K, True, 1e-6, dtype)
    gen = torch.Generator().manual_seed(31 + K)
    S0 = torch.randn((L, B, 4, D, D), generator=gen) * 0.1
    u = torch.randn((L, B, T, 4, D), generator=gen)
    k = torch.nn.functional.normalize(torch.randn((L, B, T, 2, D), generator=gen), dim=-1)
    g = 0.05 + 0.95 * torch.rand((L, B, T, 4), generator=gen)
    C = sh.C
    cs0 = torch.randn((L, B, K - 1, C), generator=gen).to(dtype)
    x = torch.randn((L, B, T, C), generator=gen).to(dtype)
    nk = torch.tensor([0, 1, 2, 5, T, 7], dtype=torch.int32)
    path = None
    if tree:
        path = torch.full((B, T), -1, dtype=torch.int32)
        for bb in range(B):
            perm = torch.randperm(T, generator=gen)[: int(nk[bb])]
            path[bb, : int(nk[bb])] = perm.to(torch.int32)
    tape = gb.Tape(u.to(DEV), k.to(DEV), g.to(DEV))
    pd = None if path is None else path.to(DEV)
    outs = []
    for combined in (True, False):
        S, cs = S0.to(DEV).clone(), cs0.to(DEV).clone()
        wi = torch.full((B, K - 1), -7, dtype=torch.int32, device=DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        if combined:
            gb.gdn_round_rollback(sh, S, tape, cs, x.to(DEV), nk.to(DEV), path=pd, win_idx=wi,
                                  dev_err=err)
        else:
            gb.gdn_tape_rollback(sh, S, tape, nk.to(DEV), path=pd, dev_err=err)
            gb.gdn_conv_state_rollback(sh, cs, x.to(DEV), nk.to(DEV), path=pd, win_idx=wi,
                                       dev_err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        outs.append((S.cpu(), cs.cpu(), wi.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    osh = oracle.Shape(L=L, B=B, Hk=2, Hv=4, Dk=D, Dv=D, K=K, silu=True, eps=1e-6)
    pnp = None if path is None else path.numpy()
    ref = oracle.tape_rollback(osh, S0.double().numpy(), u.double().numpy(), k.double().numpy(),
                               g.double().numpy(), nk.numpy(), pnp)
    check_units("S", outs[0][0], ref, "state", 1e-5)
    cs_ref, wi_ref = oracle.conv_rollback(osh, W.to_f64(cs0), W.to_f64(x), nk.numpy(), pnp)
    np.testing.assert_array_equal(outs[0][1].double().numpy(), cs_ref)
    np.testing.assert_array_equal(outs[0][2].numpy(), wi_ref)


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("tree", [False, True])
def test_rollback_every_accepted_length(D, tree):
    """gdn_tape_rollback and gdn_round_rollback with sequence b replaying
    n = b steps of a 64-entry tape, for every n in 0..64 (chains, and paths
    in a random order of tape entries): the state equals the oracle's
    tape_rollback per (layer, seq, v-head), the conv window and its indices
    the oracle's conv_rollback exactly."""
    _need_gpu()
    T, B, L = 64, 65, 2
    sh = gb.GdnShape(L, B, 2, 4, D, D, 4, True, 1e-6, torch.bfloat16)
    gen = torch.Generator().manual_seed(400 + D + tree)
    S0 = torch.randn((L, B, 4, D, D), generator=gen) * 0.1
    u = torch.randn((L, B, T, 4, D), generator=gen)
    k = torch.nn.functional.normalize(torch.randn((L, B, T, 2, D), generator=gen), dim=-1)
    g = 0.6 + 0.4 * torch.rand((L, B, T, 4), generator=gen)
    cs0 = torch.randn((L, B, 3, sh.C), generator=gen).to(torch.bfloat16)
    x = torch.randn((L, B, T, sh.C), generator=gen).to(torch.bfloat16)
    nk = torch.arange(B, dtype=torch.int32)
    path = None
    if tree:
        path = torch.full((B, T), -1, dtype=torch.int32)
        for bb in range(B):
            path[bb, :bb] = torch.randperm(T, generator=gen)[:bb].to(torch.int32)
    tape = gb.Tape(u.to(DEV), k.to(DEV), g.to(DEV))
    pd = None if path is None else path.to(DEV)
    osh = oracle.Shape(L=L, B=B, Hk=2, Hv=4, Dk=D, Dv=D, K=4, silu=True, eps=1e-6)
    pnp = None if path is None else path.numpy()
    ref = oracle.tape_rollback(osh, S0.double().numpy(), u.double().numpy(), k.double().numpy(),
                               g.double().numpy(), nk.numpy(), pnp)
    cs_ref, wi_ref = oracle.conv_rollback(osh, W.to_f64(cs0), W.to_f64(x), nk.numpy(), pnp)
    print("rollback every n", D, tree, flush=True)
    S = S0.to(DEV).clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_tape_rollback(sh, S, tape, nk.to(DEV), path=pd, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    check_units("S (tape rollback)", S, ref, "state", 1e-5)
    assert torch.equal(S[:, 0].cpu(), S0[:, 0])  # n = 0: untouched
    S, cs = S0.to(DEV).clone(), cs0.to(DEV).clone()
    wi = torch.full((B, 3), -9, dtype=torch.int32, device=DEV)
    gb.gdn_round_rollback(sh, S, tape, cs, x.to(DEV), nk.to(DEV), path=pd, win_idx=wi,
                          dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    check_units("S (round rollback)", S, ref, "state", 1e-5)
    np.testing.assert_array_equal(cs.cpu().double().numpy(), cs_ref)
    np.testing.assert_array_equal(wi.cpu().numpy(), wi_ref)


@pytest.mark.parametrize("D,B", [(32, 600), (128, 160)])
def test_rollback_layer_walk_ragged(D, B):
    """Short tapes: at this size each workgroup of the state rollback walks
    several layers (at most ~16K workgroups), and L = 7 leaves a shorter last
    group.  Sequences that accepted nothing sit between ones that did; the
    state equals the oracle's tape_rollback per (layer, seq, v-head) and the
    idle sequences' state is untouched, in both rollback calls."""
    _need_gpu()
    T, L, Hk, Hv = 16, 7, 2, 4
    rows = min(256 * 16 // D, D)
    units = L * B * Hv * (D // rows)
    lpw = -(-units // 16384)
    assert 1 < lpw < L and L % lpw != 0  # several layers per workgroup, ragged
    sh = gb.GdnShape(L, B, Hk, Hv, D, D, 4, True, 1e-6, torch.bfloat16)
    gen = torch.Generator().manual_seed(700 + D)
    S0 = torch.randn((L, B, Hv, D, D), generator=gen) * 0.1
    u = torch.randn((L, B, T, Hv, D), generator=gen)
    k = torch.nn.functional.normalize(torch.randn((L, B, T, Hk, D), generator=gen), dim=-1)
    g = 0.6 + 0.4 * torch.rand((L, B, T, Hv), generator=gen)
    nk = torch.randint(0, T + 1, (B,), generator=gen, dtype=torch.int32)
    nk[::3] = 0
    nk[1] = T
    cs0 = torch.randn((L, B, 3, sh.C), generator=gen).to(torch.bfloat16)
    x = torch.randn((L, B, T, sh.C), generator=gen).to(torch.bfloat16)
    tape = gb.Tape(u.to(DEV), k.to(DEV), g.to(DEV))
    osh = oracle.Shape(L=L, B=B, Hk=Hk, Hv=Hv, Dk=D, Dv=D, K=4, silu=True, eps=1e-6)
    ref = oracle.tape_rollback(osh, S0.double().numpy(), u.double().numpy(), k.double().numpy(),
                               g.double().numpy(), nk.numpy(), None)
    idle = (nk == 0).nonzero().flatten()
    print("rollback layer walk", D, B, "lpw", lpw, flush=True)
    S = S0.to(DEV).clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_tape_rollback(sh, S, tape, nk.to(DEV), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    check_units("S (tape rollback, layer walk)", S, ref, "state", 1e-5)
    assert torch.equal(S[:, idle].cpu(), S0[:, idle])
    S, cs = S0.to(DEV).clone(), cs0.to(DEV).clone()
    gb.gdn_round_rollback(sh, S, tape, cs, x.to(DEV), nk.to(DEV), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    check_units("S (round rollback, layer walk)", S, ref, "state", 1e-5)
    assert torch.equal(S[:, idle].cpu(), S0[:, idle])
    cs_ref, _ = oracle.conv_rollback(osh, W.to_f64(cs0), W.to_f64(x), nk.numpy())
    np.testing.assert_array_equal(cs.cpu().double().numpy(), cs_ref)


@pytest.mark.parametrize("entry", ["conv", "round"])
def test_conv_rollback_walk_batches(entry):
    """The conv window rollback with 4,800 bf16 channels (600 16-byte
    chunks per row: one whole batch of two chunks per thread, then a tail of
    88), against the oracle's conv_rollback, exactly.  The standalone call at
    5 layers x 420 sequences walks two layers per workgroup with a shorter
    last group; the round call (state and window in one launch) runs a small
    stack, its state checked too.  Sequences that accepted nothing keep
    their window."""
    _need_gpu()
    D, H, T = 32, 50, 4
    L, B = (5, 420) if entry == "conv" else (2, 8)
    sh = gb.GdnShape(L, B, H, H, D, D, 4, True, 1e-6, torch.bfloat16)
    assert sh.C == 4800
    if entry == "conv":
        lpw = -(-(L * B) // 2048)
        assert lpw == 2 and L % lpw != 0
    gen = torch.Generator().manual_seed(811 + L)
    nk = torch.randint(0, T + 1, (B,), generator=gen, dtype=torch.int32)
    nk[::4] = 0
    nk[1] = T
    cs0 = torch.randn((L, B, 3, sh.C), generator=gen).to(torch.bfloat16)
    x = torch.randn((L, B, T, sh.C), generator=gen).to(torch.bfloat16)
    osh = oracle.Shape(L=L, B=B, Hk=H, Hv=H, Dk=D, Dv=D, K=4, silu=True, eps=1e-6)
    cs_ref, wi_ref = oracle.conv_rollback(osh, W.to_f64(cs0), W.to_f64(x), nk.numpy())
    print("conv rollback walk", entry, L, B, flush=True)
    cs = cs0.to(DEV).clone()
    wi = torch.full((B, 3), -5, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    if entry == "conv":
        gb.gdn_conv_state_rollback(sh, cs, x.to(DEV), nk.to(DEV), win_idx=wi, dev_err=err)
    else:
        S0 = torch.randn((L, B, H, D, D), generator=gen) * 0.1
        u = torch.randn((L, B, T, H, D), generator=gen)
        k = torch.nn.functional.normalize(torch.randn((L, B, T, H, D), generator=gen), dim=-1)
        g = 0.6 + 0.4 * torch.rand((L, B, T, H), generator=gen)
        S = S0.to(DEV).clone()
        gb.gdn_round_rollback(sh, S, gb.Tape(u.to(DEV), k.to(DEV), g.to(DEV)), cs, x.to(DEV),
                              nk.to(DEV), win_idx=wi, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    np.testing.assert_array_equal(cs.cpu().double().numpy(), cs_ref)
    np.testing.assert_array_equal(wi.cpu().numpy(), wi_ref)
    if entry == "round":
        ref = oracle.tape_rollback(osh, S0.double().numpy(), u.double().numpy(),
                                   k.double().numpy(), g.double().numpy(), nk.numpy(), None)
        check_units("S (round rollback)", S, ref, "state", 1e-5)


# ------------------------------------------------------- device-side errors -

def test_dev_err_bad_n_keep_leaves_state():
    _need_gpu()
    cfg = W.CONFIGS[3].with_(L=1, B=2, Hk=2, Hv=4, V=100)
    inp, acc = host_round_inputs(cfg, 0)
    d = {k: v.to(DEV) for k, v in inp.items()}
    rb = make_buffers(cfg, d, {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
                               for k, v in acc.items()})
    spec_round.verify_layer(rb, 0)
    S_before = rb.S.clone()
    cs_before = rb.conv_state.clone()
    rb.n_keep.copy_(torch.tensor([cfg.T + 1, -1], dtype=torch.int32))
    spec_round.rollback(rb)
    torch.cuda.synchronize()
    assert rb.dev_err.item() & gb.DEV_ERR_N_KEEP
    assert torch.equal(rb.S, S_before) and torch.equal(rb.conv_state, cs_before)


def test_dev_err_bad_parent_and_path():
    _need_gpu()
    cfg = W.CONFIGS[5].with_(L=1, B=2, Hk=2, Hv=4, T=8, V=100)
    inp, acc = host_round_inputs(cfg, 0)
    d = {k: v.to(DEV) for k, v in inp.items()}
    par = acc["parent"].clone()
    par[1, 5] = 6  # child before parent
    sh = gb.GdnShape(1, 2, 2, 4, 128, 128, 4, True, cfg.eps, cfg.dtype)
    o = torch.full((1, 2, 8, 4, 128), 7.0, device=DEV)
    tape = gb.Tape.empty(sh, 8, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    gb.gdn_tree_verify(sh, par.to(DEV), d["x"], d["conv_state"], d["conv_w"], d["a"], d["b"],
                       d["S0"], o, tape, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & gb.DEV_ERR_PARENT
    assert torch.all(o[:, 1] == 7.0)          # bad sequence untouched
    assert not torch.all(o[:, 0] == 7.0)      # good sequence written
    err.zero_()
    path = torch.full((2, 8), -1, dtype=torch.int32, device=DEV)
    path[0, 0] = 9
    nk = torch.tensor([1, 0], dtype=torch.int32, device=DEV)
    S0 = d["S0"].clone()
    gb.gdn_tape_rollback(sh, d["S0"], tape, nk, path=path, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & gb.DEV_ERR_PATH
    assert torch.equal(d["S0"], S0)


# ---------------------------------------------------------------- determinism

def test_run_twice_bit_identical():
    _need_gpu()
    cfg = W.CONFIGS[5].with_(L=1, B=2, Hk=2, Hv=4, V=300)
    inp, acc = host_round_inputs(cfg, 4)
    outs = []
    for _ in range(2):
        d = {k: v.to(DEV) for k, v in inp.items()}
        rb = make_buffers(cfg, d, {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
                                   for k, v in acc.items()})
        spec_round.run_round(rb)
        torch.cuda.synchronize()
        outs.append(gpu_outputs(rb))
    for k in ("o", "u", "k", "S_new", "cs_new", "n_keep", "path", "bonus"):
        assert torch.equal(outs[0][k], outs[1][k]), k


# ---------------------------------------- full sizes, sampled (layer, seq) --

@pytest.mark.parametrize("cfg_id", [3, 4, 5])
def test_full_size_sampled(cfg_id):
    _need_gpu()
    cfg = W.CONFIGS[cfg_id]
    torch.cuda.empty_cache()
    inp = W.layer_inputs(cfg, 0, DEV)
    acc = (W.tree_accept_inputs(cfg, 0, DEV) if cfg.is_tree else W.chain_accept_inputs(cfg, 0, DEV))
    ls = [0, cfg.L // 2, cfg.L - 1]
    bs = [0, cfg.B // 3, cfg.B - 1]
    # sampled inputs to host before the round (rollback updates S in place)
    f64 = {}
    for k, v in inp.items():
        t = v[ls]
        if k != "conv_w":
            t = t[:, bs]
        f64[k] = W.to_f64(t)
    rb = make_buffers(cfg, inp, acc)
    spec_round.run_round(rb)
    torch.cuda.synchronize()
    got = gpu_outputs(rb, ls=ls, bs=bs)
    # every sequence's accepted length is the planted one
    np.testing.assert_array_equal(rb.n_keep.cpu().numpy(), acc["n_planted"])
    parent = acc["parent"][bs].cpu().numpy() if cfg.is_tree else None
    ref = oracle_round(cfg, f64, acc["draft"][bs].cpu().numpy(),
                       W.to_f64(acc["logits"][bs]), parent, L=len(ls), B=len(bs))
    compare(got, ref, tree=cfg.is_tree)
    del rb, inp, acc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg_id", [4, 5])
def test_full_size_fused_rounds_sampled(cfg_id):
    """The round form the benchmark times for the B=256 16-draft chain stack
    and the B=64 64-node tree stack, at full size: two fused rounds, the
    second replaying the first's accepted prefixes (paths) inside its
    verify.  Sampled (layer, sequence) units of
    the second round's outputs, tape, accepted lengths, paths and conv
    window, and of the state it leaves (one accepted prefix behind), against
    the oracle's plain rounds."""
    _need_gpu()
    cfg = W.CONFIGS[cfg_id]
    tree = cfg.is_tree
    torch.cuda.empty_cache()
    ls = [0, cfg.L // 2, cfg.L - 1]
    bs = [0, cfg.B // 3, cfg.B - 1]

    def host(inp):
        f = {}
        for k, v in inp.items():
            t = v[ls]
            if k != "conv_w":
                t = t[:, bs]
            f[k] = W.to_f64(t)
        return f

    accs = [W.tree_accept_inputs(cfg, r, DEV) if tree else W.chain_accept_inputs(cfg, r, DEV)
            for r in (0, 1)]
    inp0 = W.layer_inputs(cfg, 0, DEV)
    f0 = host(inp0)
    print("full-size fused rounds", cfg_id, flush=True)
    fr = spec_round.FusedRound(make_buffers(cfg, inp0, accs[0]))
    rb = fr.rb
    fr.round(0, first=True)
    torch.cuda.synchronize()
    inp1 = W.layer_inputs(cfg, 1, DEV)
    f1 = host(inp1)
    del inp1["S0"], inp1["conv_state"]  # the round goes on from the live state and window
    rb.x, rb.a, rb.b, rb.conv_w = inp1["x"], inp1["a"], inp1["b"], inp1["conv_w"]
    rb.logits, rb.draft = accs[1]["logits"], accs[1]["draft"]
    if tree:
        rb.parent = accs[1]["parent"]
    fr.round(1)
    torch.cuda.synchronize()

    def pick(t, has_l=True):
        return (t[ls][:, bs] if has_l else t[bs]).detach().cpu()

    tape = fr.tapes[1]
    got = dict(o=pick(rb.o), u=pick(tape.u), k=pick(tape.k), g=pick(tape.g),
               S=pick(rb.S), cs=pick(rb.conv_state), n_keep=pick(fr.n_keeps[1], False),
               path=pick(fr.paths[1], False), bonus=pick(rb.bonus, False),
               win_idx=pick(rb.win_idx, False))
    np.testing.assert_array_equal(got["n_keep"].numpy(), np.asarray(accs[1]["n_planted"])[bs])
    assert int(rb.dev_err.item()) == 0

    def ref_round(f, acc):
        par = acc["parent"][bs].cpu().numpy() if tree else None
        return oracle_round(cfg, f, acc["draft"][bs].cpu().numpy(), W.to_f64(acc["logits"][bs]),
                            par, L=len(ls), B=len(bs))

    ref0 = ref_round(f0, accs[0])
    f1["S0"], f1["conv_state"] = ref0["S_new"], ref0["cs_new"]
    ref1 = ref_round(f1, accs[1])
    for key in ("n_keep", "bonus", "win_idx"):
        np.testing.assert_array_equal(got[key].numpy(), np.asarray(ref1[key]), err_msg=key)
    if tree:
        np.testing.assert_array_equal(got["path"].numpy(), ref1["path"])
        np.testing.assert_array_equal(rb.conv_win[bs].cpu().numpy(), ref1["conv_win"])
    np.testing.assert_array_equal(got["cs"].double().numpy(), ref1["cs_new"])
    for key in ("o", "u", "k"):
        check_units(key, got[key], ref1[key], "tok")
    np.testing.assert_array_equal(got["g"].double().numpy(), ref1["g"])
    check_units("S after the replay", got["S"], ref0["S_new"], "state")
    del fr, rb, inp0, inp1, accs
    torch.cuda.empty_cache()


# ------------------------------------------------------- sampling accept --

def _sample_inputs(B, T, V, tau, dtype, seed, p_lo=0.05, p_hi=0.95):
    """Logits N(0, 1) with each draft token's logit set so that its
    probability lands near a uniform draw in [p_lo, p_hi] (bf16 rounding
    moves it slightly); seeded uniforms in [0, 1)."""
    rng = np.random.default_rng(seed)
    logits = rng.normal(size=(B, T + 1, V))
    draft = rng.integers(0, V, size=(B, T))
    for b in range(B):
        for j in range(T):
            z = logits[b, j] / tau
            z_others = np.delete(z, draft[b, j])
            lse = z_others.max() + np.log(np.exp(z_others - z_others.max()).sum())
            p = rng.uniform(p_lo, p_hi)
            logits[b, j, draft[b, j]] = (lse + np.log(p / (1 - p))) * tau
    lt = torch.from_numpy(logits).to(dtype)
    uni = torch.from_numpy(rng.uniform(size=(B, T + 1))).float()
    return draft.astype(np.int32), lt, uni


def _run_sample(draft, lt, uni, tau):
    B, T = draft.shape
    V = lt.shape[-1]
    dev = dict(device=DEV, dtype=torch.int32)
    n = torch.empty((B,), **dev)
    path = torch.empty((B, T), **dev)
    tok = torch.empty((B,), **dev)
    err = torch.zeros((1,), **dev)
    ws = torch.empty((gb.spec_sample_workspace_bytes(B, T, V),), device=DEV, dtype=torch.uint8)
    gb.spec_accept_sample(torch.from_numpy(draft).to(DEV), lt.to(DEV), tau, uni.to(DEV), n, path,
                          tok, ws, dev_err=err)
    torch.cuda.synchronize()
    return n.cpu().numpy(), path.cpu().numpy(), tok.cpu().numpy(), int(err.item())


def _check_sample(draft, lt, uni, tau, n_g, path_g, tok_g, margin=1e-5):
    """Exact agreement with the fp64 oracle, except where a uniform lies within
    `margin` of the threshold it is compared with (fp32 vs fp64 statistics):
    there the GPU's choice must still be a valid one.  Returns the number of
    such near-threshold sequences."""
    lg = lt.double().numpy()
    u = uni.double().numpy()
    B, T = draft.shape
    n_o, path_o, tok_o, pd = oracle.accept_sample(draft, lg, tau, u, detail=True)
    near = 0
    for b in range(B):
        if n_g[b] != n_o[b]:
            j = min(n_g[b], n_o[b])
            assert abs(u[b, j] - pd[b, j]) < margin, (b, j, u[b, j], pd[b, j], n_g[b], n_o[b])
            near += 1
            continue
        np.testing.assert_array_equal(path_g[b], path_o[b])
        if tok_g[b] != tok_o[b]:
            n = n_g[b]
            ban = int(draft[b, n]) if n < T and 0 <= draft[b, n] < lg.shape[-1] else -1
            c = oracle.sample_cdf(lg[b, n], tau, ban)
            target, tol, i = u[b, T] * c[-1], margin * c[-1], int(tok_g[b])
            assert i != ban and c[i] > target - tol and (i == 0 or c[i - 1] <= target + tol), \
                (b, i, int(tok_o[b]), target, c[max(i - 1, 0)], c[i])
            near += 1
    return near


@pytest.mark.parametrize("B,T,V,tau,dtype", [
    (3, 4, 7, 1.0, torch.float32), (32, 8, 151936, 1.0, torch.bfloat16),
    (5, 16, 1001, 0.5, torch.bfloat16), (4, 1, 4100, 2.0, torch.float32),
    (2, 64, 9000, 0.8, torch.bfloat16), (6, 5, 151936, 1.3, torch.float32),
    (64, 3, 8192, 1.0, torch.bfloat16)])
def test_sample_accept_matches_oracle(B, T, V, tau, dtype):
    _need_gpu()
    draft, lt, uni = _sample_inputs(B, T, V, tau, dtype, seed=B * 1000 + T * 10 + V % 97)
    n_g, path_g, tok_g, err = _run_sample(draft, lt, uni, tau)
    assert err == 0
    near = _check_sample(draft, lt, uni, tau, n_g, path_g, tok_g)
    assert near <= max(1, B // 50)


def test_sample_accept_extremes_and_bad_tokens():
    """Uniforms of zero keep every draft and draw from the last row; a token
    outside [0, V) is never kept and flags GDN_DEV_ERR_TOKEN; uniforms near
    one reject the first draft and draw high indices."""
    _need_gpu()
    B, T, V, tau = 8, 6, 5000, 1.0
    draft, lt, uni = _sample_inputs(B, T, V, tau, torch.bfloat16, seed=77)
    zero = torch.zeros_like(uni)
    n_g, path_g, tok_g, err = _run_sample(draft, lt, zero, tau)
    assert err == 0 and (n_g == T).all()
    _check_sample(draft, lt, zero, tau, n_g, path_g, tok_g)
    bad = draft.copy()
    bad[:, 3] = V + 5
    bad[1, 3] = -2
    n_g, path_g, tok_g, err = _run_sample(bad, lt, zero, tau)
    assert err & gb.DEV_ERR_TOKEN and (n_g == 3).all()
    _check_sample(bad, lt, zero, tau, n_g, path_g, tok_g)
    high = torch.full_like(uni, 0.999999)
    n_g, path_g, tok_g, err = _run_sample(draft, lt, high, tau)
    assert (n_g == 0).all()
    _check_sample(draft, lt, high, tau, n_g, path_g, tok_g)


# ---------------------------------------------------------------- prefill --

@pytest.mark.parametrize("T,L,B,Hk,Hv,D,K,dtype", [
    (1, 1, 2, 2, 4, 128, 4, torch.bfloat16), (5, 1, 2, 2, 4, 128, 4, torch.bfloat16),
    (16, 2, 2, 2, 4, 128, 4, torch.bfloat16), (17, 1, 3, 2, 4, 128, 4, torch.float32),
    (40, 1, 2, 1, 3, 64, 3, torch.bfloat16), (100, 1, 2, 2, 4, 128, 4, torch.bfloat16),
    (150, 1, 1, 1, 1, 32, 4, torch.float32), (33, 1, 2, 2, 2, 128, 2, torch.bfloat16),
    (48, 2, 3, 2, 4, 128, 3, torch.float32), (64, 1, 2, 1, 2, 128, 8, torch.bfloat16)])
def test_prefill_matches_sequential_oracle(T, L, B, Hk, Hv, D, K, dtype):
    """gdn_prefill (16-token chunks, each chunk's replay folded into the next
    verify; for 128-dim heads all chunks in one launch with the state held
    in registers) equals the oracle's sequential recurrence over all T
    tokens: every output, the final state and the final conv window."""
    _need_gpu()
    cfg = W.CONFIGS[2].with_(L=L, B=B, Hk=Hk, Hv=Hv, Dk=D, Dv=D, K=K, T=T, dtype=dtype)
    inp = W.layer_inputs(cfg, 0, "cpu")
    sh = gshape(cfg)
    d = {k: v.to(DEV) for k, v in inp.items()}
    S, cs = d["S0"].clone(), d["conv_state"].clone()
    o = torch.empty((L, B, T, Hv, D), device=DEV)
    ws = torch.empty((gb.gdn_prefill_workspace_bytes(sh),), device=DEV, dtype=torch.uint8)
    err = torch.zeros((1,), device=DEV, dtype=torch.int32)
    gb.gdn_prefill(sh, d["x"], cs, d["conv_w"], d["a"], d["b"], S, o, ws, dev_err=err)
    torch.cuda.synchronize()
    f = {k: W.to_f64(v) for k, v in inp.items()}
    osh = oracle.Shape(L=L, B=B, Hk=Hk, Hv=Hv, Dk=D, Dv=D, K=K, silu=cfg.silu, eps=cfg.eps)
    ref = oracle.verify_chunk(osh, f["x"], f["conv_state"], f["conv_w"], f["a"], f["b"], f["S0"],
                              want_final=True)
    cs_ref, _ = oracle.conv_rollback(osh, f["conv_state"], f["x"], np.full(B, T, np.int32))
    assert int(err.item()) == 0
    check_units("o", o, ref["o"], "tok")
    check_units("S", S, ref["S_final"], "state")
    np.testing.assert_array_equal(cs.cpu().double().numpy(), cs_ref)


def test_full_size_prefill_sampled():
    """The benchmark's prefill at full size: 512 tokens through the 30-layer,
    B = 32 stack of 8-draft chains (one launch, state in registers), with
    sampled (layer, sequence) units of the outputs, the final state and the
    final conv window against the oracle's sequential recurrence."""
    _need_gpu()
    cfg = W.CONFIGS[3].with_(T=512)
    torch.cuda.empty_cache()
    inp = W.layer_inputs(cfg, 11, DEV)
    ls = [0, cfg.L // 2, cfg.L - 1]
    bs = [0, cfg.B // 3, cfg.B - 1]
    f = {}
    for k, v in inp.items():
        t = v[ls]
        f[k] = W.to_f64(t if k == "conv_w" else t[:, bs])
    sh = gshape(cfg)
    o = torch.empty((cfg.L, cfg.B, cfg.T, cfg.Hv, cfg.Dv), device=DEV)
    ws = torch.empty((gb.gdn_prefill_workspace_bytes(sh),), device=DEV, dtype=torch.uint8)
    err = torch.zeros((1,), device=DEV, dtype=torch.int32)
    S, cs = inp["S0"], inp["conv_state"]
    print("full-size prefill", cfg.L, cfg.B, cfg.T, flush=True)
    gb.gdn_prefill(sh, inp["x"], cs, inp["conv_w"], inp["a"], inp["b"], S, o, ws, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got_o = o[ls][:, bs].cpu().double().numpy()
    got_S = S[ls][:, bs].cpu().double().numpy()
    got_cs = cs[ls][:, bs].cpu().double().numpy()
    del inp, o, ws, S, cs
    torch.cuda.empty_cache()
    osh = oracle.Shape(L=len(ls), B=len(bs), Hk=cfg.Hk, Hv=cfg.Hv, Dk=cfg.Dk, Dv=cfg.Dv, K=cfg.K,
                       silu=cfg.silu, eps=cfg.eps)
    ref = oracle.verify_chunk(osh, f["x"], f["conv_state"], f["conv_w"], f["a"], f["b"], f["S0"],
                              want_final=True)
    cs_ref, _ = oracle.conv_rollback(osh, f["conv_state"], f["x"],
                                     np.full(len(bs), cfg.T, np.int32))
    check_units("o", got_o, ref["o"], "tok")
    check_units("S", got_S, ref["S_final"], "state")
    np.testing.assert_array_equal(got_cs, cs_ref)


# ------------------------------------------------ per-key-channel decay gate --

def _vg_inputs(cfg, seed, gate_lo=0.05):
    """Workload inputs with the decay gate drawn per key channel, U(gate_lo, 1),
    rounded to the input dtype."""
    inp = W.layer_inputs(cfg, seed, "cpu")
    gen = torch.Generator().manual_seed(1000 + seed)
    a = gate_lo + (1 - gate_lo) * torch.rand((cfg.L, cfg.B, cfg.T, cfg.Hv, cfg.Dk), generator=gen)
    inp["a"] = a.to(cfg.dtype)
    return inp


def _vg_shapes(cfg):
    g = gb.GdnShape(cfg.L, cfg.B, cfg.Hk, cfg.Hv, cfg.Dk, cfg.Dv, cfg.K, cfg.silu, cfg.eps,
                    cfg.dtype, gate_per_key=True)
    o = oracle.Shape(L=cfg.L, B=cfg.B, Hk=cfg.Hk, Hv=cfg.Hv, Dk=cfg.Dk, Dv=cfg.Dv, K=cfg.K,
                     silu=cfg.silu, eps=cfg.eps)
    return g, o


@pytest.mark.parametrize("cfg_id", [4, 5])
def test_full_size_vgate_fused_rounds_sampled(cfg_id):
    """The per-key round form the benchmark picks for the B=256 16-draft chain
    stack and the B=64 64-node tree stack (fused), at full size, with the
    decay gate drawn per key channel: two
    rounds, the second replaying the first's accepted prefixes (paths) inside
    its verify.  Sampled (layer, sequence) units of the second round's outputs,
    tape, accepted lengths, paths and conv window, and of the state it leaves
    (one accepted prefix behind), against the oracle's per-key plain rounds."""
    _need_gpu()
    cfg = W.CONFIGS[cfg_id]
    tree = cfg.is_tree
    torch.cuda.empty_cache()
    ls = [0, cfg.L // 2, cfg.L - 1]
    bs = [0, cfg.B // 3, cfg.B - 1]
    gsh, _ = _vg_shapes(cfg)
    osh = oracle.Shape(L=len(ls), B=len(bs), Hk=cfg.Hk, Hv=cfg.Hv, Dk=cfg.Dk, Dv=cfg.Dv,
                       K=cfg.K, silu=cfg.silu, eps=cfg.eps)

    def inputs(r):
        inp = W.layer_inputs(cfg, r, DEV)
        gen = torch.Generator(device=DEV).manual_seed(5000 + r)
        a = torch.empty(gsh.gate_shape(cfg.T), device=DEV, dtype=cfg.dtype)
        for l in range(cfg.L):
            a[l] = 0.05 + 0.95 * torch.rand(a.shape[1:], device=DEV, generator=gen)
        inp["a"] = a
        host = {}
        for k, v in inp.items():
            t = v[ls]
            host[k] = W.to_f64(t if k == "conv_w" else t[:, bs])
        return inp, host

    accs = [W.tree_accept_inputs(cfg, r, DEV) if tree else W.chain_accept_inputs(cfg, r, DEV)
            for r in (0, 1)]
    inp0, f0 = inputs(0)
    print("full-size per-key fused rounds", cfg_id, flush=True)
    rb = spec_round.RoundBuffers(sh=gsh, T=cfg.T, V=cfg.V, tree=tree, S=inp0["S0"],
                                 conv_state=inp0["conv_state"], conv_w=inp0["conv_w"],
                                 x=inp0["x"], a=inp0["a"], b=inp0["b"],
                                 logits=accs[0]["logits"], draft=accs[0]["draft"],
                                 parent=accs[0]["parent"] if tree else None)
    fr = spec_round.FusedRound(rb)
    fr.round(0, first=True)
    torch.cuda.synchronize()
    inp1, f1 = inputs(1)
    rb.x, rb.a, rb.b, rb.conv_w = inp1["x"], inp1["a"], inp1["b"], inp1["conv_w"]
    rb.logits, rb.draft = accs[1]["logits"], accs[1]["draft"]
    if tree:
        rb.parent = accs[1]["parent"]
    fr.round(1)
    torch.cuda.synchronize()
    assert int(rb.dev_err.item()) == 0

    def pick(t, has_l=True):
        return (t[ls][:, bs] if has_l else t[bs]).detach().cpu()

    tape = fr.tapes[1]
    got = dict(o=pick(rb.o), u=pick(tape.u), k=pick(tape.k), g=pick(tape.g), S=pick(rb.S),
               cs=pick(rb.conv_state), n_keep=pick(fr.n_keeps[1], False),
               path=pick(fr.paths[1], False))

    def ref_round(f, S, cs, acc):
        par = acc["parent"][bs].cpu().numpy() if tree else None
        if tree:
            ref = oracle.tree_verify_vg(osh, par, f["x"], cs, f["conv_w"], f["a"], f["b"], S)
        else:
            ref = oracle.verify_chunk_vg(osh, f["x"], cs, f["conv_w"], f["a"], f["b"], S)
        n, path, _ = oracle.accept(acc["draft"][bs].cpu().numpy(), W.to_f64(acc["logits"][bs]),
                                   par)
        S_new = oracle.tape_rollback_vg(osh, S, ref["u"], ref["k"], ref["g"], n,
                                        path if tree else None)
        cs_new, _ = oracle.conv_rollback(osh, cs, f["x"], n, path if tree else None)
        return ref, n, path, S_new, cs_new

    _, _, _, S1, cs1 = ref_round(f0, f0["S0"], f0["conv_state"], accs[0])
    ref, n, path, _, cs2 = ref_round(f1, S1, cs1, accs[1])
    np.testing.assert_array_equal(got["n_keep"].numpy(), n)
    if tree:
        np.testing.assert_array_equal(got["path"].numpy(), path)
    np.testing.assert_array_equal(got["cs"].double().numpy(), cs2)
    for key in ("o", "u", "k"):
        check_units(key, got[key], ref[key], "tok")
    np.testing.assert_array_equal(got["g"].double().numpy(), ref["g"])
    check_units("S after the replay", got["S"], S1, "state")
    del fr, rb, inp0, inp1, accs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,L,B,Hk,Hv,D,K,dtype", [
    (1, 1, 2, 2, 4, 128, 4, torch.bfloat16), (8, 2, 2, 2, 4, 128, 4, torch.bfloat16),
    (16, 1, 3, 1, 2, 64, 3, torch.float32), (17, 1, 2, 2, 4, 128, 4, torch.bfloat16),
    (64, 1, 1, 1, 3, 32, 6, torch.float32), (40, 1, 2, 4, 4, 64, 4, torch.bfloat16),
    (16, 2, 3, 2, 4, 128, 4, torch.bfloat16), (12, 1, 2, 2, 2, 128, 3, torch.bfloat16),
    (5, 1, 3, 1, 2, 128, 8, torch.bfloat16), (16, 1, 2, 1, 1, 128, 2, torch.bfloat16)])
def test_vgate_verify_matches_oracle(T, L, B, Hk, Hv, D, K, dtype):
    """gdn_verify_chunk with a per-key-channel gate equals the oracle's
    verify_chunk_vg (outputs and tape) and leaves S untouched: bf16 chains of
    <= 16 tokens with 128-dim heads on the MFMA chain kernel (conv widths 2,
    3, 4, 8), the rest on the sequential kernel."""
    _need_gpu()
    cfg = W.CONFIGS[2].with_(L=L, B=B, Hk=Hk, Hv=Hv, Dk=D, Dv=D, K=K, T=T, dtype=dtype)
    inp = _vg_inputs(cfg, 3)
    gsh, osh = _vg_shapes(cfg)
    d = {k: v.to(DEV) for k, v in inp.items()}
    S0 = d["S0"].clone()
    o = torch.empty((L, B, T, Hv, D), device=DEV)
    tape = gb.Tape.empty(gsh, T, DEV)
    gb.gdn_verify_chunk(gsh, d["x"], d["conv_state"], d["conv_w"], d["a"], d["b"], d["S0"], o, tape)
    torch.cuda.synchronize()
    f = {k: W.to_f64(v) for k, v in inp.items()}
    ref = oracle.verify_chunk_vg(osh, f["x"], f["conv_state"], f["conv_w"], f["a"], f["b"], f["S0"])
    for name, got in (("o", o), ("u", tape.u), ("k", tape.k)):
        check_units(name, got, ref[name], "tok")
    np.testing.assert_array_equal(tape.g.cpu().double().numpy(), ref["g"])
    assert torch.equal(d["S0"], S0)


@pytest.mark.parametrize("D,with_path", [(128, False), (64, True), (32, False)])
def test_vgate_rollback_matches_oracle(D, with_path):
    """gdn_tape_rollback with the per-key decay tape equals the oracle's
    tape_rollback_vg for accepted lengths 0..T, chains or arbitrary paths."""
    _need_gpu()
    T, B = 12, 5
    cfg = W.CONFIGS[2].with_(L=2, B=B, Hk=2, Hv=4, Dk=D, Dv=D, T=T, dtype=torch.bfloat16)
    gsh, osh = _vg_shapes(cfg)
    gen = torch.Generator().manual_seed(21)
    S0 = torch.randn((cfg.L, B, cfg.Hv, D, D), generator=gen) * 0.1
    u = torch.randn((cfg.L, B, T, cfg.Hv, D), generator=gen)
    k = torch.nn.functional.normalize(torch.randn((cfg.L, B, T, cfg.Hk, D), generator=gen), dim=-1)
    g = 0.05 + 0.95 * torch.rand((cfg.L, B, T, cfg.Hv, D), generator=gen)
    nk = torch.tensor([0, 1, 5, T, 7], dtype=torch.int32)
    path = None
    if with_path:
        path = torch.full((B, T), -1, dtype=torch.int32)
        for bb in range(B):
            perm = torch.randperm(T, generator=gen)[: int(nk[bb])]
            path[bb, : int(nk[bb])] = perm.to(torch.int32)
    S = S0.to(DEV).clone()
    gb.gdn_tape_rollback(gsh, S, gb.Tape(u.to(DEV), k.to(DEV), g.to(DEV)), nk.to(DEV),
                         path=None if path is None else path.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.tape_rollback_vg(osh, S0.double().numpy(), u.double().numpy(),
                                  k.double().numpy(), g.double().numpy(), nk.numpy(),
                                  None if path is None else path.numpy())
    check_units("S", S, ref, "state", 1e-5)
    assert torch.equal(S[:, 0].cpu(), S0[:, 0])  # n = 0: untouched


@pytest.mark.parametrize("tree", [False, True])
def test_vgate_chained_rounds(tree):
    """Plain rounds (verify, greedy accept, per-key rollback, conv rollback)
    with a per-key-channel gate, four rounds chained, against the oracle:
    8-token chains, and 64-node trees on the MFMA tree kernel."""
    _need_gpu()
    cfg = (W.CONFIGS[5].with_(L=2, B=3, T=64, V=257) if tree
           else W.CONFIGS[3].with_(L=2, B=4, T=8, V=257))
    gsh, osh = _vg_shapes(cfg)
    inp0 = _vg_inputs(cfg, 0)
    oS, ocs = W.to_f64(inp0["S0"]), W.to_f64(inp0["conv_state"])
    rb = None
    for r in range(4):
        inp = _vg_inputs(cfg, r)
        acc = (W.tree_accept_inputs(cfg, r, "cpu") if tree
               else W.chain_accept_inputs(cfg, r, "cpu"))
        d = {k: v.to(DEV) for k, v in inp.items()}
        par = acc["parent"].to(DEV) if tree else None
        if rb is None:
            rb = spec_round.RoundBuffers(sh=gsh, T=cfg.T, V=cfg.V, tree=tree,
                                         S=inp0["S0"].to(DEV), conv_state=inp0["conv_state"].to(DEV),
                                         conv_w=d["conv_w"], x=d["x"], a=d["a"], b=d["b"],
                                         logits=acc["logits"].to(DEV), draft=acc["draft"].to(DEV),
                                         parent=par)
        else:
            rb.x, rb.a, rb.b, rb.conv_w = d["x"], d["a"], d["b"], d["conv_w"]
            rb.logits, rb.draft = acc["logits"].to(DEV), acc["draft"].to(DEV)
            if tree:
                rb.parent = par
        spec_round.run_round(rb)
        torch.cuda.synchronize()
        f = {k: W.to_f64(v) for k, v in inp.items()}
        parent = acc["parent"].numpy() if tree else None
        if tree:
            ref = oracle.tree_verify_vg(osh, parent, f["x"], ocs, f["conv_w"], f["a"], f["b"], oS)
        else:
            ref = oracle.verify_chunk_vg(osh, f["x"], ocs, f["conv_w"], f["a"], f["b"], oS)
        n, path, bonus = oracle.accept(acc["draft"].numpy(), W.to_f64(acc["logits"]), parent)
        np.testing.assert_array_equal(rb.n_keep.cpu().numpy(), n)
        np.testing.assert_array_equal(rb.bonus.cpu().numpy(), bonus)
        check_units("o", rb.o, ref["o"], "tok")
        if tree:
            np.testing.assert_array_equal(rb.path.cpu().numpy(), path)
        oS = oracle.tape_rollback_vg(osh, oS, ref["u"], ref["k"], ref["g"], n,
                                     path if tree else None)
        ocs, _ = oracle.conv_rollback(osh, ocs, f["x"], n, path if tree else None)
        check_units("S", rb.S, oS, "state")
        np.testing.assert_array_equal(rb.conv_state.cpu().double().numpy(), ocs)
    assert int(rb.dev_err.item()) == 0


@pytest.mark.parametrize("T,D,dtype,L,B,Hk,Hv,K", [
    (5, 128, torch.bfloat16, 1, 2, 2, 4, 4), (70, 64, torch.float32, 1, 2, 2, 4, 4),
    (130, 128, torch.bfloat16, 1, 2, 2, 4, 4), (33, 128, torch.bfloat16, 2, 3, 2, 2, 3),
    (48, 128, torch.float32, 1, 2, 1, 2, 4), (16, 128, torch.bfloat16, 1, 2, 1, 2, 2),
    (1, 128, torch.bfloat16, 1, 2, 2, 4, 4), (17, 128, torch.bfloat16, 2, 2, 2, 4, 8)])
def test_vgate_prefill_matches_oracle(T, D, dtype, L, B, Hk, Hv, K):
    """gdn_prefill with a per-key-channel gate equals the oracle's
    verify_chunk_vg over all T tokens: outputs, final state, final conv
    window.  bf16 inputs with 128-dim heads run the chain kernel's one-launch
    chunk loop (a two-tape workspace); other shapes one launch of the
    sequential kernel (no workspace)."""
    _need_gpu()
    cfg = W.CONFIGS[2].with_(L=L, B=B, Hk=Hk, Hv=Hv, Dk=D, Dv=D, K=K, T=T, dtype=dtype)
    inp = _vg_inputs(cfg, 5)
    gsh, osh = _vg_shapes(cfg)
    d = {k: v.to(DEV) for k, v in inp.items()}
    S, cs = d["S0"].clone(), d["conv_state"].clone()
    o = torch.empty((L, B, T, cfg.Hv, D), device=DEV)
    need = gb.gdn_prefill_workspace_bytes(gsh)
    assert (need > 0) == (D == 128 and dtype == torch.bfloat16)
    ws = torch.empty((need,), device=DEV, dtype=torch.uint8) if need else None
    err = torch.zeros((1,), device=DEV, dtype=torch.int32)
    gb.gdn_prefill(gsh, d["x"], cs, d["conv_w"], d["a"], d["b"], S, o, ws, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    f = {k: W.to_f64(v) for k, v in inp.items()}
    ref = oracle.verify_chunk_vg(osh, f["x"], f["conv_state"], f["conv_w"], f["a"], f["b"], f["S0"])
    cs_ref, _ = oracle.conv_rollback(osh, f["conv_state"], f["x"], np.full(B, T, np.int32))
    check_units("o", o, ref["o"], "tok")
    check_units("S", S, ref["S_final"], "state")
    np.testing.assert_array_equal(cs.cpu().double().numpy(), cs_ref)


# ------------------------------- per-key gate over trees, and fused replay --

def _vg_parents(rng, B, T, depth):
    """Random draft trees, or chains given as parent arrays when depth >= T."""
    if depth >= T:
        return np.tile(np.arange(-1, T - 1, dtype=np.int32), (B, 1))
    return np.stack([W.random_tree(rng, T, 4, depth) for _ in range(B)]).astype(np.int32)


@pytest.mark.parametrize("T,L,B,Hk,Hv,D,K,dtype,depth", [
    (64, 1, 2, 2, 4, 128, 4, torch.bfloat16, 8), (40, 2, 2, 1, 2, 64, 3, torch.float32, 6),
    (17, 1, 3, 2, 2, 32, 8, torch.bfloat16, 5), (1, 1, 2, 2, 4, 128, 4, torch.bfloat16, 1),
    (64, 1, 1, 1, 2, 128, 4, torch.float32, 64), (33, 1, 2, 2, 4, 64, 2, torch.bfloat16, 33),
    (48, 2, 2, 2, 2, 128, 3, torch.bfloat16, 6), (64, 1, 1, 1, 2, 128, 4, torch.bfloat16, 64),
    (40, 1, 2, 2, 4, 128, 4, torch.bfloat16, 20), (33, 1, 3, 1, 1, 128, 8, torch.bfloat16, 8),
    (13, 1, 2, 2, 4, 128, 4, torch.bfloat16, 6), (24, 1, 2, 1, 2, 128, 4, torch.bfloat16, 24),
    (12, 1, 2, 2, 4, 128, 4, torch.bfloat16, 8)])
def test_vgate_tree_verify_matches_oracle(T, L, B, Hk, Hv, D, K, dtype, depth):
    """gdn_tree_verify with a per-key-channel gate equals the oracle's
    tree_verify_vg (outputs, tape, conv windows) and leaves S untouched; the
    depth >= T cases are chains given as parent arrays (the deepest trees).
    bf16 trees of 13..64 nodes with 128-dim heads run the MFMA tree kernel
    (conv widths 3, 4 and 8; depths up to 64), the rest the closed-form
    per-key kernel."""
    _need_gpu()
    cfg = W.CONFIGS[2].with_(L=L, B=B, Hk=Hk, Hv=Hv, Dk=D, Dv=D, K=K, T=T, dtype=dtype)
    inp = _vg_inputs(cfg, 5)
    gsh, osh = _vg_shapes(cfg)
    parent = _vg_parents(np.random.default_rng(T + D), B, T, depth)
    d = {k: v.to(DEV) for k, v in inp.items()}
    S0 = d["S0"].clone()
    o = torch.empty((L, B, T, Hv, D), device=DEV)
    tape = gb.Tape.empty(gsh, T, DEV)
    win = torch.full((B, T, K), -99, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("vgate tree", T, D, K, dtype, depth, flush=True)
    gb.gdn_tree_verify(gsh, torch.from_numpy(parent).to(DEV), d["x"], d["conv_state"],
                       d["conv_w"], d["a"], d["b"], d["S0"], o, tape, conv_win=win, dev_err=err)
    torch.cuda.synchronize()
    f = {k: W.to_f64(v) for k, v in inp.items()}
    ref = oracle.tree_verify_vg(osh, parent, f["x"], f["conv_state"], f["conv_w"], f["a"], f["b"],
                                f["S0"])
    for name, got in (("o", o), ("u", tape.u), ("k", tape.k)):
        check_units(name, got, ref[name], "tok")
    np.testing.assert_array_equal(tape.g.cpu().double().numpy(), ref["g"])
    np.testing.assert_array_equal(win.cpu().numpy(), ref["conv_win"])
    assert int(err.item()) == 0
    assert torch.equal(d["S0"], S0)


def _vg_prev_tape(cfg, pT, seed):
    """A synthetic previous tape: u ~ N(0,1), unit k, per-key gates U(0.05, 1)."""
    gen = torch.Generator().manual_seed(seed)
    u = torch.randn((cfg.L, cfg.B, pT, cfg.Hv, cfg.Dv), generator=gen)
    k = torch.nn.functional.normalize(torch.randn((cfg.L, cfg.B, pT, cfg.Hk, cfg.Dk),
                                                  generator=gen), dim=-1)
    g = 0.05 + 0.95 * torch.rand((cfg.L, cfg.B, pT, cfg.Hv, cfg.Dk), generator=gen)
    return u, k, g


@pytest.mark.parametrize("tree,T,pT,D,dtype", [
    (False, 8, 8, 128, torch.bfloat16), (False, 16, 12, 64, torch.float32),
    (False, 16, 16, 128, torch.bfloat16), (False, 5, 13, 128, torch.bfloat16),
    (False, 40, 64, 32, torch.bfloat16), (True, 64, 64, 128, torch.bfloat16),
    (True, 40, 23, 128, torch.bfloat16), (True, 33, 5, 128, torch.bfloat16),
    (True, 24, 40, 32, torch.float32), (True, 16, 9, 128, torch.bfloat16),
    (True, 13, 64, 128, torch.bfloat16), (True, 12, 12, 128, torch.bfloat16)])
def test_vgate_replay_verify_equals_rollback_then_verify(tree, T, pT, D, dtype):
    """gdn_verify_chunk_replay / gdn_tree_verify_replay with a per-key gate:
    the state afterwards is the oracle's tape_rollback_vg of the previous tape
    over the accepted prefix (or path), and the outputs are the oracle's
    verify from that state.  Accepted lengths 0, 1, middle and all."""
    _need_gpu()
    L, B = 2, 4
    cfg = W.CONFIGS[2].with_(L=L, B=B, Hk=2, Hv=4, Dk=D, Dv=D, K=4, T=T, dtype=dtype)
    gsh, osh = _vg_shapes(cfg)
    inp = _vg_inputs(cfg, 7)
    pu, pk, pg = _vg_prev_tape(cfg, pT, 40 + T)
    nk = torch.tensor([0, 1, pT // 2, pT], dtype=torch.int32)
    gen = torch.Generator().manual_seed(9)
    path = None
    if tree:
        path = torch.full((B, pT), -1, dtype=torch.int32)
        for bb in range(B):
            path[bb, :int(nk[bb])] = torch.randperm(pT, generator=gen)[:int(nk[bb])].to(torch.int32)
    d = {k: v.to(DEV) for k, v in inp.items()}
    S = d["S0"].clone()
    o = torch.empty((L, B, T, cfg.Hv, D), device=DEV)
    tape = gb.Tape.empty(gsh, T, DEV)
    ptape = gb.Tape(pu.to(DEV), pk.to(DEV), pg.to(DEV))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    print("vgate replay", tree, T, pT, D, dtype, flush=True)
    f = {k: W.to_f64(v) for k, v in inp.items()}
    S_rep = oracle.tape_rollback_vg(osh, f["S0"], pu.double().numpy(), pk.double().numpy(),
                                    pg.double().numpy(), nk.numpy(),
                                    None if path is None else path.numpy())
    if tree:
        parent = _vg_parents(np.random.default_rng(T), B, T, 6)
        win = torch.empty((B, T, cfg.K), dtype=torch.int32, device=DEV)
        gb.gdn_tree_verify_replay(gsh, torch.from_numpy(parent).to(DEV), d["x"], d["conv_state"],
                                  d["conv_w"], d["a"], d["b"], S, o, tape, ptape, nk.to(DEV),
                                  prev_path=path.to(DEV), conv_win=win, dev_err=err)
        ref = oracle.tree_verify_vg(osh, parent, f["x"], f["conv_state"], f["conv_w"], f["a"],
                                    f["b"], S_rep)
    else:
        gb.gdn_verify_chunk_replay(gsh, d["x"], d["conv_state"], d["conv_w"], d["a"], d["b"], S,
                                   o, tape, ptape, nk.to(DEV), dev_err=err)
        ref = oracle.verify_chunk_vg(osh, f["x"], f["conv_state"], f["conv_w"], f["a"], f["b"],
                                     S_rep)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    check_units("S", S, S_rep, "state", 1e-5)
    assert torch.equal(S[:, 0].cpu(), inp["S0"][:, 0])  # n = 0: untouched
    for name, got in (("o", o), ("u", tape.u), ("k", tape.k)):
        check_units(name, got, ref[name], "tok")
    np.testing.assert_array_equal(tape.g.cpu().double().numpy(), ref["g"])


@pytest.mark.parametrize("T,pT,D", [(24, 8, 64), (40, 8, 128)])
def test_vgate_tree_replay_bad_inputs_flag(T, pT, D):
    """Per-key tree replay (the closed-form kernel, and the MFMA tree kernel
    for 13..64 nodes): a malformed parent array flags GDN_DEV_ERR_PARENT,
    skips that sequence's outputs and still applies its replay; an
    out-of-range accepted length or path entry flags its bit and leaves that
    sequence's state as it was."""
    _need_gpu()
    cfg = W.CONFIGS[2].with_(L=1, B=2, Hk=2, Hv=4, Dk=D, Dv=D, K=4, T=T, dtype=torch.bfloat16)
    gsh, osh = _vg_shapes(cfg)
    inp = _vg_inputs(cfg, 11)
    d = {k: v.to(DEV) for k, v in inp.items()}
    pu, pk, pg = _vg_prev_tape(cfg, pT, 77)
    ptape = gb.Tape(pu.to(DEV), pk.to(DEV), pg.to(DEV))
    parent = _vg_parents(np.random.default_rng(3), 2, T, 5)
    good_path = torch.tensor([[2, 0, 5, -1, -1, -1, -1, -1], [1, 3, -1, -1, -1, -1, -1, -1]],
                             dtype=torch.int32)
    nk = torch.tensor([3, 2], dtype=torch.int32)
    S_rep = oracle.tape_rollback_vg(osh, W.to_f64(inp["S0"]), pu.double().numpy(),
                                    pk.double().numpy(), pg.double().numpy(), nk.numpy(),
                                    good_path.numpy())

    def run(par, n, path):
        S = d["S0"].clone()
        o = torch.full((1, 2, T, cfg.Hv, D), 7.0, device=DEV)
        tape = gb.Tape.empty(gsh, T, DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        gb.gdn_tree_verify_replay(gsh, torch.from_numpy(par).to(DEV), d["x"], d["conv_state"],
                                  d["conv_w"], d["a"], d["b"], S, o, tape, ptape, n.to(DEV),
                                  prev_path=path.to(DEV), dev_err=err)
        torch.cuda.synchronize()
        return S.cpu(), o.cpu(), int(err.item())

    print("vgate bad parent", flush=True)
    bad_par = parent.copy()
    bad_par[1, 5] = 6  # child before parent
    S, o, err = run(bad_par, nk, good_path)
    assert err & gb.DEV_ERR_PARENT
    assert torch.all(o[:, 1] == 7.0)
    check_units("S", S, S_rep, "state", 1e-5)  # replay applied to both sequences
    print("vgate bad n_keep", flush=True)
    S, o, err = run(parent, torch.tensor([pT + 1, 2], dtype=torch.int32), good_path)
    assert err & gb.DEV_ERR_N_KEEP
    assert torch.equal(S[:, 0], inp["S0"][:, 0])
    check_units("S", S[:, 1], S_rep[:, 1], "state", 1e-5)
    print("vgate bad path", flush=True)
    bad_path = good_path.clone()
    bad_path[0, 1] = pT
    S, o, err = run(parent, nk, bad_path)
    assert err & gb.DEV_ERR_PATH
    assert torch.equal(S[:, 0], inp["S0"][:, 0])
    check_units("S", S[:, 1], S_rep[:, 1], "state", 1e-5)


@pytest.mark.parametrize("tree,T", [(True, 64), (True, 40), (True, 24), (True, 12), (False, 8),
                                    (False, 16)])
def test_vgate_fused_rounds(tree, T):
    """Fused rounds (spec_round.FusedRound) with a per-key-channel gate: every
    round's outputs, tape, accepted lengths and paths, conv window, and the
    state after finish(), against the oracle's plain per-key rounds."""
    _need_gpu()
    cfg = (W.CONFIGS[5] if tree else W.CONFIGS[3]).with_(L=2, B=3, T=T, V=293)
    gsh, osh = _vg_shapes(cfg)
    inp0 = _vg_inputs(cfg, 0)
    oS, ocs = W.to_f64(inp0["S0"]), W.to_f64(inp0["conv_state"])
    fr = None
    print("vgate fused rounds", tree, T, flush=True)
    for r in range(4):
        inp = _vg_inputs(cfg, r)
        acc = (W.tree_accept_inputs(cfg, r, "cpu") if tree
               else W.chain_accept_inputs(cfg, r, "cpu"))
        d = {k: v.to(DEV) for k, v in inp.items()}
        par = acc["parent"].to(DEV) if tree else None
        if fr is None:
            rb = spec_round.RoundBuffers(sh=gsh, T=T, V=cfg.V, tree=tree, S=inp0["S0"].to(DEV),
                                         conv_state=inp0["conv_state"].to(DEV),
                                         conv_w=d["conv_w"], x=d["x"], a=d["a"], b=d["b"],
                                         logits=acc["logits"].to(DEV),
                                         draft=acc["draft"].to(DEV), parent=par)
            fr = spec_round.FusedRound(rb)
        else:
            rb = fr.rb
            rb.x, rb.a, rb.b, rb.conv_w = d["x"], d["a"], d["b"], d["conv_w"]
            rb.logits, rb.draft = acc["logits"].to(DEV), acc["draft"].to(DEV)
            if tree:
                rb.parent = par
        fr.round(r, first=(r == 0))
        torch.cuda.synchronize()
        f = {k: W.to_f64(v) for k, v in inp.items()}
        parent = acc["parent"].numpy() if tree else None
        if tree:
            ref = oracle.tree_verify_vg(osh, parent, f["x"], ocs, f["conv_w"], f["a"], f["b"], oS)
        else:
            ref = oracle.verify_chunk_vg(osh, f["x"], ocs, f["conv_w"], f["a"], f["b"], oS)
        n, path, bonus = oracle.accept(acc["draft"].numpy(), W.to_f64(acc["logits"]), parent)
        np.testing.assert_array_equal(fr.n_keeps[r % 2].cpu().numpy(), n)
        np.testing.assert_array_equal(rb.bonus.cpu().numpy(), bonus)
        if tree:
            np.testing.assert_array_equal(fr.paths[r % 2].cpu().numpy(), path)
            np.testing.assert_array_equal(rb.conv_win.cpu().numpy(), ref["conv_win"])
        tape = fr.tapes[r % 2]
        for name, got, want in (("o", rb.o, ref["o"]), ("u", tape.u, ref["u"]),
                                ("k", tape.k, ref["k"])):
            check_units("%s, round %d" % (name, r), got, want, "tok")
        np.testing.assert_array_equal(tape.g.cpu().double().numpy(), ref["g"])
        oS = oracle.tape_rollback_vg(osh, oS, ref["u"], ref["k"], ref["g"], n,
                                     path if tree else None)
        ocs, _ = oracle.conv_rollback(osh, ocs, f["x"], n, path if tree else None)
        np.testing.assert_array_equal(rb.conv_state.cpu().double().numpy(), ocs)
    fr.finish(3)
    torch.cuda.synchronize()
    check_units("S", fr.rb.S, oS, "state")
    assert int(fr.rb.dev_err.item()) == 0
