"""Rounds captured into HIP graphs and replayed, the way bench.py times them,
give bit-identical results to the same C-ABI calls made eagerly, replay
after replay, with other eager work and synchronisation between the
replays: plain and fused rounds, chains and trees."""
import pytest
import torch

from speculative_decode_verify_gdn_amd import binding as gb
from speculative_decode_verify_gdn_amd import spec_round as sr
from speculative_decode_verify_gdn_amd import workload as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.lib()


def _buffers(cfg, rnd):
    """Round buffers on fresh device copies of one seeded input draw."""
    inp = W.layer_inputs(cfg, rnd, "cpu")
    acc = (W.tree_accept_inputs(cfg, rnd, "cpu") if cfg.is_tree
           else W.chain_accept_inputs(cfg, rnd, "cpu"))
    d = {k: v.to(DEV) for k, v in inp.items()}
    sh = gb.GdnShape(cfg.L, cfg.B, cfg.Hk, cfg.Hv, cfg.Dk, cfg.Dv, cfg.K, cfg.silu, cfg.eps,
                     cfg.dtype)
    return sr.RoundBuffers(sh=sh, T=cfg.T, V=cfg.V, tree=cfg.is_tree, S=d["S0"],
                           conv_state=d["conv_state"], conv_w=d["conv_w"], x=d["x"], a=d["a"],
                           b=d["b"], logits=acc["logits"].to(DEV), draft=acc["draft"].to(DEV),
                           parent=acc["parent"].to(DEV) if cfg.is_tree else None)


def _state(rb, extra=()):
    out = {"S": rb.S, "conv_state": rb.conv_state, "o": rb.o, "bonus": rb.bonus,
           "win_idx": rb.win_idx, "dev_err": rb.dev_err}
    if rb.tree:
        out["conv_win"] = rb.conv_win
    out.update(dict(extra))
    return {k: v.clone() for k, v in out.items()}


def _same(got, want, where):
    for name in want:
        assert torch.equal(got[name], want[name]), (where, name)
    assert int(want["dev_err"].item()) == 0, where


def _eager_work(stream):
    """Unrelated eager work on the launch stream between replays."""
    with torch.cuda.stream(stream):
        z = torch.randn(1 << 16, device=DEV)
        (z * 2.0 + 1.0).sum().item()


CFGS = [(3, dict(L=2, B=3, Hk=2, Hv=4, V=600)), (5, dict(L=2, B=2, Hk=2, Hv=4, V=600))]


@pytest.mark.parametrize("cfg_id,kw", CFGS)
def test_plain_round_graph_replays_match_eager(cfg_id, kw):
    """One plain round (verify every layer, accept, round rollback) captured
    once and replayed three times; the eager twin runs the same rounds."""
    _need_gpu()
    cfg = W.CONFIGS[cfg_id].with_(**kw)
    ref, gr = _buffers(cfg, 2), _buffers(cfg, 2)
    st = torch.cuda.Stream()
    print("graph plain", cfg_id, flush=True)
    g = None
    for r in range(3):
        with torch.cuda.stream(st):
            sr.run_round(ref, stream=st)
        st.synchronize()
        if g is None:
            # captured after the first eager round, as the bench does
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(st):
                with torch.cuda.graph(g, stream=st):
                    sr.run_round(gr, stream=st)
            torch.cuda.synchronize()
        _eager_work(st)
        g.replay()
        torch.cuda.synchronize()
        want = _state(ref, {"n_keep": ref.n_keep, "path": ref.path, "u": ref.tape.u,
                            "k": ref.tape.k, "g": ref.tape.g})
        got = _state(gr, {"n_keep": gr.n_keep, "path": gr.path, "u": gr.tape.u,
                          "k": gr.tape.k, "g": gr.tape.g})
        _same(got, want, ("plain", cfg_id, r))


@pytest.mark.parametrize("cfg_id,kw", CFGS)
def test_fused_rounds_graph_replays_match_eager(cfg_id, kw):
    """Fused rounds: round 0 runs eagerly on both twins, then one graph per
    tape parity (captured as rounds 1 and 2) is replayed for rounds 1..4;
    the final prefix is applied eagerly to both."""
    _need_gpu()
    cfg = W.CONFIGS[cfg_id].with_(**kw)
    ref, gr = _buffers(cfg, 3), _buffers(cfg, 3)
    fr, fg = sr.FusedRound(ref), sr.FusedRound(gr)
    st = torch.cuda.Stream()
    print("graph fused", cfg_id, flush=True)
    with torch.cuda.stream(st):
        fr.round(0, stream=st, first=True)
        fg.round(0, stream=st, first=True)
    st.synchronize()
    graphs = {}
    for par, rr in ((1, 1), (0, 2)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                fg.round(rr, stream=st)
        graphs[par] = g
    torch.cuda.synchronize()
    for r in range(1, 5):
        with torch.cuda.stream(st):
            fr.round(r, stream=st)
        st.synchronize()
        _eager_work(st)
        graphs[r % 2].replay()
        torch.cuda.synchronize()
        c = r % 2
        want = _state(ref, {"n_keep": fr.n_keeps[c], "path": fr.paths[c], "u": fr.tapes[c].u,
                            "k": fr.tapes[c].k, "g": fr.tapes[c].g})
        got = _state(gr, {"n_keep": fg.n_keeps[c], "path": fg.paths[c], "u": fg.tapes[c].u,
                          "k": fg.tapes[c].k, "g": fg.tapes[c].g})
        _same(got, want, ("fused", cfg_id, r))
    with torch.cuda.stream(st):
        fr.finish(4, stream=st)
        fg.finish(4, stream=st)
    torch.cuda.synchronize()
    assert torch.equal(gr.S, ref.S)


@pytest.mark.parametrize("cfg_id,kw", CFGS)
def test_two_streams_at_once_match_one_at_a_time(cfg_id, kw):
    """Two independent stacks (different seeded draws) run three fused rounds
    each on two streams with no synchronisation between them; each ends bit
    for bit where the same rounds run alone on one stream end (no state is
    shared between calls)."""
    _need_gpu()
    cfg = W.CONFIGS[cfg_id].with_(**kw)
    alone = [_buffers(cfg, 4), _buffers(cfg, 5)]
    both = [_buffers(cfg, 4), _buffers(cfg, 5)]
    s0 = torch.cuda.Stream()
    print("two streams", cfg_id, flush=True)
    frs = [sr.FusedRound(rb) for rb in alone]
    for fr in frs:
        with torch.cuda.stream(s0):
            for r in range(3):
                fr.round(r, stream=s0, first=(r == 0))
            fr.finish(2, stream=s0)
        s0.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    fbs = [sr.FusedRound(rb) for rb in both]
    for r in range(3):
        for fb, st in zip(fbs, streams):
            with torch.cuda.stream(st):
                fb.round(r, stream=st, first=(r == 0))
    for fb, st in zip(fbs, streams):
        with torch.cuda.stream(st):
            fb.finish(2, stream=st)
    torch.cuda.synchronize()
    for i in range(2):
        _same(_state(both[i], {"n_keep": fbs[i].n_keeps[0], "path": fbs[i].paths[0]}),
              _state(alone[i], {"n_keep": frs[i].n_keeps[0], "path": frs[i].paths[0]}),
              ("two streams", cfg_id, i))
