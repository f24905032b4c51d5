#!/usr/bin/env python3
"""Benchmark: speculative rounds through a 30-layer GDN stack on one MI355X.

One step = one speculative round over the whole stack, all on one stream,
with every input already resident in HBM, in one of two forms:
  plain   30 x gdn_verify_chunk (or gdn_tree_verify)  ->  spec_accept_prefix
          ->  gdn_tape_rollback (all layers)  ->  gdn_conv_state_rollback
  fused   30 x gdn_verify_chunk_replay, each first replaying the previous
          round's accepted prefix of its layer  ->  spec_accept_prefix
          ->  gdn_conv_state_rollback
          (gdn_tree_verify_replay for trees; where the library fuses both)
Both do the same work per round in steady state: K timed fused rounds replay
K accepted prefixes.  `value` is the form spec_round.fused_pays picks for
the shape (--round forces one); both are reported under "rounds".  Each
round is captured once per input set into a HIP graph and replayed (eager
with --eager).

Prints ONE JSON line.  `value` is verified draft tokens per second for the
30-layer stack (B * T drafted tokens per round / round time).  Extra fields
give accepted and committed tokens/s, per-kernel times, whole-round HBM
fraction from the algorithmic byte model, the dominant kernel's roofline
(measured with HIP events around its launches on the launch stream), and the
fp64 oracle's throughput on a bounded sample on the host cores.

Workloads (seeded synthetic, Qwen3.6-shaped GDN layers: 16 q/k heads and
32 v heads of 128, conv kernel 4, bf16 inputs, fp32 state):
  --config 3 (default)  30 layers, batch 32, N=8 chain, per-position acceptance 0.36
  --config 4            30 layers, batch 256, N=16 chain, acceptance 0.85
  --config 5            30 layers, batch 64, 64-node draft trees
  --config 1 / 2        tiny and one-layer cases (launch-bound; parity cases)
`value` is the --config workload's; the run also times the workloads named by
--also (default 4 and 5) and reports each under other_workloads with the same
fields.  Every chain workload also reports rejection-sampling acceptance, and
every workload a rollback sweep (each sequence forced to n accepted steps,
chain prefixes or tree paths) with its fit t(n) = c0 [n >= 1] + c1 n.  The
line ends with a measured device-to-device copy rate and the fp64 oracle's
throughput on the host cores (all threads and one core).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E datasheet peak
ROOT = os.path.dirname(os.path.abspath(__file__))


def measured_traffic(workload: str):
    """(HBM bytes, algorithmic bytes) per verify launch of the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (calibrated on a plain copy), or
    None when the sources of the kernel that serves this workload changed
    since the counters were taken (each workload records the files it
    hashed)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "verify_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    w = rec.get("workloads", {}).get(workload)
    if w is None:
        return None
    h = hashlib.sha256()
    for src in w.get("sources", []):
        with open(os.path.join(ROOT, src), "rb") as g:
            h.update(g.read())
    if not w.get("sources") or h.hexdigest() != w.get("source_sha256"):
        return None
    return w["traffic_bytes"], w["algorithmic_bytes"], w["source_sha256"]


def rollback_sweep(cfg, rb, stream, reps=10):
    """Rollback time (tape replay + conv window, one gdn_round_rollback over
    the stack) with every sequence forced to the same accepted length n;
    least-squares fit of t(n) = c0 [n >= 1] + c1 n over n >= 1.  Chains
    sweep n = 0..T.  Trees replay along a path of n tape entries (a fixed
    random order of each sequence's nodes, so the replay gathers its
    entries), n = 0..8 (the deepest accepted path) and 16, 32, 64."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    from speculative_decode_verify_gdn_amd import spec_round as sr
    if cfg.is_tree:
        gen = torch.Generator(device=rb.path.device).manual_seed(cfg.seed ^ 0x5B)
        perm = torch.argsort(torch.rand(rb.path.shape, device=rb.path.device, generator=gen), 1)
        rb.path.copy_(perm.to(torch.int32))
        ns = [n for n in list(range(9)) + [16, 32, 64] if n <= cfg.T]
    else:
        ns = list(range(cfg.T + 1))
    # `reps` calls in one graph, so that a short call is timed on the GPU
    # and not by the host's graph-launch rate
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            sr.rollback(rb, stream)
    us = []
    for n in ns:
        rb.n_keep.fill_(n)
        g.replay()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(2):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) / (2 * reps) * 1e3)
    n1 = np.array([n for n in ns if n >= 1], dtype=np.float64)
    A = np.stack([np.ones_like(n1), n1], 1)
    y = np.array([t for n, t in zip(ns, us) if n >= 1])
    coef, *_ = np.linalg.lstsq(A, y, rcond=None)
    pred = A @ coef
    r2 = 1.0 - float(np.sum((y - pred) ** 2) / max(np.sum((y - y.mean()) ** 2), 1e-30))
    tape_tok = cfg.Hv * cfg.Dv * 4 + cfg.Hk * cfg.Dk * 4 + cfg.Hv * 4
    tape_stack = cfg.L * cfg.B * tape_tok
    esz = 2 if cfg.dtype == torch.bfloat16 else 4
    state_pass = cfg.L * cfg.B * (2 * cfg.Hv * cfg.Dv * cfg.Dk * 4 + 2 * (cfg.K - 1) * cfg.C * esz)
    return {"path": "tree path (gathered tape entries)" if cfg.is_tree else "chain prefix",
            "n": ns, "us": us, "t0_us": us[0] if ns[0] == 0 else None,
            "c0_us": float(coef[0]), "c1_us_per_token": float(coef[1]), "r2": r2,
            "tape_bytes_per_token_per_stack": tape_stack,
            "c1_bound_us_at_peak": tape_stack / (HBM_PEAK_GBS * 1e3),
            "c0_bound_us_at_peak": state_pass / (HBM_PEAK_GBS * 1e3)}


def fused_pass(cfg, rbs, shared, stream, steps, warmup, eager):
    """The same rounds with each layer's state rollback folded into the next
    round's verify (gdn_verify_chunk_replay / gdn_tree_verify_replay): per
    round, 30 fused verifies, accept, conv rollback.  Returns round time, per-phase kernel times and the
    accepted lengths of the timed rounds."""
    from speculative_decode_verify_gdn_amd import binding as gb
    from speculative_decode_verify_gdn_amd import spec_round as sr
    dev = shared.S.device
    tapes = [shared.tape, gb.Tape.empty(shared.sh, cfg.T, dev)]
    nks = [torch.zeros((cfg.B,), dtype=torch.int32, device=dev) for _ in range(2)]
    paths = [torch.full((cfg.B, cfg.T), -1, dtype=torch.int32, device=dev) for _ in range(2)]
    frs = [sr.FusedRound(rb, tapes=tapes, n_keeps=nks, paths=paths) for rb in rbs]
    n = len(frs)
    # round i runs input set i % n with tape parity i % 2; capture one graph
    # per (set, parity) pair that occurs
    keys = sorted({(i % n, i % 2) for i in range(2 * n)})
    ev = lambda: torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        frs[0].round(0, first=True)
        for i in range(1, 2 * n):  # eager warm-up of every (set, parity)
            frs[i % n].round(i)
        torch.cuda.synchronize()
        graphs, phases = {}, {}
        for j, par in keys:
            if not eager:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    frs[j].round(par)
                graphs[(j, par)] = g
            gv, ga = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(gv, stream=stream):
                frs[j].verify_layers(par)
            with torch.cuda.graph(ga, stream=stream):
                frs[j].accept_and_conv(par)
            phases[(j, par)] = (gv, ga)
        torch.cuda.synchronize()
        base = 2 * n  # rounds so far (keeps the parity chain unbroken)

        def step(i):
            key = (i % n, i % 2)
            if graphs:
                graphs[key].replay()
            else:
                frs[key[0]].round(key[1])

        for i in range(base, base + warmup):
            step(i)
        base += warmup
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for i in range(base, base + steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        total_ms = e0.elapsed_time(e1)
        base += steps
        n_hist = torch.zeros((steps, cfg.B), dtype=torch.int32, device=dev)
        p_hist = torch.zeros((steps, cfg.B), dtype=torch.int32, device=dev)
        v_ev, a_ev = [], []
        for s_i, i in enumerate(range(base, base + steps)):
            gv, ga = phases[(i % n, i % 2)]
            p_hist[s_i].copy_(nks[(i + 1) % 2])  # what this round's verify replays
            for g, acc in ((gv, v_ev), (ga, a_ev)):
                s0, s1 = ev(), ev()
                s0.record(stream)
                g.replay()
                s1.record(stream)
                acc.append((s0, s1))
            n_hist[s_i].copy_(nks[i % 2])
        torch.cuda.synchronize()
    assert int(shared.dev_err.item()) == 0, "device-side error bits set"
    return {"ms": total_ms / steps,
            "verify_replay_ms": float(np.mean([a.elapsed_time(b) for a, b in v_ev])) / cfg.L,
            "accept_conv_ms": float(np.mean([a.elapsed_time(b) for a, b in a_ev])),
            "n_keep": n_hist.cpu().numpy(), "n_prev": p_hist.cpu().numpy()}


def sample_accept_pass(cfg, rb, stream, reps, oracle_seqs=2):
    """Rejection-sampling acceptance (spec_accept_sample, temperature 1) on
    the round's drafts and a copy of its logits in which each draft token's
    logit is reset so that its probability is a seeded draw from U(0.05,
    0.95) (before bf16 rounding), so drafts are kept and rejected at rates
    like a real draft model's and both branches (keep, and resample with
    the rejected token removed) run; seeded uniforms.  Reports the mean time
    per call of a replayed graph, its algorithmic bytes (every logits row
    read once, the drawn chunk re-read, partials written and read), the mean
    kept length, and the fp64 oracle's time on `oracle_seqs` sequences scaled
    to the batch."""
    from speculative_decode_verify_gdn_amd import binding as gb
    B, T, V = cfg.B, cfg.T, cfg.V
    dev = rb.S.device
    gen = torch.Generator(device=dev).manual_seed(cfg.seed ^ 0x5A)
    uni = torch.rand((B, T + 1), device=dev, generator=gen)
    p_draft = 0.05 + 0.9 * torch.rand((B, T), device=dev, generator=gen)
    logits = rb.logits.clone()
    d = rb.draft.to(torch.int64).unsqueeze(-1)
    for b0 in range(0, B, 16):  # bounded fp32 temporaries
        z = logits[b0:b0 + 16, :T].float()
        lse = torch.logsumexp(z, -1)
        zd = z.gather(-1, d[b0:b0 + 16]).squeeze(-1)
        lse_others = lse + torch.log1p(-torch.exp(zd - lse).clamp(max=1 - 1e-7))
        p = p_draft[b0:b0 + 16]
        new = (lse_others + torch.log(p / (1 - p))).to(logits.dtype)
        logits[b0:b0 + 16, :T].scatter_(-1, d[b0:b0 + 16], new.unsqueeze(-1))
        del z
    i32 = dict(device=dev, dtype=torch.int32)
    n, path, tok = torch.empty((B,), **i32), torch.empty((B, T), **i32), torch.empty((B,), **i32)
    ws = torch.empty((gb.spec_sample_workspace_bytes(B, T, V),), device=dev, dtype=torch.uint8)
    call = lambda: gb.spec_accept_sample(rb.draft, logits, 1.0, uni, n, path, tok, ws,
                                         dev_err=rb.dev_err)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            call()
        g.replay()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    esz = 2 if logits.dtype == torch.bfloat16 else 4
    split = (V + 4095) // 4096
    byts = B * (T + 1) * V * esz + B * 4096 * esz + 2 * B * (T + 1) * split * 8 \
        + B * T * (4 + esz) + B * (T + 1) * 4 + B * (T + 2) * 4
    import oracle
    k = min(oracle_seqs, B)
    lg = logits[:k].double().cpu().numpy()
    dr = rb.draft[:k].cpu().numpy()
    un = uni[:k].double().cpu().numpy()
    t0 = time.perf_counter()
    oracle.accept_sample(dr, lg, 1.0, un)
    o_us = (time.perf_counter() - t0) * 1e6 * B / k
    gbs = byts / (us * 1e-6) / 1e9
    return {"us_per_round": us, "algorithmic_bytes": byts, "achieved_GBps": gbs,
            "frac": gbs / HBM_PEAK_GBS, "mean_kept": float(n.float().mean().item()),
            "draft_probability": "U(0.05, 0.95) per draft position",
            "oracle_us_per_round": o_us, "oracle_sample_sequences": k, "temperature": 1.0}


def draft_sweep(cfg, stream, Ns=(1, 2, 4, 8, 16), reps=10):
    """Round time of the 30-layer stack for each draft length N (same batch,
    acceptance law and round form rule as the workload), the acceptance
    estimated from the rounds' accepted lengths, and the draft length the
    host policy (policy.choose_draft_length) picks from them."""
    from speculative_decode_verify_gdn_amd import binding as gb
    from speculative_decode_verify_gdn_amd import policy as pol
    from speculative_decode_verify_gdn_amd import spec_round as sr
    t_us, forms = {}, {}
    stats = pol.AcceptanceStats()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for n in Ns:
        c = cfg.with_(T=n)
        base, sets = build_sets(c, 1, "cuda")
        inp, acc = sets[0]
        rb = sr.RoundBuffers(sh=gb.GdnShape(c.L, c.B, c.Hk, c.Hv, c.Dk, c.Dv, c.K, c.silu, c.eps,
                                            c.dtype),
                             T=n, V=c.V, tree=False, S=base["S0"], conv_state=base["conv_state"],
                             conv_w=base["conv_w"], x=inp["x"], a=inp["a"], b=inp["b"],
                             logits=acc["logits"], draft=acc["draft"], parent=None)
        fused = sr.fused_pays(rb.sh, n, False)
        forms[n] = "fused" if fused else "plain"
        with torch.cuda.stream(stream):
            if fused:
                fr = sr.FusedRound(rb)
                fr.round(0, first=True)
                fr.round(1)
                graphs = []
                for par in (0, 1):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=stream):
                        fr.round(par)
                    graphs.append(g)
                nk = fr.n_keeps[1]
            else:
                sr.run_round(rb)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    sr.run_round(rb)
                graphs = [g]
                nk = rb.n_keep
            torch.cuda.synchronize()
            for i in range(2):
                graphs[i % len(graphs)].replay()
            a, b = ev(), ev()
            a.record(stream)
            for i in range(reps):
                graphs[i % len(graphs)].replay()
            b.record(stream)
            torch.cuda.synchronize()
        t_us[n] = a.elapsed_time(b) / reps * 1e3
        stats.update(nk, n)
        del rb, base, sets, inp, acc, graphs
        torch.cuda.empty_cache()
    alpha = stats.alpha()
    chosen = pol.choose_draft_length(alpha, t_us)
    return {"t_round_us": t_us, "round_form": forms, "alpha_estimate": alpha,
            "committed_tokens_per_s": {n: cfg.B * pol.expected_committed(alpha, n) / (t * 1e-6)
                                       for n, t in t_us.items()},
            "chosen_draft_length": chosen}


def prefill_pass(cfg, n_tokens, stream, reps=3, gate_per_key=False):
    """gdn_prefill of n_tokens through the workload's L layers and B
    sequences (graph replay): time per call, prefilled tokens/s (B x
    n_tokens per call; each layer sees every token) and the HBM fraction of
    the byte model: per (layer, seq) one state read and write, plus per
    token x, gates, o, and the chunk tape written then read back."""
    from speculative_decode_verify_gdn_amd import binding as gb
    from speculative_decode_verify_gdn_amd import workload as W
    c = cfg.with_(T=n_tokens)
    inp = W.layer_inputs(c, 0, "cuda")
    sh = gb.GdnShape(c.L, c.B, c.Hk, c.Hv, c.Dk, c.Dv, c.K, c.silu, c.eps, c.dtype,
                     gate_per_key=gate_per_key)
    if gate_per_key:
        gen = torch.Generator(device="cuda").manual_seed(c.seed ^ 0x3C)
        gs = sh.gate_shape(n_tokens)
        a = torch.empty(gs, device="cuda", dtype=c.dtype)
        for l in range(gs[0]):  # per layer: the fp32 draw of a whole stack can exceed HBM
            a[l] = 0.05 + 0.95 * torch.rand(gs[1:], device="cuda", generator=gen)
        inp["a"] = a
    o = torch.empty((c.L, c.B, n_tokens, c.Hv, c.Dv), device="cuda")
    need = gb.gdn_prefill_workspace_bytes(sh)
    ws = torch.empty((need,), device="cuda", dtype=torch.uint8) if need else None
    S, cs = inp["S0"], inp["conv_state"]
    call = lambda: gb.gdn_prefill(sh, inp["x"], cs, inp["conv_w"], inp["a"], inp["b"], S, o, ws)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            call()
        g.replay()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    esz = 2 if c.dtype == torch.bfloat16 else 4
    P = c.Hv * c.Dv * c.Dk * 4
    # the per-key form and the scalar gate's 128-dim heads keep the state in
    # registers across the chunks: one state read and write per call; other
    # shapes read and write it once per 16-token chunk
    one_pass = gate_per_key or (c.Dk == 128 and c.Dv == 128)
    chunks = 1 if one_pass else (n_tokens + 15) // 16
    # (the one-pass chunk loop keeps its tape's k rows per v-head)
    kh = c.Hv if c.Dk == c.Dv == 128 and (not gate_per_key or c.dtype == torch.bfloat16) else c.Hk
    tape_tok = c.Hv * c.Dv * 4 + kh * c.Dk * 4 + c.Hv * (c.Dk if gate_per_key else 1) * 4
    gate = c.Hv * (c.Dk if gate_per_key else 1) * esz + c.Hv * esz
    # the chain kernel's chunk loop writes each chunk's tape and reads it back;
    # the per-key sequential kernel (other shapes) keeps no tape
    chain_loop = not gate_per_key or (c.Dk == c.Dv == 128 and c.dtype == torch.bfloat16)
    tape = 2 * tape_tok if chain_loop else 0
    per_seq = chunks * 2 * P + n_tokens * (c.C * esz + gate + c.Hv * c.Dv * 4 + tape) \
        + chunks * 2 * (c.K - 1) * c.C * esz
    byts = c.L * c.B * per_seq
    del inp, o, ws
    torch.cuda.empty_cache()
    return {"tokens": n_tokens, "layers": c.L, "batch": c.B, "gate_per_key": gate_per_key,
            "ms_per_call": ms,
            "tokens_per_s": c.B * n_tokens / (ms * 1e-3), "algorithmic_bytes": byts,
            "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def vgate_pass(cfg, stream, steps):
    """The workload's rounds with the decay gate per key channel
    (a [L,B,T,Hv,Dk], drawn U(0.05, 1)), in both forms: the plain round
    (verify, accept, rollback) with its verify time per layer, byte model and
    HBM fraction and its rollback time, and the fused round (the rollback
    folded into the next round's verify, which replays the previous accepted
    prefix or path); value_by_rule is the form spec_round.fused_pays picks."""
    from speculative_decode_verify_gdn_amd import binding as gb
    from speculative_decode_verify_gdn_amd import spec_round as sr
    base, sets = build_sets(cfg, 1, "cuda")
    inp, acc = sets[0]
    tree = cfg.is_tree
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed ^ 0x7A)
    a = (0.05 + 0.95 * torch.rand((cfg.L, cfg.B, cfg.T, cfg.Hv, cfg.Dk), device="cuda",
                                  generator=gen)).to(cfg.dtype)
    sh = gb.GdnShape(cfg.L, cfg.B, cfg.Hk, cfg.Hv, cfg.Dk, cfg.Dv, cfg.K, cfg.silu, cfg.eps,
                     cfg.dtype, gate_per_key=True)
    rb = sr.RoundBuffers(sh=sh, T=cfg.T, V=cfg.V, tree=tree, S=base["S0"],
                         conv_state=base["conv_state"], conv_w=base["conv_w"], x=inp["x"], a=a,
                         b=inp["b"], logits=acc["logits"], draft=acc["draft"],
                         parent=acc["parent"] if tree else None)
    fr = sr.FusedRound(rb)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        return g

    def timed(gs):
        """Mean time of one graph of `gs`, replayed in turn."""
        for g in gs:
            g.replay()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(steps):
            for g in gs:
                g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (steps * len(gs))

    with torch.cuda.stream(stream):
        sr.run_round(rb)
        torch.cuda.synchronize()
        plain = [capture(lambda: sr.run_round(rb)),
                 capture(lambda: [sr.verify_layer(rb, l) for l in range(cfg.L)]),
                 capture(lambda: sr.rollback(rb))]
        t_plain = [timed([g]) for g in plain]
        fr.round(0, first=True)
        fr.round(1)
        torch.cuda.synchronize()
        f_round = [capture(lambda: fr.round(0)), capture(lambda: fr.round(1))]
        f_verify = [capture(lambda: fr.verify_layers(0)), capture(lambda: fr.verify_layers(1))]
        t_fround, t_fverify = timed(f_round), timed(f_verify)
    assert int(rb.dev_err.item()) == 0, "device-side error bits set"
    esz = 2 if cfg.dtype == torch.bfloat16 else 4
    extra = cfg.B * cfg.T * cfg.Hv * (cfg.Dk - 1) * (esz + 4)  # larger gate read and tape g
    vb = verify_bytes_per_launch(cfg, cfg.B) + extra
    v_ms = t_plain[1] / cfg.L
    pays = sr.fused_pays(sh, cfg.T, tree)
    del rb, fr, base, sets, inp, acc, a, plain, f_round, f_verify
    torch.cuda.empty_cache()
    return {"round_by_rule": "fused" if pays else "plain",
            "value_by_rule": cfg.B * cfg.T / ((t_fround if pays else t_plain[0]) * 1e-3),
            "round_ms": t_plain[0], "value": cfg.B * cfg.T / (t_plain[0] * 1e-3),
            "verify_per_layer_ms": v_ms, "verify_bytes_per_launch": vb,
            "verify_hbm_frac": vb / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "rollback_state_and_conv_ms": t_plain[2],
            "kernel": (("k_verify_tree (per-key gate)" if 12 < cfg.T <= 64 and cfg.dtype == torch.bfloat16
                        and cfg.Dk == cfg.Dv == 128 else "k_verify_vgt") if tree else
                       ("k_verify_chain (per-key gate)" if cfg.T <= 16 and cfg.dtype == torch.bfloat16
                        and cfg.Dk == cfg.Dv == 128 else "k_verify_vg")),
            "fused": {"round_ms": t_fround, "value": cfg.B * cfg.T / (t_fround * 1e-3),
                      "verify_per_layer_ms": t_fverify / cfg.L,
                      "kernel": ("k_verify_chain (per-key gate, replay)"
                                 if not tree and cfg.T <= 16 and cfg.dtype == torch.bfloat16
                                 and cfg.Dk == cfg.Dv == 128 else
                                 "k_verify_tree (per-key gate, replay)"
                                 if tree and 12 < cfg.T <= 64 and cfg.dtype == torch.bfloat16
                                 and cfg.Dk == cfg.Dv == 128 else "k_verify_vgt")}}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--input-sets", type=int, default=4,
                    help="distinct pre-generated rounds of drafts/logits cycled through")
    ap.add_argument("--eager", action="store_true", help="launch without HIP graph capture")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target host time of the oracle sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--round", choices=("auto", "plain", "fused"), default="auto",
                    help="round whose time is `value`: plain (verify, accept, rollback) or fused "
                         "(the state rollback folded into the next round's verify); auto picks "
                         "by the rule in spec_round.fused_pays; chains also report the other")
    ap.add_argument("--prefill", type=int, default=0, metavar="N",
                    help="also time gdn_prefill of N tokens through the workload's stack")
    ap.add_argument("--gate-per-key", action="store_true",
                    help="also time the rounds with the decay gate per key channel")
    ap.add_argument("--draft-sweep", action="store_true",
                    help="also time rounds at N = 1, 2, 4, 8, 16 drafts and report the draft "
                         "length the host policy picks (chain workloads)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the rollback sweeps (every sequence forced to n accepted steps)")
    ap.add_argument("--also", default="4,5",
                    help="comma-separated further workloads timed in the same run and reported "
                         "under other_workloads (default: the 256-sequence 16-draft stack and "
                         "the 64-node tree stack; empty for none)")
    return ap.parse_args()


# ------------------------------------------------------------- byte model --

def verify_bytes_per_launch(cfg, B) -> int:
    """Algorithmic HBM bytes of one verify launch (one layer, B sequences)."""
    esz = 2 if cfg.dtype == torch.bfloat16 else 4
    T, C = cfg.T, cfg.C
    P = cfg.Hv * cfg.Dv * cfg.Dk * 4                     # state read once
    per_tok = (C * esz                                  # raw qkv row
               + 2 * cfg.Hv * esz                       # gates a, b
               + cfg.Hv * cfg.Dv * 4                    # output o
               + cfg.Hv * cfg.Dv * 4 + cfg.Hk * cfg.Dk * 4 + cfg.Hv * 4)  # tape u, k, g
    per_seq = P + T * per_tok + (cfg.K - 1) * C * esz  # + conv window read
    if cfg.is_tree:
        per_seq += T * 4 + T * cfg.K * 4 // cfg.L       # parent array; conv_win once per stack
    return B * per_seq + C * cfg.K * 4                  # + conv weights


def fused_verify_bytes(cfg, B, n_prev: np.ndarray) -> float:
    """Algorithmic bytes of one fused verify launch (gdn_verify_chunk_replay,
    gdn_tree_verify_replay): the verify's bytes, plus for every sequence
    whose previous round kept n >= 1 the replayed state's write and its n
    previous tape entries (and, for trees, path entries); the state read is
    the verify's own."""
    P = cfg.Hv * cfg.Dv * cfg.Dk * 4
    tape_tok = cfg.Hv * cfg.Dv * 4 + cfg.Hk * cfg.Dk * 4 + cfg.Hv * 4 + (4 if cfg.is_tree else 0)
    n = n_prev.astype(np.int64)
    return verify_bytes_per_launch(cfg, B) + float(np.sum((n >= 1) * P + n * tape_tok))


def roofline(kernel: str, bytes_per_launch: float, ms_per_launch: float, traffic) -> dict:
    gbs = bytes_per_launch / (ms_per_launch * 1e-3) / 1e9
    # traffic: calibrated FETCH_SIZE + WRITE_SIZE bytes per launch of the
    # committed counter runs, with the algorithmic bytes of those launches
    # (equal to bytes_per_launch except where they depend on accepted lengths)
    return {"kernel": kernel, "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": None if traffic is None else traffic[0],
            "traffic_algorithmic_bytes": None if traffic is None else traffic[1],
            "traffic_source": None if traffic is None else
            "profiles/verify_traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE per launch, "
            "scaled by a plain copy's counters; sources sha256 %s" % traffic[2][:16],
            "bytes_per_launch": bytes_per_launch}


def fused_kernel(cfg) -> bool:
    """Whether the library runs the replay and the verify as one kernel."""
    if not cfg.is_tree:
        return cfg.T <= 16
    return 16 < cfg.T <= 64 and cfg.dtype == torch.bfloat16 and cfg.Dk == cfg.Dv == 128


def verify_kernel_name(cfg, fused: bool = False) -> str:
    """The verify kernel the library dispatches for this workload (one layer)."""
    if fused and cfg.is_tree:
        return "k_verify_tree, replay variant (gdn_tree_verify_replay, one layer)"
    if fused:
        return "k_verify_chain, replay variant (gdn_verify_chunk_replay, one layer)"
    if not cfg.is_tree and cfg.T <= 16:
        return "k_verify_chain (gdn_verify_chunk, chains of <= 16 tokens, one layer)"
    if cfg.is_tree and cfg.T > 16 and cfg.dtype == torch.bfloat16 and cfg.Dk == cfg.Dv == 128:
        return "k_verify_tree (gdn_tree_verify, trees of 17..64 nodes, one layer)"
    return "k_verify_wy (%s, one layer)" % ("gdn_tree_verify" if cfg.is_tree else "gdn_verify_chunk")


def rollback_bytes(cfg, n_keep: np.ndarray) -> int:
    """Tape replay: for n >= 1 read + write the state, read n tape entries."""
    P = cfg.Hv * cfg.Dv * cfg.Dk * 4
    tape_tok = cfg.Hv * cfg.Dv * 4 + cfg.Hk * cfg.Dk * 4 + cfg.Hv * 4
    n = n_keep.astype(np.int64)
    return int(cfg.L * np.sum((n >= 1) * 2 * P + n * tape_tok))


def conv_rollback_bytes(cfg, n_keep: np.ndarray) -> int:
    esz = 2 if cfg.dtype == torch.bfloat16 else 4
    return int(cfg.L * np.sum(n_keep >= 1) * 2 * (cfg.K - 1) * cfg.C * esz)


def accept_bytes(cfg, B) -> int:
    return B * (cfg.T + 1) * cfg.V * 2 + B * cfg.T * 4 * (2 if cfg.is_tree else 1)


# ---------------------------------------------------------------- helpers --

def calib_copy():
    n = 256 << 20
    a = torch.empty(n // 4, device="cuda", dtype=torch.float32).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "launches": 5}))


def build_sets(cfg, n_sets, dev):
    from speculative_decode_verify_gdn_amd import workload as W
    base = W.layer_inputs(cfg, 0, dev)
    sets = []
    for r in range(n_sets):
        inp = W.layer_inputs(cfg, r, dev) if r else base
        acc = W.tree_accept_inputs(cfg, r, dev) if cfg.is_tree else W.chain_accept_inputs(cfg, r, dev)
        sets.append((inp, acc))
    return base, sets


def oracle_baseline(cfg, seconds: float) -> dict:
    """Time the fp64 oracle's round on a bounded sample of (layer, sequence)
    units -- verify, accept, tape and conv rollback for L_s layers of B_s
    sequences -- and scale to the whole stack: the units are independent and
    equal in cost, so t_round = t_sample * (L * B) / (L_s * B_s)."""
    import oracle
    from speculative_decode_verify_gdn_amd import workload as W

    def prepare(L_s, B_s):
        c = cfg.with_(L=L_s, B=B_s)
        inp = {k: W.to_f64(v) for k, v in W.layer_inputs(c, 0, "cpu").items()}
        acc = W.tree_accept_inputs(c, 0, "cpu") if c.is_tree else W.chain_accept_inputs(c, 0, "cpu")
        sh = oracle.Shape(L_s, B_s, c.Hk, c.Hv, c.Dk, c.Dv, c.K, c.silu, c.eps)
        return (sh, inp, acc["draft"].numpy(), W.to_f64(acc["logits"]),
                acc["parent"].numpy() if c.is_tree else None)

    def run(sample):
        sh, inp, draft, logits, parent = sample
        keys = ("x", "conv_state", "conv_w", "a", "b", "S0")
        t0 = time.perf_counter()
        if parent is None:
            out = oracle.verify_chunk(sh, *[inp[k] for k in keys], want_final=False)
        else:
            out = oracle.tree_verify(sh, parent, *[inp[k] for k in keys])
        n, path, _ = oracle.accept(draft, logits, parent)
        pth = path if parent is not None else None
        oracle.tape_rollback(sh, inp["S0"], out["u"], out["k"], out["g"], n, pth)
        oracle.conv_rollback(sh, inp["conv_state"], inp["x"], n, pth)
        return time.perf_counter() - t0

    oracle.build(force=False)
    nthr = max(1, oracle.num_threads())
    L_s = min(cfg.L, nthr)
    # fp64 host bytes one sampled sequence needs (state twice, o, u, x, logits)
    per_seq = L_s * 8 * (2 * cfg.Hv * cfg.Dv * cfg.Dk + 2 * cfg.T * cfg.Hv * cfg.Dv
                         + cfg.T * cfg.C) + 8 * (cfg.T + 1) * cfg.V
    b_cap = int(max(1, min(cfg.B, 3e9 // per_seq)))
    B_s = min(2, b_cap)
    t = run(prepare(L_s, B_s))
    want = int(B_s * seconds / max(t, 1e-3))
    if want > B_s:
        B_s = int(min(b_cap, want))
    # the sample is memory-bounded; repeat it until about `seconds` of CPU work
    sample = prepare(L_s, B_s)
    times = [run(sample)]
    while sum(times) < seconds:
        times.append(run(sample))
    del sample
    t = float(np.mean(times))
    t_round = t * (cfg.L * cfg.B) / (L_s * B_s)
    # the same round on one core: one layer of one sequence, about a fifth of
    # the time budget
    oracle.set_num_threads(1)
    try:
        one = prepare(1, 1)
        t1 = [run(one)]
        while sum(t1) < seconds / 5:
            t1.append(run(one))
        del one
    finally:
        oracle.set_num_threads(nthr)
    t1m = float(np.mean(t1))
    t1_round = t1m * cfg.L * cfg.B
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": cfg.B * cfg.T / t_round, "unit": "tokens/s", "cores": nthr,
            "kind": "oracle", "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": "fp64 oracle round (verify, accept, tape and conv rollback) on %d layers x "
                      "%d sequences of the %d x %d workload, %d repetitions in %.1f s (mean "
                      "%.2f s), scaled by unit count to %.1f s per round"
                      % (L_s, B_s, cfg.L, cfg.B, len(times), sum(times), t, t_round),
            "one_core": {"value": cfg.B * cfg.T / t1_round, "unit": "tokens/s", "cores": 1,
                         "sample": "the same round on 1 layer x 1 sequence, %d repetitions in "
                                   "%.1f s (mean %.3f s), scaled by unit count to %.1f s per "
                                   "round" % (len(t1), sum(t1), t1m, t1_round)}}


# ------------------------------------------------------------------- main --

def measure_workload(cfg, args, stream, extras: bool):
    """Time the workload's rounds (plain, and fused where the library fuses)
    as replayed HIP graphs, plus per-phase kernel times.  Returns a dict of
    the round forms with their values, kernel times, byte models and the
    dominant kernel's roofline, the form the library's rule picks, and (when
    `extras`) the sampling-acceptance and rollback-sweep measurements."""
    from speculative_decode_verify_gdn_amd import binding as gb
    from speculative_decode_verify_gdn_amd import spec_round as sr
    dev = "cuda"
    torch.cuda.empty_cache()
    base, sets = build_sets(cfg, args.input_sets, dev)
    S = base["S0"]
    cs = base["conv_state"]
    conv_w = base["conv_w"]
    shared = None
    rbs = []
    for inp, acc in sets:
        rb = sr.RoundBuffers(sh=gb.GdnShape(cfg.L, cfg.B, cfg.Hk, cfg.Hv, cfg.Dk, cfg.Dv, cfg.K,
                                            cfg.silu, cfg.eps, cfg.dtype),
                             T=cfg.T, V=cfg.V, tree=cfg.is_tree, S=S, conv_state=cs,
                             conv_w=conv_w, x=inp["x"], a=inp["a"], b=inp["b"],
                             logits=acc["logits"], draft=acc["draft"],
                             parent=acc.get("parent") if cfg.is_tree else None,
                             o=None if shared is None else shared.o,
                             tape=None if shared is None else shared.tape)
        if shared is None:
            shared = rb
        rbs.append(rb)
    n_hist = torch.zeros((args.steps, cfg.B), dtype=torch.int32, device=dev)

    graphs = []
    with torch.cuda.stream(stream):
        for rb in rbs:  # eager warm-up of every set (also loads code objects)
            sr.run_round(rb)
        torch.cuda.synchronize()
        if not args.eager:
            for rb in rbs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    sr.run_round(rb)
                graphs.append(g)
        torch.cuda.synchronize()

        def step(i):
            if graphs:
                graphs[i % len(rbs)].replay()
            else:
                sr.run_round(rbs[i % len(rbs)])

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        total_ms = e0.elapsed_time(e1)

        # Kernel pass: the same rounds as three captured phases (verify of all
        # layers, accept, rollback), each replayed between HIP events on the
        # launch stream, so per-kernel times carry no host launch gaps.
        ev = lambda: torch.cuda.Event(enable_timing=True)
        phase_graphs = []
        for rb in rbs:
            gv, ga, gr = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(gv, stream=stream):
                for l in range(cfg.L):
                    sr.verify_layer(rb, l)
            with torch.cuda.graph(ga, stream=stream):
                sr.accept(rb)
            with torch.cuda.graph(gr, stream=stream):
                sr.rollback(rb)
            phase_graphs.append((gv, ga, gr))
        torch.cuda.synchronize()
        v_ms, a_ms, r_ms = [], [], []
        for i in range(args.steps):
            rb = rbs[i % len(rbs)]
            gv, ga, gr = phase_graphs[i % len(rbs)]
            for g, acc in ((gv, v_ms), (ga, a_ms)):
                s0, s1 = ev(), ev()
                s0.record(stream)
                g.replay()
                s1.record(stream)
                acc.append((s0, s1))
            n_hist[i].copy_(rb.n_keep)
            s0, s1 = ev(), ev()
            s0.record(stream)
            gr.replay()
            s1.record(stream)
            r_ms.append((s0, s1))
        torch.cuda.synchronize()
        del phase_graphs, graphs
    verify_ms = float(np.mean([a.elapsed_time(b) for a, b in v_ms])) / cfg.L
    accept_ms = float(np.mean([a.elapsed_time(b) for a, b in a_ms]))
    rollback_ms = float(np.mean([a.elapsed_time(b) for a, b in r_ms]))
    assert int(shared.dev_err.item()) == 0, "device-side error bits set"

    pays = sr.fused_pays(shared.sh, cfg.T, cfg.is_tree)
    mode = args.round if args.round != "auto" else ("fused" if pays else "plain")
    fusable = fused_kernel(cfg)
    if mode == "fused" and not fusable:
        raise SystemExit("the library fuses chains of at most 16 drafts and trees of 17..64 "
                         "nodes (bf16, 128-dim heads) only")
    fused = None
    if fusable:
        fused = fused_pass(cfg, rbs, shared, stream, args.steps, args.warmup, args.eager)

    B, T = cfg.B, cfg.T
    vb = verify_bytes_per_launch(cfg, B)
    ms = total_ms / args.steps
    n_keep = n_hist.cpu().numpy()
    plain_bytes = float(np.mean([cfg.L * vb + accept_bytes(cfg, B) + rollback_bytes(cfg, n_keep[i])
                                 + conv_rollback_bytes(cfg, n_keep[i]) for i in range(args.steps)]))
    rb_bytes = float(np.mean([rollback_bytes(cfg, n_keep[i]) + conv_rollback_bytes(cfg, n_keep[i])
                              for i in range(args.steps)]))
    rounds = {"plain": {
        "value": B * T / (ms * 1e-3), "ms_per_step": ms, "n_keep": n_keep,
        "round_bytes": plain_bytes,
        "kernel_ms": {"verify_per_layer": verify_ms, "accept": accept_ms,
                      "rollback_state_and_conv": rollback_ms},
        "rollback_hbm_frac": rb_bytes / (rollback_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": roofline(verify_kernel_name(cfg), vb, verify_ms,
                             measured_traffic(cfg.name))}}
    if fused is not None:
        fms = fused["ms"]
        nk, npv = fused["n_keep"], fused["n_prev"]
        fvb = float(np.mean([fused_verify_bytes(cfg, B, npv[i]) for i in range(args.steps)]))
        fused_bytes = float(np.mean([cfg.L * fused_verify_bytes(cfg, B, npv[i]) + accept_bytes(cfg, B)
                                     + conv_rollback_bytes(cfg, nk[i]) for i in range(args.steps)]))
        rounds["fused"] = {
            "value": B * T / (fms * 1e-3), "ms_per_step": fms, "n_keep": nk,
            "round_bytes": fused_bytes,
            "kernel_ms": {"verify_with_replay_per_layer": fused["verify_replay_ms"],
                          "accept_and_conv_rollback": fused["accept_conv_ms"]},
            "roofline": roofline(verify_kernel_name(cfg, fused=True), fvb, fused["verify_replay_ms"],
                                 measured_traffic(cfg.name + "_fused"))}
    res = {"cfg": cfg, "rounds": rounds, "mode": mode, "input_sets": len(rbs)}
    if extras:
        if not cfg.is_tree:
            res["sample_accept"] = sample_accept_pass(cfg, rbs[0], stream, args.steps)
        if not args.no_sweep:
            with torch.cuda.stream(stream):
                res["rollback_sweep"] = rollback_sweep(cfg, rbs[0], stream)
    del rbs, shared, sets, base, S, cs, conv_w
    torch.cuda.empty_cache()
    return res


def summary(res, steps) -> dict:
    """The bench line's fields for one workload: the timed form's value and
    round time, both forms, accepted / committed rates and roofline."""
    cfg, rounds, mode = res["cfg"], res["rounds"], res["mode"]
    r = rounds[mode]
    ms = r["ms_per_step"]
    acc_tok = float(r["n_keep"].sum()) / steps
    unit = "nodes" if cfg.is_tree else "tokens"
    return {
        "value": r["value"], "unit": unit + "/s", "ms_per_step": ms, "round": mode,
        "accepted_tokens_per_s": acc_tok / (ms * 1e-3),
        "committed_tokens_per_s": (acc_tok + cfg.B) / (ms * 1e-3),
        "round_hbm_frac": r["round_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "round_algorithmic_bytes": r["round_bytes"],
        "kernel_ms": r["kernel_ms"],
        "roofline": r["roofline"],
        "rounds": {k: dict({"value": v["value"], "ms_per_step": v["ms_per_step"],
                            "kernel_ms": v["kernel_ms"],
                            "verify_kernel": v["roofline"]["kernel"],
                            "verify_bytes_per_launch": v["roofline"]["bytes_per_launch"],
                            "verify_roofline_frac": v["roofline"]["frac"],
                            "round_hbm_frac": v["round_bytes"] / (v["ms_per_step"] * 1e-3) / 1e9
                            / HBM_PEAK_GBS},
                           **({"rollback_hbm_frac": v["rollback_hbm_frac"]}
                              if "rollback_hbm_frac" in v else {}))
                   for k, v in rounds.items()},
    }


def config_fields(cfg, args, mode, n_sets) -> dict:
    return {"workload": cfg.name, "layers": cfg.L, "batch": cfg.B,
            "drafts" if not cfg.is_tree else "tree_nodes": cfg.T,
            "acceptance": (cfg.p_accept if cfg.law == "bernoulli" else cfg.law),
            "k_heads": cfg.Hk, "v_heads": cfg.Hv, "d_k": cfg.Dk, "d_v": cfg.Dv,
            "conv_kernel": cfg.K, "inputs": "bf16" if cfg.dtype == torch.bfloat16 else "f32",
            "state": "f32", "vocab": cfg.V, "hip_graph": not args.eager,
            "input_sets": n_sets, "round": mode}


def copy_bandwidth(n_bytes=1 << 30, reps=10) -> dict:
    """Device-to-device copy rate (read + write bytes / time), median of reps."""
    a = torch.empty(n_bytes // 4, device="cuda", dtype=torch.float32).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    del a, b
    torch.cuda.empty_cache()
    gbs = 2 * n_bytes / (ms * 1e-3) / 1e9
    return {"bytes_copied": n_bytes, "ms": ms, "GBps_read_plus_write": gbs,
            "frac_of_peak": gbs / HBM_PEAK_GBS}


def main():
    args = parse()
    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU only: this build runs on a single MI355X "
                         "and has no multi-GPU path (got --gpus %d)\n" % args.gpus)
        sys.exit(2)
    if not torch.cuda.is_available():
        sys.stderr.write("bench.py needs a GPU\n")
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return

    from speculative_decode_verify_gdn_amd import binding as gb
    from speculative_decode_verify_gdn_amd import workload as W
    gb.lib()  # fail loudly if the HIP library is missing

    cfg = W.CONFIGS[args.config]
    stream = torch.cuda.Stream()
    res = measure_workload(cfg, args, stream, extras=True)
    head = summary(res, args.steps)
    out = {
        "metric": "verified draft tokens/s per 30-layer GDN stack",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config_fields(cfg, args, res["mode"], res["input_sets"]),
    }
    out.update({k: v for k, v in head.items()
                if k not in ("value", "unit", "ms_per_step", "round")})
    for k in ("sample_accept", "rollback_sweep"):
        if k in res:
            out[k] = res[k]
    del res

    others = {}
    for cid in [int(c) for c in args.also.split(",") if c.strip()]:
        if cid == args.config:
            continue
        ocfg = W.CONFIGS[cid]
        print("bench: %s" % ocfg.name, file=sys.stderr, flush=True)
        ores = measure_workload(ocfg, args, stream, extras=not args.no_sweep)
        o = summary(ores, args.steps)
        o["config"] = config_fields(ocfg, args, ores["mode"], ores["input_sets"])
        if "rollback_sweep" in ores:
            o["rollback_sweep"] = ores["rollback_sweep"]
        if "sample_accept" in ores:
            o["sample_accept"] = ores["sample_accept"]
        others[ocfg.name] = o
        del ores
    if others:
        out["other_workloads"] = others

    if args.prefill > 0:
        out["prefill"] = prefill_pass(cfg, args.prefill, stream)
        if args.gate_per_key and not cfg.is_tree:
            out["prefill_per_key_gate"] = prefill_pass(cfg, args.prefill, stream,
                                                       gate_per_key=True)
    if args.gate_per_key:
        out["per_key_gate"] = vgate_pass(cfg, stream, args.steps)
    if args.draft_sweep and not cfg.is_tree:
        out["draft_policy"] = draft_sweep(cfg, stream)
    out["copy_bandwidth"] = copy_bandwidth()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = oracle_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
