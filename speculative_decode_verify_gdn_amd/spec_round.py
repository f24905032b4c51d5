"""One speculative round through a GDN layer stack, as calls into the C ABI.

A round is: per layer, verify the drafted chain (or tree) reading the live
state and conv window as the snapshot; accept the greedy prefix (or tree
path) from the target logits; then roll the whole stack back in two calls,
the state by tape replay and the conv window by re-gathering the accepted raw
rows ("Speculative Decoding on GDN Hybrid Architectures", s4; accept rule:
xserv "Phase 25", s2).  Nothing in a round synchronises with the host: the
accepted lengths and paths stay on the device between the calls.

This module only orders the calls and owns the device buffers; all
arithmetic happens in libgdnverify.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import torch

from . import binding as gb


@dataclass
class RoundBuffers:
    """Device buffers of one layer stack for chunks / trees of T nodes."""
    sh: gb.GdnShape
    T: int
    V: int
    tree: bool
    S: torch.Tensor            # [L,B,Hv,Dv,Dk] live state (= snapshot during verify)
    conv_state: torch.Tensor   # [L,B,K-1,C] live conv window
    conv_w: torch.Tensor       # [L,C,K]
    x: torch.Tensor            # [L,B,T,C] drafted raw qkv (also the tape's qkv entry)
    a: torch.Tensor            # [L,B,T,Hv]
    b: torch.Tensor            # [L,B,T,Hv]
    logits: torch.Tensor       # [B,T+1,V]
    draft: torch.Tensor        # [B,T] int32
    parent: Optional[torch.Tensor]  # [B,T] int32 for trees
    o: torch.Tensor = None
    tape: gb.Tape = None
    n_keep: torch.Tensor = None
    path: torch.Tensor = None
    bonus: torch.Tensor = None
    workspace: torch.Tensor = None
    win_idx: torch.Tensor = None
    conv_win: Optional[torch.Tensor] = None
    dev_err: torch.Tensor = None
    layer_shape: gb.GdnShape = field(init=False)

    def __post_init__(self):
        sh, T, dev = self.sh, self.T, self.S.device
        f32 = dict(device=dev, dtype=torch.float32)
        i32 = dict(device=dev, dtype=torch.int32)
        if self.o is None:
            self.o = torch.empty((sh.L, sh.B, T, sh.Hv, sh.Dv), **f32)
        if self.tape is None:
            self.tape = gb.Tape.empty(sh, T, dev)
        self.n_keep = torch.zeros((sh.B,), **i32)
        self.path = torch.full((sh.B, T), -1, **i32)
        self.bonus = torch.zeros((sh.B,), **i32)
        self.workspace = torch.empty((gb.spec_accept_workspace_bytes(sh.B, T, self.V),),
                                     device=dev, dtype=torch.uint8)
        self.win_idx = torch.zeros((sh.B, sh.K - 1), **i32)
        if self.tree and self.conv_win is None:
            self.conv_win = torch.zeros((sh.B, T, sh.K), **i32)
        self.dev_err = torch.zeros((1,), **i32)
        self.layer_shape = dataclasses.replace(sh, L=1)

    def layer_tape(self, l: int) -> gb.Tape:
        return gb.Tape(self.tape.u[l:l + 1], self.tape.k[l:l + 1], self.tape.g[l:l + 1])


def verify_layer(rb: RoundBuffers, l: int, stream=None):
    """Verify layer l (one C-ABI call; S and conv_state are not written)."""
    sl = slice(l, l + 1)
    if rb.tree:
        gb.gdn_tree_verify(rb.layer_shape, rb.parent, rb.x[sl], rb.conv_state[sl],
                           rb.conv_w[sl], rb.a[sl], rb.b[sl], rb.S[sl], rb.o[sl],
                           rb.layer_tape(l), conv_win=rb.conv_win if l == 0 else None,
                           dev_err=rb.dev_err, stream=stream)
    else:
        gb.gdn_verify_chunk(rb.layer_shape, rb.x[sl], rb.conv_state[sl], rb.conv_w[sl],
                            rb.a[sl], rb.b[sl], rb.S[sl], rb.o[sl], rb.layer_tape(l),
                            stream=stream)


def accept(rb: RoundBuffers, stream=None):
    gb.spec_accept_prefix(rb.draft, rb.logits, rb.n_keep, rb.path, rb.bonus, rb.workspace,
                          parent=rb.parent if rb.tree else None, dev_err=rb.dev_err,
                          stream=stream)


def rollback(rb: RoundBuffers, stream=None):
    """Tape-replay the state and rebuild the conv window for all layers (one
    call; one launch where the library can)."""
    path = rb.path if rb.tree else None
    gb.gdn_round_rollback(rb.sh, rb.S, rb.tape, rb.conv_state, rb.x, rb.n_keep, path=path,
                          win_idx=rb.win_idx, dev_err=rb.dev_err, stream=stream)


def run_round(rb: RoundBuffers, stream=None):
    """verify (per layer) -> accept -> rollback, all enqueued on one stream."""
    for l in range(rb.sh.L):
        verify_layer(rb, l, stream)
    accept(rb, stream)
    rollback(rb, stream)


def fused_pays(sh: gb.GdnShape, T: int, tree: bool, device=None) -> bool:
    """Whether rounds should fold the state rollback into the next verify.

    The fused verify writes the replayed state back from inside the verify.
    When the verify grid fits the chip in about one pass, every workgroup
    streams its state at once and the kernel is latency bound: the extra
    writes land on that critical path.  The chain kernel (chains of at most
    16 drafts) puts the sequences that replay first in its workgroup order,
    so that one pass spreads them evenly over the CUs; with that, the fused
    round is faster at one pass too (30-layer stack, B = 32, 8 drafts:
    0.865 against 0.879 ms per round), and from two passes of workgroups on
    the writes overlap other workgroups' loads anyway.  The tree kernel
    (trees of 17..64 nodes, bf16 inputs, 128-dim heads) takes one workgroup
    per CU per pass and fuses from two passes on: below that, the separate
    rollback, a single launch over all layers that streams at a much higher
    fraction of HBM bandwidth, costs less than the writes on the verify's
    critical path.  Other shapes are not fused by the library.

    With the decay gate per key channel, chains of at most 16 drafts (bf16
    inputs, 128-dim heads) fuse from two passes of workgroups on: at one pass
    the per-key replay's gate products keep the verify at 34 against 22 us
    per layer and the fused round is the slower one (1.065 against 0.964 ms
    at B = 32, 8 drafts).  Trees of 13..64 nodes (the per-key form of the
    tree kernel) follow the per-head tree rule.  Other chains
    would fuse on the closed-form per-key kernel, slower than their plain
    verify, so they stay plain.  Other trees run the closed-form kernel in
    both forms, and folding the rollback in saves its state pass."""
    cus = torch.cuda.get_device_properties(device or torch.cuda.current_device()).multi_processor_count
    if sh.gate_per_key:
        mfma = sh.dtype == torch.bfloat16 and sh.Dk == sh.Dv == 128
        if not tree:
            return mfma and T <= 16 and sh.B * sh.Hv >= 2 * 4 * cus
        if mfma and 12 < T <= 64:
            return sh.B * sh.Hv >= 2 * cus
        return T <= 64
    if not tree:
        # the replaying sequences go first only for batches of at most 256
        return T <= 16 and (sh.B <= 256 or sh.B * sh.Hv >= 2 * 4 * cus)
    tree_kernel = 16 < T <= 64 and sh.dtype == torch.bfloat16 and sh.Dk == sh.Dv == 128
    return tree_kernel and sh.B * sh.Hv >= 2 * cus


@dataclass
class FusedRound:
    """Rounds with each layer's state rollback folded into the next round's
    verify of that layer (gdn_verify_chunk_replay, gdn_tree_verify_replay).
    Two tapes and two sets of accepted lengths (and, for trees, paths)
    alternate: round r writes tape[r % 2] and n_keep[r % 2] and replays
    tape[(r - 1) % 2] with n_keep[(r - 1) % 2].  Between rounds the live state
    lags one accepted prefix behind; finish() applies the last one with
    gdn_tape_rollback.  The conv window is rolled back every round (the next
    verify reads it as its snapshot).  Several FusedRound objects over
    different input buffers may share `tapes`, `n_keeps` and `paths`."""
    rb: RoundBuffers
    tapes: list = None
    n_keeps: list = None
    paths: list = None

    def __post_init__(self):
        rb = self.rb
        if self.tapes is None:
            self.tapes = [rb.tape, gb.Tape.empty(rb.sh, rb.T, rb.S.device)]
        if self.n_keeps is None:
            self.n_keeps = [rb.n_keep, torch.zeros_like(rb.n_keep)]
        if self.paths is None:
            self.paths = [rb.path, torch.full_like(rb.path, -1)]

    def verify_layers(self, r: int, stream=None, first: bool = False):
        """Every layer's verify of round r, replaying round r-1's prefix first
        (r = 0 with first=True has nothing to replay)."""
        rb, cur, prev = self.rb, r % 2, (r + 1) % 2
        tape, ptape = self.tapes[cur], self.tapes[prev]
        for l in range(rb.sh.L):
            sl = slice(l, l + 1)
            lt = gb.Tape(tape.u[sl], tape.k[sl], tape.g[sl])
            pt = gb.Tape(ptape.u[sl], ptape.k[sl], ptape.g[sl])
            if rb.tree:
                cw = rb.conv_win if l == 0 else None
                args = (rb.layer_shape, rb.parent, rb.x[sl], rb.conv_state[sl], rb.conv_w[sl],
                        rb.a[sl], rb.b[sl], rb.S[sl], rb.o[sl], lt)
                if first:
                    gb.gdn_tree_verify(*args, conv_win=cw, dev_err=rb.dev_err, stream=stream)
                else:
                    gb.gdn_tree_verify_replay(*args, pt, self.n_keeps[prev],
                                              prev_path=self.paths[prev], conv_win=cw,
                                              dev_err=rb.dev_err, stream=stream)
            elif first:
                gb.gdn_verify_chunk(rb.layer_shape, rb.x[sl], rb.conv_state[sl], rb.conv_w[sl],
                                    rb.a[sl], rb.b[sl], rb.S[sl], rb.o[sl], lt, stream=stream)
            else:
                gb.gdn_verify_chunk_replay(rb.layer_shape, rb.x[sl], rb.conv_state[sl],
                                           rb.conv_w[sl], rb.a[sl], rb.b[sl], rb.S[sl],
                                           rb.o[sl], lt, pt, self.n_keeps[prev],
                                           dev_err=rb.dev_err, stream=stream)

    def accept_and_conv(self, r: int, stream=None):
        """Greedy accept into n_keep[r % 2] (and path[r % 2]), then the
        conv-window rollback."""
        rb, nk, path = self.rb, self.n_keeps[r % 2], self.paths[r % 2]
        gb.spec_accept_prefix(rb.draft, rb.logits, nk, path, rb.bonus, rb.workspace,
                              parent=rb.parent if rb.tree else None, dev_err=rb.dev_err,
                              stream=stream)
        gb.gdn_conv_state_rollback(rb.sh, rb.conv_state, rb.x, nk,
                                   path=path if rb.tree else None, win_idx=rb.win_idx,
                                   dev_err=rb.dev_err, stream=stream)

    def round(self, r: int, stream=None, first: bool = False):
        """Round r: verify (with the previous round's replay), accept, conv rollback."""
        self.verify_layers(r, stream, first)
        self.accept_and_conv(r, stream)

    def finish(self, r: int, stream=None):
        """Apply round r's accepted prefix to the state (after the last round)."""
        cur = r % 2
        gb.gdn_tape_rollback(self.rb.sh, self.rb.S, self.tapes[cur], self.n_keeps[cur],
                             path=self.paths[cur] if self.rb.tree else None,
                             dev_err=self.rb.dev_err, stream=stream)
