"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

from speculative_decode_verify_gdn_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_verify.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gb.LIB_PATH):
        from speculative_decode_verify_gdn_amd import build
        build.build()
    return gb.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9]+)\s*\(", text,
                                 flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(gb.EXPORTS) <= set(names), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert gb.abi_version() == 8
    assert gb.status_string(0) == "GDN_OK"
    assert gb.status_string(1) == "GDN_ERR_INVALID_ARG"
    assert gb.status_string(4) == "GDN_ERR_WORKSPACE"
    assert gb.status_string(99) == "GDN_UNKNOWN_STATUS"


def test_workspace_size(lib):
    assert gb.spec_accept_workspace_bytes(32, 8, 151936) > 32 * 9 * 8
    assert gb.spec_accept_workspace_bytes(0, 8, 100) == 0
    assert gb.spec_accept_workspace_bytes(1, 65, 100) == 0


def _shape(**kw):
    d = dict(L=1, B=2, Hk=2, Hv=4, Dk=128, Dv=128, K=4)
    d.update(kw)
    return gb.GdnShape(**d).c()


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _verify(shape, T=4, null_x=False):
    tape = gb._CTape(FAKE.value, FAKE.value, FAKE.value)
    x = None if null_x else FAKE
    return gb.lib().gdn_verify_chunk(ctypes.byref(shape), T, x, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, ctypes.byref(tape), None)


def test_host_validation_before_launch(lib):
    assert _verify(_shape(), null_x=True) == gb.GDN_ERR_INVALID_ARG
    assert _verify(_shape(Hv=3)) == gb.GDN_ERR_INVALID_ARG          # Hv % Hk != 0
    assert _verify(_shape(), T=0) == gb.GDN_ERR_INVALID_ARG
    assert _verify(_shape(), T=65) == gb.GDN_ERR_UNSUPPORTED
    assert _verify(_shape(Dk=96, Dv=96)) == gb.GDN_ERR_UNSUPPORTED
    assert _verify(_shape(Dk=64, Dv=128)) == gb.GDN_ERR_UNSUPPORTED
    assert _verify(_shape(K=9)) == gb.GDN_ERR_UNSUPPORTED
    assert _verify(_shape(B=0)) == gb.GDN_ERR_INVALID_ARG
    # sizes whose grids or channel offsets would leave 32 bits
    assert _verify(_shape(L=64, B=1 << 12, Hk=64, Hv=512)) == gb.GDN_ERR_UNSUPPORTED
    assert _verify(_shape(Hk=1, Hv=1 << 22)) == gb.GDN_ERR_UNSUPPORTED
    assert _verify(_shape(Hk=1 << 21, Hv=1 << 21, B=1)) == gb.GDN_ERR_UNSUPPORTED
    # fused replay: previous tape missing, aliasing the current one, bad prev_T
    cur = gb._CTape(0x1000, 0x2000, 0x3000)
    prev = gb._CTape(0x4000, 0x5000, 0x6000)
    rv = lambda pT, pt, pn: lib.gdn_verify_chunk_replay(
        ctypes.byref(_shape()), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(cur),
        pT, pt, pn, None, None)
    assert rv(4, None, FAKE) == gb.GDN_ERR_INVALID_ARG
    assert rv(4, ctypes.byref(prev), None) == gb.GDN_ERR_INVALID_ARG
    assert rv(4, ctypes.byref(cur), FAKE) == gb.GDN_ERR_INVALID_ARG
    assert rv(0, ctypes.byref(prev), FAKE) == gb.GDN_ERR_INVALID_ARG
    assert rv(65, ctypes.byref(prev), FAKE) == gb.GDN_ERR_UNSUPPORTED
    # tree replay: no parent, previous tape missing or aliased, bad prev_T
    tv = lambda par, pT, pt, pn: lib.gdn_tree_verify_replay(
        ctypes.byref(_shape()), 40, par, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        ctypes.byref(cur), None, pT, pt, None, pn, None, None)
    assert tv(None, 40, ctypes.byref(prev), FAKE) == gb.GDN_ERR_INVALID_ARG
    assert tv(FAKE, 40, None, FAKE) == gb.GDN_ERR_INVALID_ARG
    assert tv(FAKE, 40, ctypes.byref(prev), None) == gb.GDN_ERR_INVALID_ARG
    assert tv(FAKE, 40, ctypes.byref(cur), FAKE) == gb.GDN_ERR_INVALID_ARG
    assert tv(FAKE, 0, ctypes.byref(prev), FAKE) == gb.GDN_ERR_INVALID_ARG
    assert tv(FAKE, 65, ctypes.byref(prev), FAKE) == gb.GDN_ERR_UNSUPPORTED
    tape = gb._CTape(FAKE.value, FAKE.value, None)
    assert lib.gdn_tape_rollback(ctypes.byref(_shape()), 4, FAKE, ctypes.byref(tape), None, FAKE,
                                 None, None) == gb.GDN_ERR_INVALID_ARG
    assert lib.gdn_conv_state_rollback(ctypes.byref(_shape()), 4, FAKE, FAKE, None, None, None,
                                       None, None) == gb.GDN_ERR_INVALID_ARG
    assert lib.gdn_tree_verify(ctypes.byref(_shape()), 4, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, FAKE, ctypes.byref(gb._CTape(1, 1, 1)), None, None,
                               None) == gb.GDN_ERR_INVALID_ARG
    # sampling accept: bad temperature, missing uniforms, short workspace
    sa = lambda T, tau, uni, ws, wsb: lib.spec_accept_sample(
        2, T, 100, FAKE, FAKE, gb.GDN_BF16, tau, uni, FAKE, FAKE, FAKE, ws, wsb, None, None)
    big = 1 << 24
    assert sa(4, 0.0, FAKE, FAKE, big) == gb.GDN_ERR_INVALID_ARG
    assert sa(4, -1.0, FAKE, FAKE, big) == gb.GDN_ERR_INVALID_ARG
    assert sa(4, float("inf"), FAKE, FAKE, big) == gb.GDN_ERR_INVALID_ARG
    assert sa(4, float("nan"), FAKE, FAKE, big) == gb.GDN_ERR_INVALID_ARG
    assert sa(4, 1e-40, FAKE, FAKE, big) == gb.GDN_ERR_INVALID_ARG  # 1/temperature overflows
    assert sa(4, 1.0, None, FAKE, big) == gb.GDN_ERR_INVALID_ARG
    assert sa(65, 1.0, FAKE, FAKE, big) == gb.GDN_ERR_UNSUPPORTED
    assert sa(4, 1.0, FAKE, FAKE, 8) == gb.GDN_ERR_WORKSPACE
    assert sa(4, 1.0, FAKE, None, big) == gb.GDN_ERR_WORKSPACE
    assert gb.spec_sample_workspace_bytes(32, 8, 151936) >= 32 * 9 * 38 * 8
    assert gb.spec_sample_workspace_bytes(1, 65, 100) == 0
    # per-key-channel gate: flag must be 0/1; the tree and replay calls take
    # it with the same host-side validation as the per-head form
    assert _verify(_shape(gate_per_key=2)) == gb.GDN_ERR_INVALID_ARG
    vg = _shape(gate_per_key=True)
    assert lib.gdn_tree_verify(ctypes.byref(vg), 40, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, ctypes.byref(gb._CTape(1, 1, 1)), None, None,
                               None) == gb.GDN_ERR_INVALID_ARG
    assert lib.gdn_tree_verify(ctypes.byref(vg), 65, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, ctypes.byref(gb._CTape(1, 1, 1)), None, None,
                               None) == gb.GDN_ERR_UNSUPPORTED
    assert lib.gdn_verify_chunk_replay(ctypes.byref(vg), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, ctypes.byref(cur), 65, ctypes.byref(prev), FAKE,
                                       None, None) == gb.GDN_ERR_UNSUPPORTED
    assert lib.gdn_verify_chunk_replay(ctypes.byref(vg), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, ctypes.byref(cur), 4, ctypes.byref(cur), FAKE,
                                       None, None) == gb.GDN_ERR_INVALID_ARG
    # prefill: bad T, missing pointers, short workspace
    pf = lambda T, xx, ws, wsb: lib.gdn_prefill(ctypes.byref(_shape()), T, xx, FAKE, FAKE, FAKE,
                                                FAKE, FAKE, FAKE, ws, wsb, None, None)
    wsb = gb.lib().gdn_prefill_workspace_bytes(ctypes.byref(_shape()))
    assert wsb > 0
    assert pf(0, FAKE, FAKE, wsb) == gb.GDN_ERR_INVALID_ARG
    assert pf(100, None, FAKE, wsb) == gb.GDN_ERR_INVALID_ARG
    assert pf(100, FAKE, FAKE, wsb - 1) == gb.GDN_ERR_WORKSPACE
    assert pf(100, FAKE, None, wsb) == gb.GDN_ERR_WORKSPACE
    assert lib.gdn_prefill(ctypes.byref(_shape(Dk=96, Dv=96)), 10, FAKE, FAKE, FAKE, FAKE, FAKE,
                           FAKE, FAKE, FAKE, wsb, None, None) == gb.GDN_ERR_UNSUPPORTED
    # workspace sizes: two 16-token tapes (u, k, g) per (layer, seq); the
    # one-launch loop (128-dim heads) keeps k rows per v-head, the chunked
    # form per k-head; the per-key gate's g has Dk entries per v-head, and
    # the per-key sequential kernel (fp32 inputs, other head sizes) none
    def wsize(**kw):
        return gb.lib().gdn_prefill_workspace_bytes(ctypes.byref(_shape(**kw)))

    def tapes(L, B, Hk, Hv, D, gdk, kh):
        fl = L * B * 16 * (Hv * D + kh * D + Hv * gdk)
        return 2 * ((fl * 4 + 255) // 256 * 256)

    assert wsize() == tapes(1, 2, 2, 4, 128, 1, 4)
    assert wsize(Dk=64, Dv=64) == tapes(1, 2, 2, 4, 64, 1, 2)
    assert wsize(gate_per_key=True) == tapes(1, 2, 2, 4, 128, 128, 4)
    import torch
    assert wsize(gate_per_key=True, dtype=torch.float32) == 0
    assert wsize(gate_per_key=True, Dk=64, Dv=64) == 0
    # accept: missing / short workspace, bad dtype
    assert lib.spec_accept_prefix(2, 4, 100, None, FAKE, FAKE, gb.GDN_BF16, FAKE, FAKE, FAKE,
                                  FAKE, 8, None, None) == gb.GDN_ERR_WORKSPACE
    assert lib.spec_accept_prefix(2, 4, 100, None, FAKE, FAKE, 7, FAKE, FAKE, FAKE, FAKE,
                                  1 << 20, None, None) == gb.GDN_ERR_INVALID_ARG
    assert lib.spec_accept_prefix(2, 4, 100, None, None, FAKE, gb.GDN_BF16, FAKE, FAKE, FAKE,
                                  FAKE, 1 << 20, None, None) == gb.GDN_ERR_INVALID_ARG


def test_binding_rejects_mismatched_tensors():
    import torch
    sh = gb.GdnShape(1, 1, 1, 1, 32, 32, 4, dtype=torch.float32)
    x = torch.zeros((1, 1, 4, sh.C))
    with pytest.raises((ValueError, TypeError)):
        gb._need(x, "x", torch.float32, (1, 1, 5, sh.C))
    with pytest.raises(TypeError):
        gb._need(x, "x", torch.bfloat16, (1, 1, 4, sh.C))
    with pytest.raises(ValueError):  # host tensor
        gb._need(x, "x", torch.float32, (1, 1, 4, sh.C))


def test_noalloc_accept_rejects_oversize_before_launch(lib):
    """spec_accept_prefix_noalloc refuses, on the host, inputs whose partials
    exceed the static scratch (B*(T+1) > 131040 rows for small vocabularies,
    > 13104 at V = 151936), and takes the ordinary argument checks first."""
    P = ctypes.c_void_p
    call = lambda B, T, V, d=FAKE: lib.spec_accept_prefix_noalloc(
        B, T, V, None, d, FAKE, gb.GDN_BF16, FAKE, FAKE, FAKE, None, None)
    assert call(2100, 63, 7) == gb.GDN_ERR_SCRATCH
    assert call(2017, 64, 7) == gb.GDN_ERR_SCRATCH      # 131105 rows
    assert gb.spec_accept_workspace_bytes(2017, 64, 7) > gb.ACCEPT_SCRATCH_BYTES
    assert gb.spec_accept_workspace_bytes(2016, 64, 7) == gb.ACCEPT_SCRATCH_BYTES  # 131040 rows
    # at the full vocabulary every row takes ten partials: 13104 rows fit
    assert gb.spec_accept_workspace_bytes(6552, 1, 151936) == gb.ACCEPT_SCRATCH_BYTES
    assert call(6553, 1, 151936) == gb.GDN_ERR_SCRATCH   # 13106 rows
    assert call(2, 4, 7, d=None) == gb.GDN_ERR_INVALID_ARG
    assert call(2, 65, 7) == gb.GDN_ERR_UNSUPPORTED
    assert gb.status_string(gb.GDN_ERR_SCRATCH) == "GDN_ERR_SCRATCH"
    del P
