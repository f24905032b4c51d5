"""ctypes binding of libgdnverify (include/gdn_verify.h) for torch tensors.

Argument marshalling only: every step runs in the HIP library.  Each call
checks on the host that the tensors it passes have the dtype, device,
contiguity and exact size the shape implies, because the kernels index them
by those sizes.  Nothing here computes anything of the method, and there is
no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdnverify.so")

(GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_LAUNCH, GDN_ERR_WORKSPACE,
 GDN_ERR_SCRATCH) = range(6)
ACCEPT_SCRATCH_BYTES = 1 << 20  # GDN_ACCEPT_SCRATCH_BYTES
GDN_F32, GDN_BF16 = 0, 1
DEV_ERR_N_KEEP, DEV_ERR_PARENT, DEV_ERR_PATH, DEV_ERR_TOKEN, DEV_ERR_NAN = 1, 2, 4, 8, 16

EXPORTS = ("gdn_verify_chunk", "gdn_verify_chunk_replay", "gdn_tree_verify",
           "gdn_tree_verify_replay", "spec_accept_prefix", "spec_accept_prefix_noalloc",
           "spec_accept_sample",
           "spec_sample_workspace_bytes", "gdn_prefill", "gdn_prefill_workspace_bytes",
           "gdn_round_rollback",
           "spec_accept_workspace_bytes", "gdn_tape_rollback", "gdn_conv_state_rollback",
           "gdn_status_string", "gdn_abi_version")


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s" % (what, status_string(status)))
        self.status = status


class _CShape(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("n_k_heads", ctypes.c_int32), ("n_v_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("conv_kernel", ctypes.c_int32), ("conv_silu", ctypes.c_int32),
                ("l2_eps", ctypes.c_float), ("in_dtype", ctypes.c_int32),
                ("gate_per_key", ctypes.c_int32)]


class _CTape(ctypes.Structure):
    _fields_ = [("u", ctypes.c_void_p), ("k", ctypes.c_void_p), ("g", ctypes.c_void_p)]


@dataclass(frozen=True)
class GdnShape:
    """Mirror of gdn_shape.  C = 2*Hk*Dk + Hv*Dv qkv channels."""
    L: int
    B: int
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    K: int
    silu: bool = True
    eps: float = 1e-6
    dtype: torch.dtype = torch.bfloat16
    gate_per_key: bool = False  # decay a / tape g per key channel: [..,Hv,Dk]

    @property
    def C(self) -> int:
        return 2 * self.Hk * self.Dk + self.Hv * self.Dv

    def c(self) -> _CShape:
        if self.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("input dtype must be float32 or bfloat16")
        return _CShape(self.L, self.B, self.Hk, self.Hv, self.Dk, self.Dv, self.K,
                       int(self.silu), float(self.eps),
                       GDN_BF16 if self.dtype == torch.bfloat16 else GDN_F32,
                       int(self.gate_per_key))

    def gate_shape(self, T: int) -> tuple:
        """Shape of the decay gate a and of the tape's g for T tokens."""
        return ((self.L, self.B, T, self.Hv, self.Dk) if self.gate_per_key
                else (self.L, self.B, T, self.Hv))


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgdnverify.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdnverify.so is not built; run "
                               "`python -m speculative_decode_verify_gdn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        SP, TP = ctypes.POINTER(_CShape), ctypes.POINTER(_CTape)
        L.gdn_verify_chunk.argtypes = [SP, I32, P, P, P, P, P, P, P, TP, P]
        L.gdn_verify_chunk_replay.argtypes = [SP, I32, P, P, P, P, P, P, P, TP, I32, TP, P, P, P]
        L.gdn_tree_verify.argtypes = [SP, I32, P, P, P, P, P, P, P, P, TP, P, P, P]
        L.gdn_tree_verify_replay.argtypes = [SP, I32, P, P, P, P, P, P, P, P, TP, P, I32, TP, P,
                                             P, P, P]
        L.spec_accept_prefix.argtypes = [I32, I32, I32, P, P, P, I32, P, P, P, P, SZ, P, P]
        L.spec_accept_prefix_noalloc.argtypes = [I32, I32, I32, P, P, P, I32, P, P, P, P, P]
        L.spec_accept_workspace_bytes.argtypes = [I32, I32, I32]
        L.spec_accept_workspace_bytes.restype = SZ
        L.spec_accept_sample.argtypes = [I32, I32, I32, P, P, I32, ctypes.c_float, P, P, P, P, P,
                                         SZ, P, P]
        L.spec_sample_workspace_bytes.argtypes = [I32, I32, I32]
        L.spec_sample_workspace_bytes.restype = SZ
        L.gdn_prefill.argtypes = [SP, I32, P, P, P, P, P, P, P, P, SZ, P, P]
        L.gdn_prefill_workspace_bytes.argtypes = [SP]
        L.gdn_prefill_workspace_bytes.restype = SZ
        L.gdn_tape_rollback.argtypes = [SP, I32, P, TP, P, P, P, P]
        L.gdn_round_rollback.argtypes = [SP, I32, P, TP, P, P, P, P, P, P, P]
        L.gdn_conv_state_rollback.argtypes = [SP, I32, P, P, P, P, P, P, P]
        L.gdn_status_string.argtypes = [I32]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        for name in ("gdn_verify_chunk", "gdn_verify_chunk_replay", "gdn_tree_verify",
                     "gdn_tree_verify_replay", "spec_accept_prefix",
                     "spec_accept_prefix_noalloc", "spec_accept_sample",
                     "gdn_prefill", "gdn_round_rollback",
                     "gdn_tape_rollback", "gdn_conv_state_rollback", "gdn_abi_version"):
            getattr(L, name).restype = I32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().gdn_abi_version())


def _check(status: int, what: str):
    if status != GDN_OK:
        raise GdnError(status, what)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(device, *tensors):
    for t in tensors:
        if t is not None and t.device != device:
            raise ValueError("all tensors must be on %s (got %s)" % (device, t.device))


def _need(t: torch.Tensor, name: str, dtype, shape, align: int = 16):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.data_ptr() % align:
        raise ValueError("%s must be %d-byte aligned" % (name, align))
    return t.data_ptr()


def _opt(t, name, dtype, shape, align: int = 4):
    return None if t is None else _need(t, name, dtype, shape, align)


@dataclass
class Tape:
    """Innovation tape: u [L,B,T,Hv,Dv], k [L,B,T,Hk,Dk], g [L,B,T,Hv]
    ([L,B,T,Hv,Dk] with a per-key-channel gate), all fp32."""
    u: torch.Tensor
    k: torch.Tensor
    g: torch.Tensor

    @staticmethod
    def empty(sh: GdnShape, T: int, device="cuda") -> "Tape":
        f = dict(device=device, dtype=torch.float32)
        return Tape(torch.empty((sh.L, sh.B, T, sh.Hv, sh.Dv), **f),
                    torch.empty((sh.L, sh.B, T, sh.Hk, sh.Dk), **f),
                    torch.empty(sh.gate_shape(T), **f))

    def c(self, sh: GdnShape, T: int) -> _CTape:
        return _CTape(_need(self.u, "tape.u", torch.float32, (sh.L, sh.B, T, sh.Hv, sh.Dv)),
                      _need(self.k, "tape.k", torch.float32, (sh.L, sh.B, T, sh.Hk, sh.Dk)),
                      _need(self.g, "tape.g", torch.float32, sh.gate_shape(T), 4))


def _verify_ptrs(sh: GdnShape, T: int, x, conv_state, conv_w, a, b, S, o):
    dt = sh.dtype
    return [_need(x, "x", dt, (sh.L, sh.B, T, sh.C)),
            _need(conv_state, "conv_state", dt, (sh.L, sh.B, sh.K - 1, sh.C)),
            _need(conv_w, "conv_w", torch.float32, (sh.L, sh.C, sh.K)),
            _need(a, "a", dt, sh.gate_shape(T), 2),
            _need(b, "b", dt, (sh.L, sh.B, T, sh.Hv), 2),
            _need(S, "S", torch.float32, (sh.L, sh.B, sh.Hv, sh.Dv, sh.Dk)),
            _need(o, "o", torch.float32, (sh.L, sh.B, T, sh.Hv, sh.Dv))]


def gdn_verify_chunk(sh: GdnShape, x, conv_state, conv_w, a, b, S, o, tape: Tape, stream=None):
    """Verify the chain of T = x.shape[2] drafted tokens; S and conv_state are read only."""
    T = int(x.shape[2])
    ptrs = _verify_ptrs(sh, T, x, conv_state, conv_w, a, b, S, o)
    _dev(x.device, conv_state, conv_w, a, b, S, o, tape.u, tape.k, tape.g)
    ct = tape.c(sh, T)
    _check(lib().gdn_verify_chunk(ctypes.byref(sh.c()), T, *ptrs, ctypes.byref(ct),
                                  _stream(stream)), "gdn_verify_chunk")


def gdn_verify_chunk_replay(sh: GdnShape, x, conv_state, conv_w, a, b, S, o, tape: Tape,
                            prev_tape: Tape, prev_n_keep, dev_err=None, stream=None):
    """Replay the previous round's accepted prefix (prev_tape, prev_n_keep)
    onto S in place, then verify the chain of T = x.shape[2] tokens from it."""
    T = int(x.shape[2])
    pT = int(prev_tape.g.shape[2])
    ptrs = _verify_ptrs(sh, T, x, conv_state, conv_w, a, b, S, o)
    _dev(x.device, conv_state, conv_w, a, b, S, o, tape.u, tape.k, tape.g, prev_tape.u,
         prev_tape.k, prev_tape.g, prev_n_keep, dev_err)
    ct = tape.c(sh, T)
    pt = prev_tape.c(sh, pT)
    pn = _need(prev_n_keep, "prev_n_keep", torch.int32, (sh.B,), 4)
    de = _opt(dev_err, "dev_err", torch.int32, (1,))
    _check(lib().gdn_verify_chunk_replay(ctypes.byref(sh.c()), T, *ptrs, ctypes.byref(ct), pT,
                                         ctypes.byref(pt), pn, de, _stream(stream)),
           "gdn_verify_chunk_replay")


def gdn_tree_verify(sh: GdnShape, parent, x, conv_state, conv_w, a, b, S, o, tape: Tape,
                    conv_win=None, dev_err=None, stream=None):
    """Verify a T-node draft tree per sequence (parent [B,T] int32)."""
    T = int(x.shape[2])
    pp = _need(parent, "parent", torch.int32, (sh.B, T), 4)
    ptrs = _verify_ptrs(sh, T, x, conv_state, conv_w, a, b, S, o)
    cw = _opt(conv_win, "conv_win", torch.int32, (sh.B, T, sh.K))
    de = _opt(dev_err, "dev_err", torch.int32, (1,))
    _dev(x.device, parent, conv_state, conv_w, a, b, S, o, tape.u, tape.k, tape.g, conv_win,
         dev_err)
    ct = tape.c(sh, T)
    _check(lib().gdn_tree_verify(ctypes.byref(sh.c()), T, pp, *ptrs, ctypes.byref(ct), cw, de,
                                 _stream(stream)), "gdn_tree_verify")


def gdn_prefill_workspace_bytes(sh: GdnShape) -> int:
    return int(lib().gdn_prefill_workspace_bytes(ctypes.byref(sh.c())))


def gdn_prefill(sh: GdnShape, x, conv_state, conv_w, a, b, S, o, workspace, dev_err=None,
                stream=None):
    """Run T = x.shape[2] tokens through the layers and commit them: S and
    conv_state are updated in place, o receives every token's output."""
    T = int(x.shape[2])
    ptrs = _verify_ptrs(sh, T, x, conv_state, conv_w, a, b, S, o)
    need = gdn_prefill_workspace_bytes(sh)
    if need == 0 and workspace is None:
        wp, wn = None, 0
    elif (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8
            or workspace.numel() < need or not workspace.is_cuda
            or not workspace.is_contiguous() or workspace.data_ptr() % 256):
        raise ValueError("workspace must be a 256-byte aligned device uint8 tensor of >= %d bytes"
                         % need)
    else:
        wp, wn = workspace.data_ptr(), workspace.numel()
    de = _opt(dev_err, "dev_err", torch.int32, (1,))
    _dev(x.device, conv_state, conv_w, a, b, S, o, workspace, dev_err)
    _check(lib().gdn_prefill(ctypes.byref(sh.c()), T, *ptrs, wp, wn, de, _stream(stream)),
           "gdn_prefill")


def gdn_tree_verify_replay(sh: GdnShape, parent, x, conv_state, conv_w, a, b, S, o, tape: Tape,
                           prev_tape: Tape, prev_n_keep, prev_path=None, conv_win=None,
                           dev_err=None, stream=None):
    """Replay the previous round's accepted path (prev_tape, prev_path,
    prev_n_keep) onto S in place, then verify the T-node tree from it."""
    T = int(x.shape[2])
    pT = int(prev_tape.g.shape[2])
    pp = _need(parent, "parent", torch.int32, (sh.B, T), 4)
    ptrs = _verify_ptrs(sh, T, x, conv_state, conv_w, a, b, S, o)
    cw = _opt(conv_win, "conv_win", torch.int32, (sh.B, T, sh.K))
    de = _opt(dev_err, "dev_err", torch.int32, (1,))
    pn = _need(prev_n_keep, "prev_n_keep", torch.int32, (sh.B,), 4)
    ppath = _opt(prev_path, "prev_path", torch.int32, (sh.B, pT))
    _dev(x.device, parent, conv_state, conv_w, a, b, S, o, tape.u, tape.k, tape.g, prev_tape.u,
         prev_tape.k, prev_tape.g, prev_n_keep, prev_path, conv_win, dev_err)
    ct = tape.c(sh, T)
    pt = prev_tape.c(sh, pT)
    _check(lib().gdn_tree_verify_replay(ctypes.byref(sh.c()), T, pp, *ptrs, ctypes.byref(ct), cw,
                                        pT, ctypes.byref(pt), ppath, pn, de, _stream(stream)),
           "gdn_tree_verify_replay")


def spec_accept_workspace_bytes(B: int, T: int, V: int) -> int:
    return int(lib().spec_accept_workspace_bytes(B, T, V))


def spec_accept_prefix(draft, logits, n_keep, path, bonus, workspace, parent=None, dev_err=None,
                       stream=None):
    """Greedy chain (parent=None) or tree acceptance; outputs stay on the device."""
    B, T = int(draft.shape[0]), int(draft.shape[1])
    V = int(logits.shape[-1])
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("logits must be float32 or bfloat16")
    lp = _need(logits, "logits", logits.dtype, (B, T + 1, V))
    dp = _need(draft, "draft", torch.int32, (B, T), 4)
    pp = _opt(parent, "parent", torch.int32, (B, T))
    need = spec_accept_workspace_bytes(B, T, V)
    if (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8
            or workspace.numel() < need or not workspace.is_cuda
            or not workspace.is_contiguous()):
        raise ValueError("workspace must be a device uint8 tensor of >= %d bytes" % need)
    args = [_need(n_keep, "n_keep", torch.int32, (B,), 4),
            _need(path, "path", torch.int32, (B, T), 4),
            _need(bonus, "bonus", torch.int32, (B,), 4)]
    de = _opt(dev_err, "dev_err", torch.int32, (1,))
    _dev(draft.device, logits, n_keep, path, bonus, workspace, parent, dev_err)
    _check(lib().spec_accept_prefix(B, T, V, pp, dp, lp,
                                    GDN_BF16 if logits.dtype == torch.bfloat16 else GDN_F32,
                                    *args, workspace.data_ptr(), workspace.numel(), de,
                                    _stream(stream)), "spec_accept_prefix")


def spec_accept_prefix_noalloc(draft, logits, n_keep, path, bonus, parent=None, dev_err=None,
                               stream=None):
    """spec_accept_prefix with the library's static scratch instead of a
    workspace (no device allocation anywhere in the call)."""
    B, T = int(draft.shape[0]), int(draft.shape[1])
    V = int(logits.shape[-1])
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("logits must be float32 or bfloat16")
    lp = _need(logits, "logits", logits.dtype, (B, T + 1, V))
    dp = _need(draft, "draft", torch.int32, (B, T), 4)
    pp = _opt(parent, "parent", torch.int32, (B, T))
    args = [_need(n_keep, "n_keep", torch.int32, (B,), 4),
            _need(path, "path", torch.int32, (B, T), 4),
            _need(bonus, "bonus", torch.int32, (B,), 4)]
    de = _opt(dev_err, "dev_err", torch.int32, (1,))
    _dev(draft.device, logits, n_keep, path, bonus, parent, dev_err)
    _check(lib().spec_accept_prefix_noalloc(B, T, V, pp, dp, lp,
                                            GDN_BF16 if logits.dtype == torch.bfloat16
                                            else GDN_F32, *args, de, _stream(stream)),
           "spec_accept_prefix_noalloc")


def spec_sample_workspace_bytes(B: int, T: int, V: int) -> int:
    return int(lib().spec_sample_workspace_bytes(B, T, V))


def spec_accept_sample(draft, logits, temperature: float, uniforms, n_keep, path, token,
                       workspace, dev_err=None, stream=None):
    """Rejection-sampling acceptance of a draft chain at temperature > 0
    (uniforms [B, T+1] fp32 in [0, 1)); outputs stay on the device."""
    B, T = int(draft.shape[0]), int(draft.shape[1])
    V = int(logits.shape[-1])
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("logits must be float32 or bfloat16")
    lp = _need(logits, "logits", logits.dtype, (B, T + 1, V))
    dp = _need(draft, "draft", torch.int32, (B, T), 4)
    up = _need(uniforms, "uniforms", torch.float32, (B, T + 1), 4)
    need = spec_sample_workspace_bytes(B, T, V)
    if (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8
            or workspace.numel() < need or not workspace.is_cuda
            or not workspace.is_contiguous()):
        raise ValueError("workspace must be a device uint8 tensor of >= %d bytes" % need)
    args = [_need(n_keep, "n_keep", torch.int32, (B,), 4),
            _need(path, "path", torch.int32, (B, T), 4),
            _need(token, "token", torch.int32, (B,), 4)]
    de = _opt(dev_err, "dev_err", torch.int32, (1,))
    _dev(draft.device, logits, uniforms, n_keep, path, token, workspace, dev_err)
    _check(lib().spec_accept_sample(B, T, V, dp, lp,
                                    GDN_BF16 if logits.dtype == torch.bfloat16 else GDN_F32,
                                    float(temperature), up, *args, workspace.data_ptr(),
                                    workspace.numel(), de, _stream(stream)),
           "spec_accept_sample")


def gdn_round_rollback(sh: GdnShape, S, tape: Tape, conv_state, x, n_keep, path=None,
                       win_idx=None, dev_err=None, stream=None):
    """gdn_tape_rollback + gdn_conv_state_rollback in one call (one launch
    where the library can)."""
    T = int(tape.g.shape[2])
    dt = sh.dtype
    sp = _need(S, "S", torch.float32, (sh.L, sh.B, sh.Hv, sh.Dv, sh.Dk))
    ct = tape.c(sh, T)
    cp = _need(conv_state, "conv_state", dt, (sh.L, sh.B, sh.K - 1, sh.C))
    xp = _need(x, "x", dt, (sh.L, sh.B, T, sh.C))
    np_ = _need(n_keep, "n_keep", torch.int32, (sh.B,), 4)
    pp = _opt(path, "path", torch.int32, (sh.B, T))
    wi = _opt(win_idx, "win_idx", torch.int32, (sh.B, sh.K - 1))
    de = _opt(dev_err, "dev_err", torch.int32, (1,))
    _dev(S.device, tape.u, tape.k, tape.g, conv_state, x, n_keep, path, win_idx, dev_err)
    _check(lib().gdn_round_rollback(ctypes.byref(sh.c()), T, sp, ctypes.byref(ct), cp, xp, pp,
                                    np_, wi, de, _stream(stream)), "gdn_round_rollback")


def gdn_tape_rollback(sh: GdnShape, S, tape: Tape, n_keep, path=None, dev_err=None, stream=None):
    """Replay the accepted tape entries onto the snapshot S in place."""
    T = int(tape.g.shape[2])
    sp = _need(S, "S", torch.float32, (sh.L, sh.B, sh.Hv, sh.Dv, sh.Dk))
    ct = tape.c(sh, T)
    np_ = _need(n_keep, "n_keep", torch.int32, (sh.B,), 4)
    pp = _opt(path, "path", torch.int32, (sh.B, T))
    de = _opt(dev_err, "dev_err", torch.int32, (1,))
    _dev(S.device, tape.u, tape.k, tape.g, n_keep, path, dev_err)
    _check(lib().gdn_tape_rollback(ctypes.byref(sh.c()), T, sp, ctypes.byref(ct), pp, np_, de,
                                   _stream(stream)), "gdn_tape_rollback")


def gdn_conv_state_rollback(sh: GdnShape, conv_state, x, n_keep, path=None, win_idx=None,
                            dev_err=None, stream=None):
    """Rebuild the conv window in place from the accepted raw rows of x."""
    T = int(x.shape[2])
    cp = _need(conv_state, "conv_state", sh.dtype, (sh.L, sh.B, sh.K - 1, sh.C))
    xp = _need(x, "x", sh.dtype, (sh.L, sh.B, T, sh.C))
    np_ = _need(n_keep, "n_keep", torch.int32, (sh.B,), 4)
    pp = _opt(path, "path", torch.int32, (sh.B, T))
    wp = _opt(win_idx, "win_idx", torch.int32, (sh.B, sh.K - 1))
    de = _opt(dev_err, "dev_err", torch.int32, (1,))
    _dev(conv_state.device, x, n_keep, path, win_idx, dev_err)
    _check(lib().gdn_conv_state_rollback(ctypes.byref(sh.c()), T, cp, xp, pp, np_, wp, de,
                                         _stream(stream)), "gdn_conv_state_rollback")
