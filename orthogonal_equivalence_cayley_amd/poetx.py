"""ctypes binding of libpoetx (include/poetx.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libpoetx.so. torch supplies device memory (tensor data pointers) and the
stream (torch.cuda.current_stream()). The module raises at import time if the
built library is missing; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpoetx.so")

POETX_OK = 0
POETX_ERR_INVALID_ARG = 1
POETX_ERR_SHAPE = 2
POETX_ERR_DTYPE = 3
POETX_ERR_ALIGNMENT = 4
POETX_ERR_UNSUPPORTED = 5
POETX_ERR_HIP = 6
POETX_ERR_WORKSPACE = 7

POETX_FP32 = 0
POETX_BF16 = 1
SIDE_R = 0
SIDE_P = 1
WS_BUILD = 0
WS_FORWARD = 1
WS_BACKWARD = 2
WS_PARAM_GRAD = 3
WS_MERGE = 4

WEIGHT_DENSE = 0
WEIGHT_INT8_ROWS = 1
WEIGHT_DENSE_T = 2
WEIGHT_INT8_ROWS_T = 3

CAYLEY_NEUMANN = 0
CAYLEY_EXACT = 1

FOLD_NONE = 0
FOLD_WEIGHT = 1

INDEX_SEPARATE = 0
INDEX_FUSED = 1

SERIES_CHAIN = 0
SERIES_PS = 1

EXPORTED = (
    "poetx_plan_create", "poetx_plan_destroy", "poetx_param_count", "poetx_block_elems",
    "poetx_workspace_size", "poetx_status_string", "poetx_last_hip_error", "poetx_permute_weight",
    "poetx_merge_weight", "poetx_weight_bytes", "poetx_quantize_weight",
    "poetx_build_orth", "poetx_build_orth_batch", "poetx_forward", "poetx_backward",
    "poetx_backward_dq", "poetx_param_grad_batch", "poetx_gather_cols",
    "poetx_scatter_cols", "poetx_timing_enable", "poetx_timing_read", "poetx_timing_reset",
    "poetx_forward_noalloc", "poetx_forward_noalloc_max_bytes",
)

STAGES = ("build", "gather", "block_fwd", "w0_fwd", "scatter", "dq", "block_bwd", "w0_bwd",
          "cnp_bwd")


class PoetxError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: status {status} ({status_string(status)})"
        if status == POETX_ERR_HIP:
            msg += f": {LIB.poetx_last_hip_error().decode()}"
        super().__init__(msg)
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [
        ("m", ctypes.c_int32), ("n", ctypes.c_int32),
        ("nb_R", ctypes.c_int32), ("nb_P", ctypes.c_int32),
        ("bsz_R", ctypes.POINTER(ctypes.c_int32)), ("bsz_P", ctypes.POINTER(ctypes.c_int32)),
        ("k", ctypes.c_int32), ("dtype", ctypes.c_int32), ("weight", ctypes.c_int32),
        ("cayley", ctypes.c_int32), ("fold", ctypes.c_int32), ("index", ctypes.c_int32),
        ("series", ctypes.c_int32),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libpoetx.so is not built ({LIB_PATH}); run __graft_entry__.build()")
    # torch ships its own HIP runtime under an unversioned file name. Loaded
    # first, it satisfies this library's libamdhip64.so.7 dependency by soname,
    # so the process holds one HIP runtime; loaded after us, it would bring a
    # second runtime, and this library's calls would then find no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "poetx_plan_create": (st, [ctypes.POINTER(Desc), ctypes.POINTER(vp)]),
        "poetx_plan_destroy": (None, [vp]),
        "poetx_param_count": (i64, [vp, i32]),
        "poetx_block_elems": (i64, [vp, i32]),
        "poetx_workspace_size": (sz, [vp, i64, i32]),
        "poetx_status_string": (ctypes.c_char_p, [st]),
        "poetx_last_hip_error": (ctypes.c_char_p, []),
        "poetx_permute_weight": (st, [vp, vp, vp, vp, vp, vp]),
        "poetx_merge_weight": (st, [vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "poetx_weight_bytes": (sz, [vp]),
        "poetx_quantize_weight": (st, [vp, vp, vp, vp, vp, vp]),
        "poetx_build_orth": (st, [vp, i32, vp, vp, vp, vp, sz, vp]),
        "poetx_build_orth_batch": (st, [i32, vp, vp, vp, vp, vp, vp, vp, vp]),
        "poetx_forward": (st, [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "poetx_forward_noalloc": (st, [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "poetx_forward_noalloc_max_bytes": (sz, []),
        "poetx_backward": (st, [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                vp, sz, vp]),
        "poetx_backward_dq": (st, [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                   vp]),
        "poetx_param_grad_batch": (st, [i32, vp, vp, vp, vp, vp, vp, vp, vp]),
        "poetx_gather_cols": (st, [vp, i64, i32, vp, vp, vp, vp]),
        "poetx_scatter_cols": (st, [vp, i64, i32, vp, vp, vp, vp]),
        "poetx_timing_enable": (st, [ctypes.c_uint32]),
        "poetx_timing_read": (st, [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]),
        "poetx_timing_reset": (None, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.poetx_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != POETX_OK:
        raise PoetxError(status, where)


def _ptr(t) -> Optional[int]:
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def timing_enable(stages) -> None:
    """Record HIP events around the named stages of every later call."""
    mask = 0
    for name in stages:
        mask |= 1 << STAGES.index(name)
    _check(LIB.poetx_timing_enable(mask), "poetx_timing_enable")


def timing_read(stage: str):
    """(total milliseconds, number of intervals) recorded for one stage."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(LIB.poetx_timing_read(STAGES.index(stage), ctypes.byref(ms), ctypes.byref(n)),
           "poetx_timing_read")
    return ms.value, n.value


def timing_reset() -> None:
    LIB.poetx_timing_reset()


def build_orth_batch(items, stream=None) -> None:
    """Build many (plan, side, theta, Q_f32, Q_act, ws) items in one call."""
    n = len(items)
    if n == 0:
        return
    VP = ctypes.c_void_p * n
    plans = VP(*[it[0].handle for it in items])
    sides = (ctypes.c_int32 * n)(*[it[1] for it in items])
    thetas = VP(*[_ptr(it[2]) for it in items])
    q32 = VP(*[_ptr(it[3]) for it in items])
    qact = VP(*[_ptr(it[4]) for it in items])
    ws = VP(*[_ptr(it[5]) for it in items])
    wsb = (ctypes.c_size_t * n)(*[it[5].numel() for it in items])
    _check(LIB.poetx_build_orth_batch(n, plans, sides, thetas, q32, qact, ws, wsb, _stream(stream)),
           "poetx_build_orth_batch")


def param_grad_batch(items, stream=None) -> None:
    """dL/dQ -> packed parameter gradients for many (plan, side, theta, dQ, g, ws) items."""
    n = len(items)
    if n == 0:
        return
    VP = ctypes.c_void_p * n
    plans = VP(*[it[0].handle for it in items])
    sides = (ctypes.c_int32 * n)(*[it[1] for it in items])
    thetas = VP(*[_ptr(it[2]) for it in items])
    dqs = VP(*[_ptr(it[3]) for it in items])
    gs = VP(*[_ptr(it[4]) for it in items])
    ws = VP(*[_ptr(it[5]) for it in items])
    wsb = (ctypes.c_size_t * n)(*[it[5].numel() for it in items])
    _check(LIB.poetx_param_grad_batch(n, plans, sides, thetas, dqs, gs, ws, wsb, _stream(stream)),
           "poetx_param_grad_batch")


class Plan:
    """Owns a poetx_plan (host-only object; creating one needs no GPU)."""

    def __init__(self, m: int, n: int, bsz_R: Sequence[int], bsz_P: Sequence[int], k: int,
                 dtype: int, weight: int = WEIGHT_DENSE, cayley: int = CAYLEY_NEUMANN,
                 fold: int = FOLD_NONE, index: int = INDEX_SEPARATE, series: int = SERIES_CHAIN):
        self.m, self.n, self.k, self.dtype = int(m), int(n), int(k), int(dtype)
        self.weight, self.cayley, self.fold = int(weight), int(cayley), int(fold)
        self.index, self.series = int(index), int(series)
        self.bsz_R, self.bsz_P = tuple(int(b) for b in bsz_R), tuple(int(b) for b in bsz_P)
        aR = (ctypes.c_int32 * max(1, len(self.bsz_R)))(*self.bsz_R)
        aP = (ctypes.c_int32 * max(1, len(self.bsz_P)))(*self.bsz_P)
        d = Desc(self.m, self.n, len(self.bsz_R), len(self.bsz_P), aR, aP, self.k, self.dtype,
                 self.weight, self.cayley, self.fold, self.index, self.series)
        h = ctypes.c_void_p()
        self._h = None
        _check(LIB.poetx_plan_create(ctypes.byref(d), ctypes.byref(h)), "poetx_plan_create")
        self._h = h.value

    @property
    def handle(self) -> int:
        return self._h

    def close(self) -> None:
        if self._h:
            LIB.poetx_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def param_count(self, side: int) -> int:
        return int(LIB.poetx_param_count(self._h, side))

    def block_elems(self, side: int) -> int:
        return int(LIB.poetx_block_elems(self._h, side))

    def workspace_size(self, T: int, kind: int) -> int:
        return int(LIB.poetx_workspace_size(self._h, T, kind))

    # ---- calls (tensors are torch tensors on the GPU, or raw int addresses)
    def permute_weight(self, W0, pi_R, pi_P, Wt, stream=None) -> None:
        _check(LIB.poetx_permute_weight(self._h, _ptr(W0), _ptr(pi_R), _ptr(pi_P), _ptr(Wt),
                                        _stream(stream)), "poetx_permute_weight")

    def weight_bytes(self) -> int:
        return int(LIB.poetx_weight_bytes(self._h))

    def quantize_weight(self, W0, pi_R, pi_P, Wq, stream=None) -> None:
        _check(LIB.poetx_quantize_weight(self._h, _ptr(W0), _ptr(pi_R), _ptr(pi_P), _ptr(Wq),
                                         _stream(stream)), "poetx_quantize_weight")

    def merge_weight(self, Wt, pi_R, pi_P, Q_R, Q_P, W_out, ws, ws_bytes: int, stream=None) -> None:
        _check(LIB.poetx_merge_weight(self._h, _ptr(Wt), _ptr(pi_R), _ptr(pi_P), _ptr(Q_R),
                                      _ptr(Q_P), _ptr(W_out), _ptr(ws), ws_bytes, _stream(stream)),
               "poetx_merge_weight")

    def build_orth(self, side: int, theta, Q_f32, Q_act, ws, ws_bytes: int, stream=None) -> None:
        _check(LIB.poetx_build_orth(self._h, side, _ptr(theta), _ptr(Q_f32), _ptr(Q_act),
                                    _ptr(ws), ws_bytes, _stream(stream)), "poetx_build_orth")

    def forward(self, T: int, X, Wt, pi_R, pi_P, Q_R, Q_P, Y, Wa_saved, ws, ws_bytes: int,
                stream=None, U_saved=None) -> None:
        _check(LIB.poetx_forward(self._h, T, _ptr(X), _ptr(Wt), _ptr(pi_R), _ptr(pi_P),
                                 _ptr(Q_R), _ptr(Q_P), _ptr(Y), _ptr(Wa_saved), _ptr(U_saved),
                                 _ptr(ws), ws_bytes, _stream(stream)), "poetx_forward")

    def forward_noalloc(self, T: int, X, Wt, pi_R, pi_P, Q_R, Q_P, Y, Wa_saved, stream=None,
                        U_saved=None) -> None:
        _check(LIB.poetx_forward_noalloc(self._h, T, _ptr(X), _ptr(Wt), _ptr(pi_R), _ptr(pi_P),
                                         _ptr(Q_R), _ptr(Q_P), _ptr(Y), _ptr(Wa_saved),
                                         _ptr(U_saved), _stream(stream)), "poetx_forward_noalloc")

    def backward(self, T: int, X, Wt, pi_R, pi_P, theta_R, theta_P, Q_R, Q_P, Wa_saved, G_Y,
                 G_X, g_theta_R, g_theta_P, ws, ws_bytes: int, stream=None, U_saved=None) -> None:
        _check(LIB.poetx_backward(self._h, T, _ptr(X), _ptr(Wt), _ptr(pi_R), _ptr(pi_P),
                                  _ptr(theta_R), _ptr(theta_P), _ptr(Q_R), _ptr(Q_P),
                                  _ptr(Wa_saved), _ptr(U_saved), _ptr(G_Y), _ptr(G_X),
                                  _ptr(g_theta_R), _ptr(g_theta_P), _ptr(ws), ws_bytes,
                                  _stream(stream)), "poetx_backward")

    def backward_dq(self, T: int, X, Wt, pi_R, pi_P, Q_R, Q_P, Wa_saved, G_Y, G_X, dQ_R, dQ_P,
                    ws, ws_bytes: int, stream=None, U_saved=None) -> None:
        _check(LIB.poetx_backward_dq(self._h, T, _ptr(X), _ptr(Wt), _ptr(pi_R), _ptr(pi_P),
                                     _ptr(Q_R), _ptr(Q_P), _ptr(Wa_saved), _ptr(U_saved),
                                     _ptr(G_Y), _ptr(G_X), _ptr(dQ_R), _ptr(dQ_P), _ptr(ws),
                                     ws_bytes, _stream(stream)), "poetx_backward_dq")

    def gather_cols(self, T: int, dim: int, inp, idx, out, stream=None) -> None:
        _check(LIB.poetx_gather_cols(self._h, T, dim, _ptr(inp), _ptr(idx), _ptr(out),
                                     _stream(stream)), "poetx_gather_cols")

    def scatter_cols(self, T: int, dim: int, inp, idx, out, stream=None) -> None:
        _check(LIB.poetx_scatter_cols(self._h, T, dim, _ptr(inp), _ptr(idx), _ptr(out),
                                      _stream(stream)), "poetx_scatter_cols")
