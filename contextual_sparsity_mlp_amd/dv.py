"""Thin ctypes binding of ``libdv.so`` (include/dv.h).

Argument marshalling only: every step of the decode path runs in the library's HIP
kernels.  Tensors are PyTorch device tensors; the binding passes their device
addresses, the current HIP stream and the sizes the C functions expect.  A pointer
argument may also be a raw integer address or ``None`` (NULL), which the tests use
to exercise the argument checks.  The library is loaded on first use; if it has not
been built, the first call raises ``ImportError``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libdv.so")

DV_F32, DV_BF16, DV_FP8 = 0, 1, 2
DV_ACT_RELU, DV_ACT_GELU = 0, 1
DV_OK, DV_EINVAL, DV_EALIGN, DV_EUNSUPPORTED, DV_EWORKSPACE, DV_EHIP, DV_ETIMEOUT = \
    0, -1, -2, -3, -4, -5, -6
OP_PREDICT, OP_SELECT_TOPK, OP_SPARSE_MLP, OP_SPARSE_MHA, OP_DECODE_LAYER = 1, 2, 3, 4, 5

# Every function declared in include/dv.h.
EXPORTS = ("dv_last_error", "dv_version", "dv_workspace_bytes", "dv_predict", "dv_select_topk",
           "dv_sparse_mlp", "dv_sparse_mha", "dv_decode_layer", "dv_decode_layer_noalloc",
           "dv_noalloc_scratch_bytes", "dv_check", "dv_debug_wait_limits", "dv_set_step_path", "dv_timing_enable",
           "dv_timing_read")


class DvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dv error {code}: {msg}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("batch", "d", "F", "h", "dh", "n_ctx", "r", "N", "max_count_m", "max_count_a")]


class LayerStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("d", "F", "h", "dh", "n_ctx", "r", "k_m", "k_a",
                                             "wdt", "kvdt")] + \
               [("scale", ctypes.c_float)] + \
               [(n, ctypes.c_void_p) for n in ("W1t", "W2t", "Wq", "Wo", "K", "V",
                                                "A_M", "B_M", "A_A", "B_A")] + \
               [("act", ctypes.c_int), ("pwdt", ctypes.c_int)] + \
               [(n, ctypes.c_void_p) for n in ("W1s", "W2s", "Wqs", "Wos")] + \
               [(n, ctypes.c_void_p) for n in ("Wk", "Wv", "Wks", "Wvs")] + \
               [("kv_cap", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m contextual_sparsity_mlp_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        L.dv_last_error.restype = ctypes.c_char_p
        L.dv_last_error.argtypes = []
        L.dv_version.restype = i
        L.dv_workspace_bytes.restype = sz
        L.dv_workspace_bytes.argtypes = [i, ctypes.POINTER(Shape)]
        L.dv_predict.argtypes = [vp, i, i, vp, vp, i, i, i, vp, vp, sz, vp]
        L.dv_select_topk.argtypes = [vp, i, i, i, i, vp, vp, vp, sz, vp]
        L.dv_sparse_mlp.argtypes = [vp, i, i, vp, vp, i, i, vp, vp, i, vp, i, i, vp, sz, vp]
        L.dv_sparse_mha.argtypes = [vp, i, i, i, i, vp, vp, i, vp, vp, i, i, vp, vp, i, f, vp, i,
                                    vp, sz, vp]
        L.dv_decode_layer.argtypes = [ctypes.POINTER(LayerStruct), ctypes.POINTER(LayerStruct), i,
                                      vp, vp, vp, vp, i, vp, vp, i, vp, vp, vp, vp, vp, sz, vp]
        L.dv_decode_layer_noalloc.argtypes = [ctypes.POINTER(LayerStruct),
                                              ctypes.POINTER(LayerStruct), i, vp, vp, vp, vp, i,
                                              vp, vp, i, vp, vp, vp, vp, vp]
        L.dv_noalloc_scratch_bytes.restype = sz
        L.dv_noalloc_scratch_bytes.argtypes = []
        L.dv_check.argtypes = [vp]
        L.dv_debug_wait_limits.argtypes = [ctypes.c_uint, ctypes.c_uint]
        L.dv_timing_enable.argtypes = [i]
        L.dv_timing_read.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int),
                                     i, ctypes.POINTER(ctypes.c_int)]
        for name in EXPORTS:
            if name not in ("dv_last_error", "dv_workspace_bytes", "dv_noalloc_scratch_bytes"):
                getattr(L, name).restype = i
        _lib = L
    return _lib


def last_error() -> str:
    return lib().dv_last_error().decode()


def _check(code: int):
    if code != DV_OK:
        raise DvError(code, last_error())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _dtype(t) -> int:
    if isinstance(t, int):
        return t
    if t.dtype == torch.bfloat16:
        return DV_BF16
    if t.dtype == torch.float32:
        return DV_F32
    if t.dtype == torch.uint8:          # fp8 E4M3 codes (with row scales)
        return DV_FP8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _nbytes(ws) -> int:
    if ws is None:
        return 0
    if isinstance(ws, int):
        return 0
    return ws.numel() * ws.element_size()


def workspace_bytes(op: int, **shape) -> int:
    s = Shape(**{k: int(v) for k, v in shape.items()})
    n = lib().dv_workspace_bytes(op, ctypes.byref(s))
    if n == 0:
        raise DvError(DV_EINVAL, last_error())
    return n


def workspace(op: int, device="cuda", **shape) -> torch.Tensor:
    """A workspace tensor of the size dv_workspace_bytes reports."""
    return torch.empty(workspace_bytes(op, **shape), dtype=torch.uint8, device=device)


def predict(y, A, Bm, scores, ws, stream=None, *, batch=None, d=None, r=None, N=None, wdt=None):
    batch = y.shape[0] if batch is None else batch
    d = y.shape[1] if d is None else d
    r = A.shape[0] if r is None else r
    N = Bm.shape[1] if N is None else N
    wdt = _dtype(A) if wdt is None else wdt
    _check(lib().dv_predict(_ptr(y), batch, d, _ptr(A), _ptr(Bm), r, N, wdt, _ptr(scores),
                            _ptr(ws), _nbytes(ws), _stream(stream)))


def select_topk(scores, k, union_rows, idx, count, ws, stream=None, *, batch=None, N=None):
    batch = scores.shape[0] if batch is None else batch
    N = scores.shape[1] if N is None else N
    _check(lib().dv_select_topk(_ptr(scores), batch, N, int(k), int(union_rows), _ptr(idx),
                                _ptr(count), _ptr(ws), _nbytes(ws), _stream(stream)))


def sparse_mlp(y, W1t, W2t, idx, count, max_count, out, accumulate, ws, stream=None, *,
               batch=None, d=None, F=None, wdt=None, act=DV_ACT_RELU):
    batch = y.shape[0] if batch is None else batch
    d = y.shape[1] if d is None else d
    F = W1t.shape[0] if F is None else F
    wdt = _dtype(W1t) if wdt is None else wdt
    _check(lib().dv_sparse_mlp(_ptr(y), batch, d, _ptr(W1t), _ptr(W2t), F, wdt, _ptr(idx),
                               _ptr(count), int(max_count), _ptr(out), int(accumulate), int(act),
                               _ptr(ws), _nbytes(ws), _stream(stream)))


def sparse_mha(y, Wq, Wo, K, V, heads, count, max_count, scale, out, accumulate, ws, stream=None,
               *, batch=None, d=None, h=None, dh=None, n_ctx=None, wdt=None, kvdt=None):
    batch = y.shape[0] if batch is None else batch
    d = y.shape[1] if d is None else d
    h = Wq.shape[0] if h is None else h
    dh = Wq.shape[1] if dh is None else dh
    n_ctx = K.shape[2] if n_ctx is None else n_ctx
    wdt = _dtype(Wq) if wdt is None else wdt
    kvdt = _dtype(K) if kvdt is None else kvdt
    _check(lib().dv_sparse_mha(_ptr(y), batch, d, h, dh, _ptr(Wq), _ptr(Wo), wdt, _ptr(K), _ptr(V),
                               n_ctx, kvdt, _ptr(heads), _ptr(count), int(max_count), float(scale),
                               _ptr(out), int(accumulate), _ptr(ws), _nbytes(ws), _stream(stream)))


class Layer:
    """A dv_layer built from a layer's tensors; keeps them alive while in use."""

    def __init__(self, W1t, W2t, Wq, Wo, K, V, A_M=None, B_M=None, A_A=None, B_A=None, *,
                 k_m=0, k_a=0, scale=1.0, act=DV_ACT_RELU, row_scales=None, Wk=None, Wv=None,
                 kv_scales=None, n_ctx=None):
        """row_scales = (W1s, W2s, Wqs, Wos) for fp8 weights (uint8 E4M3 codes).

        K, V are [batch][h][kv_cap][dh]; n_ctx (default kv_cap) rows are the cache.
        Wk, Wv (with kv_scales = (Wks, Wvs) for fp8) make each decode step append the
        current token's k and v at row n_ctx; advance with ``set_n_ctx``."""
        self.tensors = (W1t, W2t, Wq, Wo, K, V, A_M, B_M, A_A, B_A, row_scales, Wk, Wv, kv_scales)
        r = A_M.shape[0] if A_M is not None else 0
        rs = row_scales if row_scales is not None else (None, None, None, None)
        ks = kv_scales if kv_scales is not None else (None, None)
        self.s = LayerStruct(d=W1t.shape[1], F=W1t.shape[0], h=Wq.shape[0], dh=Wq.shape[1],
                             n_ctx=K.shape[2] if n_ctx is None else int(n_ctx), r=r,
                             k_m=int(k_m), k_a=int(k_a),
                             wdt=_dtype(W1t), kvdt=_dtype(K), scale=float(scale),
                             W1t=_ptr(W1t), W2t=_ptr(W2t), Wq=_ptr(Wq), Wo=_ptr(Wo), K=_ptr(K),
                             V=_ptr(V), A_M=_ptr(A_M), B_M=_ptr(B_M), A_A=_ptr(A_A), B_A=_ptr(B_A),
                             act=int(act),
                             pwdt=_dtype(A_M) if A_M is not None else DV_BF16,
                             W1s=_ptr(rs[0]), W2s=_ptr(rs[1]), Wqs=_ptr(rs[2]), Wos=_ptr(rs[3]),
                             Wk=_ptr(Wk), Wv=_ptr(Wv), Wks=_ptr(ks[0]), Wvs=_ptr(ks[1]),
                             kv_cap=K.shape[2])

    def set_n_ctx(self, n: int):
        """Rows of the cache the next step reads (the append goes to row n)."""
        self.s.n_ctx = int(n)


def decode_layer(layer: Layer, next_layer, y_in, y_out, idx_m, count_m, max_count_m, idx_a, count_a,
                 max_count_a, next_idx_m, next_count_m, next_idx_a, next_count_a, ws, stream=None,
                 *, batch=None):
    batch = y_in.shape[0] if batch is None else batch
    nxt = ctypes.byref(next_layer.s) if next_layer is not None else None
    _check(lib().dv_decode_layer(ctypes.byref(layer.s), nxt, batch, _ptr(y_in), _ptr(y_out),
                                 _ptr(idx_m), _ptr(count_m), int(max_count_m), _ptr(idx_a),
                                 _ptr(count_a), int(max_count_a), _ptr(next_idx_m),
                                 _ptr(next_count_m), _ptr(next_idx_a), _ptr(next_count_a),
                                 _ptr(ws), _nbytes(ws), _stream(stream)))


def decode_layer_noalloc(layer: Layer, next_layer, y_in, y_out, idx_m, count_m, max_count_m,
                         idx_a, count_a, max_count_a, next_idx_m, next_count_m, next_idx_a,
                         next_count_a, stream=None, *, batch=None):
    """dv_decode_layer_noalloc: decode_layer with the library's per-device scratch as
    its workspace (no workspace argument, nothing allocated)."""
    batch = y_in.shape[0] if batch is None else batch
    nxt = ctypes.byref(next_layer.s) if next_layer is not None else None
    _check(lib().dv_decode_layer_noalloc(ctypes.byref(layer.s), nxt, batch, _ptr(y_in),
                                         _ptr(y_out), _ptr(idx_m), _ptr(count_m),
                                         int(max_count_m), _ptr(idx_a), _ptr(count_a),
                                         int(max_count_a), _ptr(next_idx_m), _ptr(next_count_m),
                                         _ptr(next_idx_a), _ptr(next_count_a), _stream(stream)))


def noalloc_scratch_bytes() -> int:
    return int(lib().dv_noalloc_scratch_bytes())


def check(stream=None):
    """dv_check: synchronise the stream; raise DvError(DV_ETIMEOUT) if an in-launch wait
    of an earlier call gave up (DV_EHIP on a runtime error)."""
    _check(lib().dv_check(_stream(stream)))


def debug_wait_limits(spins: int = 0, extra: int = 0):
    """Test hook: poll limit of in-launch waits (0 = default) and an offset added to their
    targets (extra > 0 makes every such wait give up)."""
    _check(lib().dv_debug_wait_limits(int(spins), int(extra)))


PATH_AUTO, PATH_TWO_LAUNCH, PATH_ONE_LAUNCH = 0, 1, 2


def set_step_path(path: int):
    """dv_set_step_path: launch plan of the one-token bf16 sparse step (PATH_AUTO takes
    the faster one)."""
    _check(lib().dv_set_step_path(int(path)))


def timing_enable(on: bool):
    _check(lib().dv_timing_enable(1 if on else 0))


def timing_read(max_slots: int = 8):
    """Summed milliseconds and launch counts per launch slot since the last read."""
    ms = (ctypes.c_float * max_slots)()
    cnt = (ctypes.c_int * max_slots)()
    n = ctypes.c_int(0)
    _check(lib().dv_timing_read(ms, cnt, max_slots, ctypes.byref(n)))
    return [float(ms[i]) for i in range(n.value)], [int(cnt[i]) for i in range(n.value)]
