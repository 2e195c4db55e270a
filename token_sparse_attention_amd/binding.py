"""ctypes binding of libtsa.so.  Argument marshalling only: every step runs in the library's HIP
kernels.  torch tensors supply device memory (``data_ptr()``) and the stream
(``torch.cuda.current_stream()``); nothing here computes.  A missing library is an error."""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsa.so")
_lib = None

F32, BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "unsupported dtype",
           4: "tensor not 16-byte aligned", 5: "workspace missing, misaligned or too small",
           6: "HIP launch failed", 7: "not implemented for these parameters",
           8: "intermediates exceed the fixed scratch of the allocation-free entry point"}


class TsaError(RuntimeError):
    def __init__(self, fn, status, detail=None):
        self.status = status
        msg = f"{fn} failed with status {status} ({_STATUS.get(status, 'unknown')})"
        super().__init__(msg if detail is None else f"{msg}: {detail}")


class Shape(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int64), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("q", ctypes.c_int32), ("tau", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


# name -> argument types after the leading `const tsa_shape*`
_P = ctypes.c_void_p
_SIGS = {
    "tsa_score": [_P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_budget": [_P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_select": [_P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_gather": [_P, _P, _P, _P, _P, _P, _P, _P, _P],
    "tsa_attn_causal": [_P, _P, _P, _P, _P, _P],
    "tsa_scatter_residual": [_P, _P, _P, _P, _P, _P, _P],
    "tsa_layer": [_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_layer_noalloc": [_P, _P, _P, _P, _P, _P, _P],
    "tsa_dense_attn_causal": [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_budget_ratio": [ctypes.c_float, _P, _P, _P],
    "tsa_layer_ratio": [ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_attn_causal_varlen": [ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P],
    "tsa_layer_varlen": [ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_dense_attn_causal_varlen": [ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_block_select": [ctypes.c_float, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_attn_block_sparse": [_P, _P, _P, _P, _P, _P, _P, _P],
    "tsa_layer_block_sparse": [ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
}
_SHAPE_WS = ("tsa_block_select_workspace_bytes", "tsa_layer_block_sparse_workspace_bytes")
_VARLEN_WS = ("tsa_layer_varlen_workspace_bytes", "tsa_dense_varlen_workspace_bytes")
EXPORTS = ["tsa_status_string", "tsa_check_args", "tsa_capacity", "tsa_stage_workspace_bytes",
           "tsa_layer_workspace_bytes", "tsa_dense_workspace_bytes", *_SIGS, "tsa_varlen_capacity", *_VARLEN_WS,
           "tsa_block_count", *_SHAPE_WS]


def lib():
    """Open libtsa.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(_LIB_PATH)
        sp = ctypes.POINTER(Shape)
        L.tsa_status_string.restype = ctypes.c_char_p
        L.tsa_status_string.argtypes = [ctypes.c_int]
        L.tsa_check_args.restype = ctypes.c_int
        L.tsa_check_args.argtypes = [sp]
        L.tsa_capacity.restype = ctypes.c_int64
        L.tsa_capacity.argtypes = [ctypes.c_int64]
        L.tsa_block_count.restype = ctypes.c_int64
        L.tsa_block_count.argtypes = [ctypes.c_int64]
        for n in ("tsa_stage_workspace_bytes", "tsa_layer_workspace_bytes", "tsa_dense_workspace_bytes", *_SHAPE_WS):
            getattr(L, n).restype = ctypes.c_size_t
            getattr(L, n).argtypes = [sp]
        for n, args in _SIGS.items():
            getattr(L, n).restype = ctypes.c_int
            getattr(L, n).argtypes = [sp, *args]
        L.tsa_varlen_capacity.restype = ctypes.c_int64
        L.tsa_varlen_capacity.argtypes = [ctypes.c_int32, _P]
        for n in _VARLEN_WS:
            getattr(L, n).restype = ctypes.c_size_t
            getattr(L, n).argtypes = [sp, ctypes.c_int32, _P]
        _lib = L
    return _lib


def shape(L, Hq, Hkv, d, q, tau, dtype):
    """A tsa_shape; dtype is "bf16", "f32" or a torch dtype."""
    if dtype in ("bf16", torch.bfloat16):
        dt = BF16
    elif dtype in ("f32", torch.float32):
        dt = F32
    else:
        raise ValueError(f"unsupported dtype {dtype}")
    return Shape(int(L), int(Hq), int(Hkv), int(d), int(q), float(tau), dt)


def shape_of(cfg):
    return shape(cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.q, cfg.tau, cfg.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_I32 = (torch.int32,)
_F32 = (torch.float32,)
_U16 = (torch.int16, torch.uint16)


def _storage(s):
    return (torch.bfloat16,) if s.dtype == BF16 else (torch.float32,)


def _validate(fn, specs):
    """Host-side checks of every torch tensor argument before libtsa sees its address: on the
    current CUDA device, contiguous, of the element type the call reads or writes, and holding at
    least the elements that call touches.  A wrong tensor would make a kernel read or write past its
    buffer, so it raises TsaError here instead.  None and objects that are not tensors (raw
    addresses the caller vouches for) pass through to the library's own checks."""
    tensors = [(name, t, dtypes, numel) for name, t, dtypes, numel in specs if isinstance(t, torch.Tensor)]
    for name, t, dtypes, numel in tensors:
        if not t.is_contiguous():
            raise TsaError(fn, 1, f"{name} is not contiguous")
        if dtypes is not None and t.dtype not in dtypes:
            raise TsaError(fn, 3, f"{name} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
        if t.numel() < numel:
            raise TsaError(fn, 1, f"{name} holds {t.numel()} elements, the call touches {numel}")
    dev = None
    for name, t, _, _ in tensors:
        if not t.is_cuda:
            raise TsaError(fn, 1, f"{name} is not a device tensor")
        if dev is None:
            dev = torch.cuda.current_device()
        if t.device.index != dev:
            raise TsaError(fn, 1, f"{name} is on {t.device}, the current device is cuda:{dev}")


def _dims(s):
    """(L, Hq, Hkv, d, C) of a shape as Python ints."""
    return int(s.L), int(s.Hq), int(s.Hkv), int(s.d), int(capacity(s.L)) if s.L > 0 else 0


def _layer_io(s, Q, K, V, X, Y):
    L, Hq, Hkv, d, _ = _dims(s)
    st = _storage(s)
    return [("Q", Q, st, L * Hq * d), ("K", K, st, L * Hkv * d), ("V", V, st, L * Hkv * d),
            ("X", X, st, L * Hq * d), ("Y", Y, st, L * Hq * d)]


def _compressed(s, cap, **ts):
    _, Hq, _, d, _ = _dims(s)
    return [(n, t, _storage(s), Hq * cap * d) for n, t in ts.items()]


def _stream(stream):
    """None: torch's current stream; an int: a raw hipStream_t handle; else a torch stream."""
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise TsaError(fn, status)


def check_args(s):
    return lib().tsa_check_args(ctypes.byref(s))


def capacity(L):
    return lib().tsa_capacity(int(L))


def stage_workspace_bytes(s):
    return lib().tsa_stage_workspace_bytes(ctypes.byref(s))


def layer_workspace_bytes(s):
    return lib().tsa_layer_workspace_bytes(ctypes.byref(s))


def dense_workspace_bytes(s):
    return lib().tsa_dense_workspace_bytes(ctypes.byref(s))


def workspace(nbytes, device="cuda"):
    """A device buffer for the library's workspace (torch's allocator returns 256-byte aligned
    blocks)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _ws(ws):
    return _ptr(ws), ctypes.c_size_t(0 if ws is None else ws.numel() * ws.element_size())


def score(s, Q, K, s_h, s_l=None, ws=None, stream=None):
    L, Hq, Hkv, d, _ = _dims(s)
    _validate("tsa_score", [("Q", Q, _storage(s), L * Hq * d), ("K", K, _storage(s), L * Hkv * d),
                            ("s_h", s_h, _F32, Hq * L), ("s_l", s_l, _F32, L), ("ws", ws, None, 0)])
    p, n = _ws(ws)
    _check("tsa_score", lib().tsa_score(ctypes.byref(s), _ptr(Q), _ptr(K), _ptr(s_h), _ptr(s_l), p, n,
                                        _stream(stream)))


def budget(s, s_l, k_dev=None, Lp_dev=None, ws=None, stream=None):
    _validate("tsa_budget", [("s_l", s_l, _F32, int(s.L)), ("k_dev", k_dev, _I32, 1), ("Lp_dev", Lp_dev, _I32, 1),
                             ("ws", ws, None, 0)])
    p, n = _ws(ws)
    _check("tsa_budget", lib().tsa_budget(ctypes.byref(s), _ptr(s_l), _ptr(k_dev), _ptr(Lp_dev), p, n,
                                          _stream(stream)))


def select(s, s_h, Lp_dev, idx, inv=None, ws=None, stream=None):
    hl = int(s.Hq) * int(s.L)
    _validate("tsa_select", [("s_h", s_h, _F32, hl), ("Lp_dev", Lp_dev, _I32, 1), ("idx", idx, _I32, hl),
                             ("inv", inv, _I32, hl), ("ws", ws, None, 0)])
    p, n = _ws(ws)
    _check("tsa_select", lib().tsa_select(ctypes.byref(s), _ptr(s_h), _ptr(Lp_dev), _ptr(idx), _ptr(inv),
                                          p, n, _stream(stream)))


def gather(s, Q, K, V, idx, Lp_dev, Qh, Kh, Vht, stream=None):
    _validate("tsa_gather", _layer_io(s, Q, K, V, None, None) + _compressed(s, _dims(s)[4], Qh=Qh, Kh=Kh, Vht=Vht)
              + [("idx", idx, _I32, int(s.Hq) * int(s.L)), ("Lp_dev", Lp_dev, _I32, 1)])
    _check("tsa_gather", lib().tsa_gather(ctypes.byref(s), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx),
                                          _ptr(Lp_dev), _ptr(Qh), _ptr(Kh), _ptr(Vht), _stream(stream)))


def attn_causal(s, Qh, Kh, Vht, Lp_dev, Oh, stream=None):
    _validate("tsa_attn_causal", _compressed(s, _dims(s)[4], Qh=Qh, Kh=Kh, Vht=Vht, Oh=Oh)
              + [("Lp_dev", Lp_dev, _I32, 1)])
    _check("tsa_attn_causal", lib().tsa_attn_causal(ctypes.byref(s), _ptr(Qh), _ptr(Kh), _ptr(Vht),
                                                    _ptr(Lp_dev), _ptr(Oh), _stream(stream)))


def scatter_residual(s, Oh, idx, inv, Lp_dev, X, Y, stream=None):
    hl = int(s.Hq) * int(s.L)
    _validate("tsa_scatter_residual", _layer_io(s, None, None, None, X, Y) + _compressed(s, _dims(s)[4], Oh=Oh)
              + [("idx", idx, _I32, hl), ("inv", inv, _I32, hl), ("Lp_dev", Lp_dev, _I32, 1)])
    _check("tsa_scatter_residual", lib().tsa_scatter_residual(ctypes.byref(s), _ptr(Oh), _ptr(idx), _ptr(inv),
                                                              _ptr(Lp_dev), _ptr(X), _ptr(Y), _stream(stream)))


def layer(s, Q, K, V, X, Y, kLp_dev=None, ws=None, stream=None):
    _validate("tsa_layer", _layer_io(s, Q, K, V, X, Y) + [("kLp_dev", kLp_dev, _I32, 2), ("ws", ws, None, 0)])
    p, n = _ws(ws)
    _check("tsa_layer", lib().tsa_layer(ctypes.byref(s), _ptr(Q), _ptr(K), _ptr(V), _ptr(X), _ptr(Y),
                                        _ptr(kLp_dev), p, n, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 256 << 20       # TSA_NOALLOC_SCRATCH_BYTES of tsa.h


def layer_noalloc(s, Q, K, V, X, Y, kLp_dev=None, stream=None):
    """tsa_layer with the library's fixed per-GPU scratch in place of a caller workspace."""
    _validate("tsa_layer_noalloc", _layer_io(s, Q, K, V, X, Y) + [("kLp_dev", kLp_dev, _I32, 2)])
    _check("tsa_layer_noalloc", lib().tsa_layer_noalloc(ctypes.byref(s), _ptr(Q), _ptr(K), _ptr(V), _ptr(X), _ptr(Y),
                                                        _ptr(kLp_dev), _stream(stream)))


def budget_ratio(s, sparsity, k_dev=None, Lp_dev=None, stream=None):
    _validate("tsa_budget_ratio", [("k_dev", k_dev, _I32, 1), ("Lp_dev", Lp_dev, _I32, 1)])
    _check("tsa_budget_ratio", lib().tsa_budget_ratio(ctypes.byref(s), float(sparsity), _ptr(k_dev),
                                                      _ptr(Lp_dev), _stream(stream)))


def layer_ratio(s, sparsity, Q, K, V, X, Y, kLp_dev=None, ws=None, stream=None):
    _validate("tsa_layer_ratio", _layer_io(s, Q, K, V, X, Y) + [("kLp_dev", kLp_dev, _I32, 2), ("ws", ws, None, 0)])
    p, n = _ws(ws)
    _check("tsa_layer_ratio", lib().tsa_layer_ratio(ctypes.byref(s), float(sparsity), _ptr(Q), _ptr(K), _ptr(V),
                                                    _ptr(X), _ptr(Y), _ptr(kLp_dev), p, n, _stream(stream)))


def dense_attn_causal(s, Q, K, V, X, Y, ws=None, stream=None):
    _validate("tsa_dense_attn_causal", _layer_io(s, Q, K, V, X, Y) + [("ws", ws, None, 0)])
    p, n = _ws(ws)
    _check("tsa_dense_attn_causal", lib().tsa_dense_attn_causal(ctypes.byref(s), _ptr(Q), _ptr(K), _ptr(V),
                                                                _ptr(X), _ptr(Y), p, n, _stream(stream)))


# -- varlen batches: cu_seqlens is a host sequence of B+1 token offsets ---------------------------

def _cu(cu_seqlens):
    arr = (ctypes.c_int64 * len(cu_seqlens))(*[int(v) for v in cu_seqlens])
    return ctypes.c_int32(len(cu_seqlens) - 1), arr


def varlen_capacity(cu_seqlens):
    B, arr = _cu(cu_seqlens)
    return lib().tsa_varlen_capacity(B, ctypes.cast(arr, _P))


def layer_varlen_workspace_bytes(s, cu_seqlens):
    B, arr = _cu(cu_seqlens)
    return lib().tsa_layer_varlen_workspace_bytes(ctypes.byref(s), B, ctypes.cast(arr, _P))


def dense_varlen_workspace_bytes(s, cu_seqlens):
    B, arr = _cu(cu_seqlens)
    return lib().tsa_dense_varlen_workspace_bytes(ctypes.byref(s), B, ctypes.cast(arr, _P))


def attn_causal_varlen(s, cu_seqlens, Qh, Kh, Vht, Lp_dev, Oh, stream=None):
    B, arr = _cu(cu_seqlens)
    P = max(varlen_capacity(cu_seqlens), 0)
    _validate("tsa_attn_causal_varlen", _compressed(s, P, Qh=Qh, Kh=Kh, Vht=Vht, Oh=Oh)
              + [("Lp_dev", Lp_dev, _I32, B.value)])
    _check("tsa_attn_causal_varlen", lib().tsa_attn_causal_varlen(
        ctypes.byref(s), B, ctypes.cast(arr, _P), _ptr(Qh), _ptr(Kh), _ptr(Vht), _ptr(Lp_dev), _ptr(Oh),
        _stream(stream)))


def layer_varlen(s, cu_seqlens, Q, K, V, X, Y, kLp_dev=None, ws=None, stream=None):
    B, arr = _cu(cu_seqlens)
    _validate("tsa_layer_varlen", _layer_io(s, Q, K, V, X, Y) + [("kLp_dev", kLp_dev, _I32, 2 * B.value),
                                                                 ("ws", ws, None, 0)])
    p, n = _ws(ws)
    _check("tsa_layer_varlen", lib().tsa_layer_varlen(
        ctypes.byref(s), B, ctypes.cast(arr, _P), _ptr(Q), _ptr(K), _ptr(V), _ptr(X), _ptr(Y), _ptr(kLp_dev), p, n,
        _stream(stream)))


def dense_attn_causal_varlen(s, cu_seqlens, Q, K, V, X, Y, ws=None, stream=None):
    B, arr = _cu(cu_seqlens)
    _validate("tsa_dense_attn_causal_varlen", _layer_io(s, Q, K, V, X, Y) + [("ws", ws, None, 0)])
    p, n = _ws(ws)
    _check("tsa_dense_attn_causal_varlen", lib().tsa_dense_attn_causal_varlen(
        ctypes.byref(s), B, ctypes.cast(arr, _P), _ptr(Q), _ptr(K), _ptr(V), _ptr(X), _ptr(Y), p, n,
        _stream(stream)))


# -- block sparsity in the compressed space ---------------------------------------------------------

def block_count(L):
    return lib().tsa_block_count(int(L))


def block_select_workspace_bytes(s):
    return lib().tsa_block_select_workspace_bytes(ctypes.byref(s))


def layer_block_sparse_workspace_bytes(s):
    return lib().tsa_layer_block_sparse_workspace_bytes(ctypes.byref(s))


def _block_lists(s, blist, bcnt):
    nb = block_count(s.L)
    return [("blist", blist, _U16, int(s.Hq) * nb * nb), ("bcnt", bcnt, _I32, int(s.Hq) * nb)]


def block_select(s, gamma, Qh, Kh, Lp_dev, blist, bcnt, ws=None, stream=None):
    _validate("tsa_block_select", _compressed(s, _dims(s)[4], Qh=Qh, Kh=Kh) + _block_lists(s, blist, bcnt)
              + [("Lp_dev", Lp_dev, _I32, 1), ("ws", ws, None, 0)])
    p, n = _ws(ws)
    _check("tsa_block_select", lib().tsa_block_select(ctypes.byref(s), float(gamma), _ptr(Qh), _ptr(Kh), _ptr(Lp_dev),
                                                      _ptr(blist), _ptr(bcnt), p, n, _stream(stream)))


def attn_block_sparse(s, Qh, Kh, Vht, Lp_dev, blist, bcnt, Oh, stream=None):
    _validate("tsa_attn_block_sparse", _compressed(s, _dims(s)[4], Qh=Qh, Kh=Kh, Vht=Vht, Oh=Oh)
              + _block_lists(s, blist, bcnt) + [("Lp_dev", Lp_dev, _I32, 1)])
    _check("tsa_attn_block_sparse", lib().tsa_attn_block_sparse(ctypes.byref(s), _ptr(Qh), _ptr(Kh), _ptr(Vht),
                                                                _ptr(Lp_dev), _ptr(blist), _ptr(bcnt), _ptr(Oh),
                                                                _stream(stream)))


def layer_block_sparse(s, gamma, Q, K, V, X, Y, kLp_dev=None, ws=None, stream=None):
    _validate("tsa_layer_block_sparse", _layer_io(s, Q, K, V, X, Y) + [("kLp_dev", kLp_dev, _I32, 2),
                                                                       ("ws", ws, None, 0)])
    p, n = _ws(ws)
    _check("tsa_layer_block_sparse", lib().tsa_layer_block_sparse(ctypes.byref(s), float(gamma), _ptr(Q), _ptr(K),
                                                                  _ptr(V), _ptr(X), _ptr(Y), _ptr(kLp_dev), p, n,
                                                                  _stream(stream)))
