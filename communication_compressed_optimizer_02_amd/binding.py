"""Python binding of liboba.so (the C ABI in include/oba.h).

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  torch supplies device memory (``torch.Tensor.data_ptr``) and
the stream (``torch.cuda.current_stream()``).  There is no fallback: if the
library is missing or a call fails, an exception is raised.

Buffers (all CUDA tensors on the layout's device, C-contiguous):
  g      [n][ld]  float32, float16 or bfloat16   delta [n][ld] float32
         (ld = row stride, a multiple of 8 >= d; default d rounded up to 8)
  x, m, v, denom, eps  [d] float32
  wbits  [n][W]  int64 (packed 64-bit words)   sbits [W] int64
  wscale [n][n_wseg] float32                   sscale [n_sseg] float32
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboba.so")

OBA_F32, OBA_F16, OBA_BF16 = 0, 1, 2
_lib = None

# name -> (restype, argtypes); mirrors include/oba.h
_P, _I64, _I32, _D, _SZ, _I = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double,
                               ctypes.c_size_t, ctypes.c_int)
SIGNATURES = {
    "oba_version": (_I, []),
    "oba_status_string": (ctypes.c_char_p, [_I]),
    "oba_layout_validate": (_I, [_I64, _I32, _I64, _P, _I32, _P, _I32]),
    "oba_layout_create": (_I, [ctypes.POINTER(_P), _I64, _I32, _I64, _P, _I32, _P, _I32]),
    "oba_layout_destroy": (None, [_P]),
    "oba_workspace_bytes": (_SZ, [_P]),
    "oba_adam_warmup_step": (_I, [_P, _P, _I, _P, _P, _P, _D, _D, _D, _D, _D, _D, _P]),
    "oba_adam_warmup_step_vnorm": (_I, [_P, _P, _I, _P, _P, _P, _D, _D, _D, _D, _D, _D, _P, _P,
                                         _SZ, _P]),
    "oba_plateau_init": (_I, [_P, _I32, _D, _I32]),
    "oba_plateau_observe": (_I, [_P, _D]),
    "oba_freeze_variance": (_I, [_P, _P, _P, _D, _D, _P]),
    "oba_compress": (_I, [_P, _P, _I, _P, _P, _P, _P, _D, _P, _SZ, _P]),
    "oba_server_reduce_recompress": (_I, [_P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "oba_decompress_update": (_I, [_P, _P, _P, _P, _P, _P, _D, _P]),
    "oba_server_momentum": (_I, [_P, _P, _P, _P, _P]),
    "oba_compress_deferred": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _D, _P, _SZ, _P]),
    "oba_compress_deferred_noalloc": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _D, _P]),
    "oba_compress_deferred16": (_I, [_P, _P, _I, _P, _P, _P, _P, _I, _P, _P, _D, _P, _SZ,
                                     _P]),
    "oba_compress_deferred_local": (_I, [_P, _P, _I, _P, _P, _P, _P, _D, _P, _SZ, _P]),
    "oba_server_reduce_recompress_deferred": (_I, [_P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "oba_deferred_errors": (_I, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "oba_tensors_create": (_I, [ctypes.POINTER(_P), _P, _I32, _P, _P, _P, _I]),
    "oba_tensors_destroy": (None, [_P]),
    "oba_adam_warmup_step_listed": (_I, [_P, _P, _P, _P, _D, _D, _D, _D, _D, _D, _P, _P, _SZ,
                                         _P]),
    "oba_compress_deferred_listed": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _D, _P, _SZ, _P]),
    "oba_compress_deferred16_listed": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _D, _P, _SZ,
                                            _P]),
    "oba_decompress_update_listed": (_I, [_P, _P, _P, _P, _P, _P, _D, _P]),
    "oba_step_small": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _D, _D, _P]),
    "oba_timing_enable": (_I, [_I, _I32]),
    "oba_timing_read": (_I, [ctypes.c_char_p, ctypes.POINTER(_D), ctypes.POINTER(_I64)]),
    "oba_timing_reset": (_I, []),
}


class ObaError(RuntimeError):
    pass


def lib():
    """Load liboba.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -c 'import __graft_entry__ as e; e.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(rc: int) -> str:
    return lib().oba_status_string(rc).decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise ObaError(f"{what}: {status_string(rc)} (status {rc})")


def _stream(stream=None):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t, name, dtypes, shape=None):
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name}: expected a CUDA tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _table(seg):
    import numpy as np

    a = np.ascontiguousarray(np.asarray(seg, dtype=np.int64))
    return a, a.ctypes.data_as(ctypes.c_void_p), len(a) - 1


def default_ld(d: int) -> int:
    """Row stride of the [n][ld] buffers: d rounded up to a multiple of 8."""
    return (int(d) + 7) // 8 * 8


def validate(d, n, wseg, sseg, ld=None) -> int:
    ld = default_ld(d) if ld is None else ld
    w, wp, nw = _table(wseg)
    s, sp, ns = _table(sseg)
    return lib().oba_layout_validate(d, n, ld, wp, nw, sp, ns)


class Layout:
    """Owns an oba_layout handle and a workspace tensor on the current device."""

    def __init__(self, d, n, wseg, sseg, ld=None):
        import torch

        self.d, self.n = int(d), int(n)
        self.ld = default_ld(self.d) if ld is None else int(ld)
        self.W = (self.d + 63) // 64
        self.wseg, wp, self.n_wseg = _table(wseg)
        self.sseg, sp, self.n_sseg = _table(sseg)
        h = ctypes.c_void_p()
        _check(lib().oba_layout_create(ctypes.byref(h), self.d, self.n, self.ld, wp, self.n_wseg,
                                       sp, self.n_sseg), "oba_layout_create")
        self.handle = h
        self.device = torch.cuda.current_device()
        self.ws_bytes = lib().oba_workspace_bytes(h)
        self.ws = torch.empty(max(8, self.ws_bytes), dtype=torch.uint8, device="cuda")

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().oba_layout_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _gdtype(g):
    import torch

    return {torch.float16: OBA_F16, torch.bfloat16: OBA_BF16}.get(g.dtype, OBA_F32)


def _gtypes():
    import torch

    return (torch.float32, torch.float16, torch.bfloat16)


def adam_warmup_step(L: Layout, g, x, m, v, lr, beta1, beta2, eta, bc1=1.0, bc2=1.0, stream=None):
    import torch

    f32 = (torch.float32,)
    rc = lib().oba_adam_warmup_step(
        L.handle, _ptr(g, "g", _gtypes(), (L.n, L.ld)), _gdtype(g),
        _ptr(x, "x", f32, (L.d,)), _ptr(m, "m", f32, (L.d,)), _ptr(v, "v", f32, (L.d,)),
        lr, beta1, beta2, eta, bc1, bc2, _stream(stream))
    _check(rc, "oba_adam_warmup_step")


def adam_warmup_step_vnorm(L: Layout, g, x, m, v, lr, beta1, beta2, eta, vnorm, bc1=1.0,
                           bc2=1.0, stream=None):
    """The warm-up step; vnorm (a float64 CUDA tensor of one element) gets
    ||v||_2 of the updated v."""
    import torch

    f32 = (torch.float32,)
    rc = lib().oba_adam_warmup_step_vnorm(
        L.handle, _ptr(g, "g", _gtypes(), (L.n, L.ld)), _gdtype(g),
        _ptr(x, "x", f32, (L.d,)), _ptr(m, "m", f32, (L.d,)), _ptr(v, "v", f32, (L.d,)),
        lr, beta1, beta2, eta, bc1, bc2, _ptr(vnorm, "vnorm", (torch.float64,), (1,)),
        ctypes.c_void_p(L.ws.data_ptr()), L.ws_bytes, _stream(stream))
    _check(rc, "oba_adam_warmup_step_vnorm")


PLATEAU_MAX_WINDOW = 1024


class _PlateauState(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("min_steps", ctypes.c_int32),
                ("steps", ctypes.c_int32), ("fired", ctypes.c_int32), ("rtol", ctypes.c_double),
                ("ring", ctypes.c_double * PLATEAU_MAX_WINDOW)]


class Plateau:
    """The library's plateau test on a scalar series (oba_plateau_*)."""

    def __init__(self, window, rtol, min_steps=0):
        self._s = _PlateauState()
        _check(lib().oba_plateau_init(ctypes.byref(self._s), window, rtol, min_steps),
               "oba_plateau_init")

    def observe(self, value) -> bool:
        rc = lib().oba_plateau_observe(ctypes.byref(self._s), float(value))
        if rc < 0:
            _check(rc, "oba_plateau_observe")
        return rc == 1

    @property
    def steps(self):
        return self._s.steps


def freeze_variance(L: Layout, v, denom, eta, bc2=1.0, stream=None):
    import torch

    f32 = (torch.float32,)
    rc = lib().oba_freeze_variance(L.handle, _ptr(v, "v", f32, (L.d,)),
                                   _ptr(denom, "denom", f32, (L.d,)), eta, bc2, _stream(stream))
    _check(rc, "oba_freeze_variance")


def compress(L: Layout, g, m, delta, wbits, wscale, beta1, stream=None):
    import torch

    f32 = (torch.float32,)
    rc = lib().oba_compress(
        L.handle, _ptr(g, "g", _gtypes(), (L.n, L.ld)), _gdtype(g),
        _ptr(m, "m", f32, (L.d,)), _ptr(delta, "delta", f32, (L.n, L.ld)),
        _ptr(wbits, "wbits", (torch.int64,), (L.n, L.W)),
        _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)), beta1,
        ctypes.c_void_p(L.ws.data_ptr()), L.ws_bytes, _stream(stream))
    _check(rc, "oba_compress")


def server_reduce_recompress(L: Layout, wbits, wscale, eps, sbits, sscale, stream=None):
    import torch

    f32 = (torch.float32,)
    rc = lib().oba_server_reduce_recompress(
        L.handle, _ptr(wbits, "wbits", (torch.int64,), (L.n, L.W)),
        _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)), _ptr(eps, "eps", f32, (L.d,)),
        _ptr(sbits, "sbits", (torch.int64,), (L.W,)), _ptr(sscale, "sscale", f32, (L.n_sseg,)),
        ctypes.c_void_p(L.ws.data_ptr()), L.ws_bytes, _stream(stream))
    _check(rc, "oba_server_reduce_recompress")


def decompress_update(L: Layout, sbits, sscale, denom, m, x, lr, stream=None):
    """m=None: the momentum is not stored (implicit in sbits, sscale)."""
    import torch

    f32 = (torch.float32,)
    mp = _ptr(m, "m", f32, (L.d,)) if m is not None else ctypes.c_void_p(None)
    rc = lib().oba_decompress_update(
        L.handle, _ptr(sbits, "sbits", (torch.int64,), (L.W,)),
        _ptr(sscale, "sscale", f32, (L.n_sseg,)), _ptr(denom, "denom", f32, (L.d,)),
        mp, _ptr(x, "x", f32, (L.d,)), lr, _stream(stream))
    _check(rc, "oba_decompress_update")


def server_momentum(L: Layout, sbits, sscale, m, stream=None):
    """m = sbar*sign from the server message."""
    import torch

    f32 = (torch.float32,)
    rc = lib().oba_server_momentum(
        L.handle, _ptr(sbits, "sbits", (torch.int64,), (L.W,)),
        _ptr(sscale, "sscale", f32, (L.n_sseg,)), _ptr(m, "m", f32, (L.d,)), _stream(stream))
    _check(rc, "oba_server_momentum")


def compress_deferred(L: Layout, g, m, c, wbits, wscale, beta1, sbits_prev=None,
                      sscale_prev=None, stream=None):
    """c: last step's compensated vectors in, this step's out; wscale: last
    step's worker scales in, this step's out.  The momentum is m, or (m=None)
    the last server message (sbits_prev, sscale_prev)."""
    import torch

    f32 = (torch.float32,)
    P = ctypes.c_void_p
    mp = _ptr(m, "m", f32, (L.d,)) if m is not None else P(None)
    bp = (_ptr(sbits_prev, "sbits_prev", (torch.int64,), (L.W,)) if sbits_prev is not None
          else P(None))
    sp = (_ptr(sscale_prev, "sscale_prev", f32, (L.n_sseg,)) if sscale_prev is not None
          else P(None))
    rc = lib().oba_compress_deferred(
        L.handle, _ptr(g, "g", _gtypes(), (L.n, L.ld)), _gdtype(g),
        mp, bp, sp, _ptr(c, "c", f32, (L.n, L.ld)),
        _ptr(wbits, "wbits", (torch.int64,), (L.n, L.W)),
        _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)), beta1,
        ctypes.c_void_p(L.ws.data_ptr()), L.ws_bytes, _stream(stream))
    _check(rc, "oba_compress_deferred")


def compress_deferred_noalloc(L: Layout, g, m, c, wbits, wscale, beta1, sbits_prev=None,
                              sscale_prev=None, stream=None):
    """compress_deferred without a workspace: the library's fixed device
    scratch holds the partial sums (for callers that cannot allocate)."""
    import torch

    f32 = (torch.float32,)
    P = ctypes.c_void_p
    mp = _ptr(m, "m", f32, (L.d,)) if m is not None else P(None)
    bp = (_ptr(sbits_prev, "sbits_prev", (torch.int64,), (L.W,)) if sbits_prev is not None
          else P(None))
    sp = (_ptr(sscale_prev, "sscale_prev", f32, (L.n_sseg,)) if sscale_prev is not None
          else P(None))
    rc = lib().oba_compress_deferred_noalloc(
        L.handle, _ptr(g, "g", _gtypes(), (L.n, L.ld)), _gdtype(g),
        mp, bp, sp, _ptr(c, "c", f32, (L.n, L.ld)),
        _ptr(wbits, "wbits", (torch.int64,), (L.n, L.W)),
        _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)), beta1, _stream(stream))
    _check(rc, "oba_compress_deferred_noalloc")


def compress_deferred16(L: Layout, g, m, c16, wbits, wscale, beta1, sbits_prev=None,
                        sscale_prev=None, stream=None):
    """As compress_deferred with a 16-bit state: c16 [n][ld] torch.float16
    (binary16) or torch.bfloat16, in (last c) / out (this c, rounded to the
    format before it is compressed)."""
    import torch

    f32 = (torch.float32,)
    P = ctypes.c_void_p
    mp = _ptr(m, "m", f32, (L.d,)) if m is not None else P(None)
    bp = (_ptr(sbits_prev, "sbits_prev", (torch.int64,), (L.W,)) if sbits_prev is not None
          else P(None))
    sp = (_ptr(sscale_prev, "sscale_prev", f32, (L.n_sseg,)) if sscale_prev is not None
          else P(None))
    cp = _ptr(c16, "c16", (torch.float16, torch.bfloat16), (L.n, L.ld))
    rc = lib().oba_compress_deferred16(
        L.handle, _ptr(g, "g", _gtypes(), (L.n, L.ld)), _gdtype(g),
        mp, bp, sp, cp, _gdtype(c16),
        _ptr(wbits, "wbits", (torch.int64,), (L.n, L.W)),
        _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)), beta1,
        ctypes.c_void_p(L.ws.data_ptr()), L.ws_bytes, _stream(stream))
    _check(rc, "oba_compress_deferred16")


def compress_deferred_local(L: Layout, g, m_local, c, wbits, wscale, beta1, stream=None):
    """Per-worker momentum: m_local [n][ld] and c [n][ld] in/out."""
    import torch

    f32 = (torch.float32,)
    rc = lib().oba_compress_deferred_local(
        L.handle, _ptr(g, "g", _gtypes(), (L.n, L.ld)), _gdtype(g),
        _ptr(m_local, "m_local", f32, (L.n, L.ld)), _ptr(c, "c", f32, (L.n, L.ld)),
        _ptr(wbits, "wbits", (torch.int64,), (L.n, L.W)),
        _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)), beta1,
        ctypes.c_void_p(L.ws.data_ptr()), L.ws_bytes, _stream(stream))
    _check(rc, "oba_compress_deferred_local")


def server_reduce_recompress_deferred(L: Layout, wbits, wscale, a, sbits, sscale, stream=None):
    """a: last step's server vector in, this step's out; sscale: last step's
    server scales in, this step's out."""
    import torch

    f32 = (torch.float32,)
    rc = lib().oba_server_reduce_recompress_deferred(
        L.handle, _ptr(wbits, "wbits", (torch.int64,), (L.n, L.W)),
        _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)), _ptr(a, "a", f32, (L.d,)),
        _ptr(sbits, "sbits", (torch.int64,), (L.W,)), _ptr(sscale, "sscale", f32, (L.n_sseg,)),
        ctypes.c_void_p(L.ws.data_ptr()), L.ws_bytes, _stream(stream))
    _check(rc, "oba_server_reduce_recompress_deferred")


def deferred_errors(L: Layout, c, wscale, a, sscale, delta=None, eps=None, stream=None):
    """delta = c - s*sign(c) and/or eps = a - sbar*sign(a), out of place."""
    import torch

    f32 = (torch.float32,)
    P = ctypes.c_void_p
    dp = _ptr(delta, "delta", f32, (L.n, L.ld)) if delta is not None else P(None)
    ep = _ptr(eps, "eps", f32, (L.d,)) if eps is not None else P(None)
    cp = _ptr(c, "c", f32, (L.n, L.ld)) if delta is not None else P(None)
    wp = _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)) if delta is not None else P(None)
    ap = _ptr(a, "a", f32, (L.d,)) if eps is not None else P(None)
    sp = _ptr(sscale, "sscale", f32, (L.n_sseg,)) if eps is not None else P(None)
    _check(lib().oba_deferred_errors(L.handle, cp, wp, ap, sp, dp, ep, _stream(stream)),
           "oba_deferred_errors")


class TensorList:
    """Model tensors in their own allocations (oba_tensors): x as a list of T
    float32 CUDA tensors, the gradients as n lists (one per worker) of T
    tensors of the same lengths.  Keeps references to every tensor."""

    def __init__(self, L: Layout, xs, gs):
        import numpy as np
        import torch

        self.L = L
        self.xs = list(xs)
        self.gs = [list(row) for row in gs]
        T = len(self.xs)
        if len(self.gs) != L.n or any(len(row) != T for row in self.gs):
            raise ValueError("gs must hold n rows of T tensors")
        gdt = self.gs[0][0].dtype if T else torch.float32
        self.g_dtype = _gdtype(self.gs[0][0]) if T else OBA_F32
        lengths = np.array([t.numel() for t in self.xs], dtype=np.int64)
        for t, x in enumerate(self.xs):
            _ptr(x, f"x[{t}]", (torch.float32,))
            for i in range(L.n):
                g = self.gs[i][t]
                _ptr(g, f"g[{i}][{t}]", (gdt,))
                if g.numel() != x.numel():
                    raise ValueError(f"g[{i}][{t}] length differs from x[{t}]")
        self.lengths = lengths
        xp = (ctypes.c_void_p * max(T, 1))(*[x.data_ptr() for x in self.xs])
        gp = (ctypes.c_void_p * max(L.n * T, 1))(*[g.data_ptr() for row in self.gs for g in row])
        h = ctypes.c_void_p()
        _check(lib().oba_tensors_create(ctypes.byref(h), L.handle, T,
                                        lengths.ctypes.data_as(ctypes.c_void_p), xp, gp,
                                        self.g_dtype), "oba_tensors_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().oba_tensors_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _same_layout(L: Layout, TLs: TensorList):
    """A tensor list's device tables belong to the layout it was made with
    (the library refuses any other with OBA_EINVAL as well)."""
    if TLs.L is not L:
        raise ValueError("the tensor list was made for another layout")


def adam_warmup_step_listed(L: Layout, TLs: TensorList, m, v, lr, beta1, beta2, eta, bc1=1.0,
                            bc2=1.0, vnorm=None, stream=None):
    _same_layout(L, TLs)
    import torch

    f32 = (torch.float32,)
    vp = _ptr(vnorm, "vnorm", (torch.float64,), (1,)) if vnorm is not None else ctypes.c_void_p()
    rc = lib().oba_adam_warmup_step_listed(
        L.handle, TLs.handle, _ptr(m, "m", f32, (L.d,)), _ptr(v, "v", f32, (L.d,)), lr, beta1,
        beta2, eta, bc1, bc2, vp, ctypes.c_void_p(L.ws.data_ptr()), L.ws_bytes, _stream(stream))
    _check(rc, "oba_adam_warmup_step_listed")


def compress_deferred_listed(L: Layout, TLs: TensorList, m, c, wbits, wscale, beta1,
                             sbits_prev=None, sscale_prev=None, stream=None):
    _same_layout(L, TLs)
    import torch

    f32 = (torch.float32,)
    P = ctypes.c_void_p
    mp = _ptr(m, "m", f32, (L.d,)) if m is not None else P(None)
    bp = (_ptr(sbits_prev, "sbits_prev", (torch.int64,), (L.W,)) if sbits_prev is not None
          else P(None))
    sp = (_ptr(sscale_prev, "sscale_prev", f32, (L.n_sseg,)) if sscale_prev is not None
          else P(None))
    rc = lib().oba_compress_deferred_listed(
        L.handle, TLs.handle, mp, bp, sp, _ptr(c, "c", f32, (L.n, L.ld)),
        _ptr(wbits, "wbits", (torch.int64,), (L.n, L.W)),
        _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)), beta1,
        ctypes.c_void_p(L.ws.data_ptr()), L.ws_bytes, _stream(stream))
    _check(rc, "oba_compress_deferred_listed")


def compress_deferred16_listed(L: Layout, TLs: TensorList, m, c16, wbits, wscale, beta1,
                               sbits_prev=None, sscale_prev=None, stream=None):
    """compress_deferred16 on the listed gradients (c16 [n][ld] float16 or
    bfloat16, flat)."""
    _same_layout(L, TLs)
    import torch

    f32 = (torch.float32,)
    P = ctypes.c_void_p
    mp = _ptr(m, "m", f32, (L.d,)) if m is not None else P(None)
    bp = (_ptr(sbits_prev, "sbits_prev", (torch.int64,), (L.W,)) if sbits_prev is not None
          else P(None))
    sp = (_ptr(sscale_prev, "sscale_prev", f32, (L.n_sseg,)) if sscale_prev is not None
          else P(None))
    rc = lib().oba_compress_deferred16_listed(
        L.handle, TLs.handle, mp, bp, sp,
        _ptr(c16, "c16", (torch.float16, torch.bfloat16), (L.n, L.ld)), _gdtype(c16),
        _ptr(wbits, "wbits", (torch.int64,), (L.n, L.W)),
        _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)), beta1,
        ctypes.c_void_p(L.ws.data_ptr()), L.ws_bytes, _stream(stream))
    _check(rc, "oba_compress_deferred16_listed")


def decompress_update_listed(L: Layout, TLs: TensorList, sbits, sscale, denom, m, lr,
                             stream=None):
    _same_layout(L, TLs)
    import torch

    f32 = (torch.float32,)
    mp = _ptr(m, "m", f32, (L.d,)) if m is not None else ctypes.c_void_p(None)
    rc = lib().oba_decompress_update_listed(
        L.handle, TLs.handle, _ptr(sbits, "sbits", (torch.int64,), (L.W,)),
        _ptr(sscale, "sscale", f32, (L.n_sseg,)), _ptr(denom, "denom", f32, (L.d,)), mp, lr,
        _stream(stream))
    _check(rc, "oba_decompress_update_listed")


def step_small(L: Layout, g, m, c, wbits, wscale, a, sbits, sscale, denom, m_out, x, beta1, lr,
               stream=None):
    """The whole deferred step in one launch (small layouts).  m=None: the
    implicit momentum in (sbits, sscale); m_out=None: m not stored."""
    import torch

    f32 = (torch.float32,)
    P = ctypes.c_void_p
    rc = lib().oba_step_small(
        L.handle, _ptr(g, "g", _gtypes(), (L.n, L.ld)), _gdtype(g),
        _ptr(m, "m", f32, (L.d,)) if m is not None else P(None),
        _ptr(c, "c", f32, (L.n, L.ld)), _ptr(wbits, "wbits", (torch.int64,), (L.n, L.W)),
        _ptr(wscale, "wscale", f32, (L.n, L.n_wseg)), _ptr(a, "a", f32, (L.d,)),
        _ptr(sbits, "sbits", (torch.int64,), (L.W,)), _ptr(sscale, "sscale", f32, (L.n_sseg,)),
        _ptr(denom, "denom", f32, (L.d,)),
        _ptr(m_out, "m_out", f32, (L.d,)) if m_out is not None else P(None),
        _ptr(x, "x", f32, (L.d,)), beta1, lr, _stream(stream))
    _check(rc, "oba_step_small")


def timing_enable(on=True, capacity=4096):
    _check(lib().oba_timing_enable(1 if on else 0, capacity), "oba_timing_enable")


def timing_read(kernel: str):
    ms = ctypes.c_double()
    cnt = ctypes.c_int64()
    _check(lib().oba_timing_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(cnt)),
           "oba_timing_read")
    return ms.value, cnt.value


def timing_reset():
    _check(lib().oba_timing_reset(), "oba_timing_reset")


class State:
    """Device buffers of one simulated data-parallel job (allocation only)."""

    def __init__(self, L: Layout, g_dtype="f32"):
        import torch

        dev = "cuda"
        f = torch.float32
        self.L = L
        gt = {"f16": torch.float16, "bf16": torch.bfloat16}.get(g_dtype, f)
        self.g = torch.zeros((L.n, L.ld), dtype=gt, device=dev)
        self.x = torch.zeros(L.d, dtype=f, device=dev)
        self.m = torch.zeros(L.d, dtype=f, device=dev)
        self.v = torch.zeros(L.d, dtype=f, device=dev)
        self.denom = torch.zeros(L.d, dtype=f, device=dev)
        self.eps = torch.zeros(L.d, dtype=f, device=dev)
        self.delta = torch.zeros((L.n, L.ld), dtype=f, device=dev)
        self.wbits = torch.zeros((L.n, L.W), dtype=torch.int64, device=dev)
        self.wscale = torch.zeros((L.n, L.n_wseg), dtype=f, device=dev)
        self.sbits = torch.zeros(L.W, dtype=torch.int64, device=dev)
        self.sscale = torch.zeros(L.n_sseg, dtype=f, device=dev)

        # True while m is implicit: the momentum is sbar*sign of (sbits,
        # sscale) and the buffer m is stale (see oba_compress_deferred)
        self.m_implicit = False

    def momentum(self):
        """The momentum every worker holds, written to self.m if implicit."""
        if self.m_implicit:
            server_momentum(self.L, self.sbits, self.sscale, self.m)
        return self.m

    def _explicit_m(self):
        self.momentum()
        self.m_implicit = False

    def warmup(self, lr, beta1, beta2, eta, bc1=1.0, bc2=1.0, g=None, vnorm=None):
        """One warm-up step; with vnorm (float64 [1] CUDA tensor) also ||v||_2."""
        self._explicit_m()
        g = self.g if g is None else g
        if vnorm is None:
            adam_warmup_step(self.L, g, self.x, self.m, self.v, lr, beta1, beta2, eta, bc1, bc2)
        else:
            adam_warmup_step_vnorm(self.L, g, self.x, self.m, self.v, lr, beta1, beta2, eta,
                                   vnorm, bc1, bc2)

    def freeze(self, eta, bc2=1.0):
        """End of the warm-up: denom from v; errors (or, in the deferred
        layout, the stored c, a and the scales) start at zero."""
        freeze_variance(self.L, self.v, self.denom, eta, bc2)
        self.start_compression()

    def start_compression(self):
        """State of the first compression step: m explicit, errors (or the
        stored c, a) and scales zero."""
        self._explicit_m()
        if self.delta is not None:
            self.delta.zero_()
        if getattr(self, "c16", None) is not None:
            self.c16.zero_()
        self.eps.zero_()
        self.wscale.zero_()
        self.sscale.zero_()

    def step(self, beta1, lr, g=None):
        """One compression step: compress -> server -> decompress+update."""
        self._rows32()
        self._explicit_m()
        compress(self.L, self.g if g is None else g, self.m, self.delta, self.wbits, self.wscale,
                 beta1)
        server_reduce_recompress(self.L, self.wbits, self.wscale, self.eps, self.sbits,
                                 self.sscale)
        decompress_update(self.L, self.sbits, self.sscale, self.denom, self.m, self.x, lr)

    def start_local_momentum(self):
        """Per-worker momentum from here on: every worker's m_i starts as the
        shared m (call after the freeze)."""
        import torch

        self.m_local = self.momentum().unsqueeze(0).repeat(self.L.n, 1)
        if self.L.ld != self.L.d:
            self.m_local = torch.nn.functional.pad(self.m_local, (0, self.L.ld - self.L.d))
        self.m_local = self.m_local.contiguous()

    def step_local(self, beta1, lr, g=None):
        """A compression step with per-worker momentum (deferred layout): the
        broadcast m_hat moves x; each worker keeps its own m_i."""
        self._rows32()
        compress_deferred_local(self.L, self.g if g is None else g, self.m_local, self.delta,
                                self.wbits, self.wscale, beta1)
        server_reduce_recompress_deferred(self.L, self.wbits, self.wscale, self.eps, self.sbits,
                                          self.sscale)
        decompress_update(self.L, self.sbits, self.sscale, self.denom, None, self.x, lr)

    def step_small(self, beta1, lr, g=None, implicit_m=True):
        """step_deferred in one launch (layouts of at most 65536 coordinates)."""
        self._rows32()
        step_small(self.L, self.g if g is None else g, None if self.m_implicit else self.m,
                   self.delta, self.wbits, self.wscale, self.eps, self.sbits, self.sscale,
                   self.denom, None if implicit_m else self.m, self.x, beta1, lr)
        self.m_implicit = implicit_m

    def start_state16(self, kind="bf16"):
        """Hold the workers' compensated vectors in a 16-bit format ("f16"
        binary16 or "bf16" bfloat16) for step_deferred16: c16 [n][ld] zero,
        scales zero, m explicit (the warm-up's); frees the binary32 rows."""
        import torch

        dt = {"f16": torch.float16, "bf16": torch.bfloat16}[kind]
        self.delta = None
        self.c16 = torch.zeros((self.L.n, self.L.ld), dtype=dt, device="cuda")
        self.start_compression()

    def step_deferred16(self, beta1, lr, g=None):
        """The deferred step with the 16-bit worker state c16 (see
        oba_compress_deferred16); the momentum stays implicit."""
        g = self.g if g is None else g
        if self.m_implicit:
            compress_deferred16(self.L, g, None, self.c16, self.wbits, self.wscale, beta1,
                                self.sbits, self.sscale)
        else:
            compress_deferred16(self.L, g, self.m, self.c16, self.wbits, self.wscale, beta1)
        server_reduce_recompress_deferred(self.L, self.wbits, self.wscale, self.eps, self.sbits,
                                          self.sscale)
        decompress_update(self.L, self.sbits, self.sscale, self.denom, None, self.x, lr)
        self.m_implicit = True

    def _rows32(self):
        if self.delta is None:
            raise RuntimeError("the binary32 worker rows were released by start_state16(); "
                               "use step_deferred16() or a new State")

    def step_deferred(self, beta1, lr, g=None, implicit_m=True):
        """The same step in the deferred-residual layout: `delta` holds the
        last c and `eps` the last a (see oba_compress_deferred).  With
        implicit_m the update does not store m and the next step rebuilds it
        from the server message; momentum() writes it out."""
        self._rows32()
        g = self.g if g is None else g
        if self.m_implicit:
            compress_deferred(self.L, g, None, self.delta, self.wbits, self.wscale, beta1,
                              self.sbits, self.sscale)
        else:
            compress_deferred(self.L, g, self.m, self.delta, self.wbits, self.wscale, beta1)
        server_reduce_recompress_deferred(self.L, self.wbits, self.wscale, self.eps, self.sbits,
                                          self.sscale)
        decompress_update(self.L, self.sbits, self.sscale, self.denom,
                          None if implicit_m else self.m, self.x, lr)
        self.m_implicit = implicit_m
