"""CPU oracle of the 1-bit Adam compression-stage step (numpy front end).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  The
arithmetic lives in ``oracle.c`` (plain C, single thread, built with
``-O2 -ffp-contract=off``); this module only marshals numpy arrays.  It
imports nothing of the GPU package.

Every array argument is a C-contiguous numpy array; state is float32,
gradients float32 or float16, packed signs uint64, segment tables int64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (seconds), also when a source is newer."""
    stale = not os.path.exists(_LIB_PATH) or any(
        os.path.getmtime(os.path.join(_HERE, f)) > os.path.getmtime(_LIB_PATH)
        for f in ("oracle.c", "oracle.h"))
    if force or stale:
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I32, F, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
        I = ctypes.c_int
        sig = {
            "oracle_half_to_double": (D, [ctypes.c_uint16]),
            "oracle_bfloat16_to_double": (D, [ctypes.c_uint16]),
            "oracle_adam_warmup_step": (None, [I64, I32, I64, P, I, P, P, P, D, D, D, D, D, D]),
            "oracle_freeze_variance": (None, [I64, P, P, D, D]),
            "oracle_l2norm": (D, [I64, P]),
            "oracle_plateau_first": (I64, [I64, P, I32, D, I32]),
            "oracle_sumsq": (D, [I64, P]),
            "oracle_scale": (F, [D, I64]),
            "oracle_pack_signs": (None, [I64, P, P, I64]),
            "oracle_bit": (I, [P, I64]),
            "oracle_residual": (None, [I64, P, F, P]),
            "oracle_compensate": (None, [I64, D, P, P, I, I64, P, P]),
            "oracle_compress": (None, [I64, I32, I64, P, I32, P, I, P, P, P, P, D]),
            "oracle_compress_local": (None, [I64, I32, I64, P, I32, P, I, P, P, P, P, D]),
            "oracle_server_average": (None, [I64, I64, I64, I32, P, I32, P, P, P, P]),
            "oracle_server_reduce_recompress": (None, [I64, I32, P, I32, P, I32, P, P, P, P, P]),
            "oracle_decompress_update": (None, [I64, I64, P, I32, P, P, P, P, P, D]),
            "oracle_float_to_half": (ctypes.c_uint16, [F]),
            "oracle_float_to_bfloat16": (ctypes.c_uint16, [F]),
            "oracle_round16": (None, [I64, P, P, I]),
            "oracle_compress_deferred16": (None, [I64, I32, I64, P, I32, P, I, P, P, I, P, P, P,
                                                  D]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _chk(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"{name}: expected C-contiguous numpy {np.dtype(dtype).name}")


class BF16(np.ndarray):
    """bfloat16 gradients: a uint16 array of bfloat16 bit patterns
    (``oracle.bf16(bits)``); numpy has no bfloat16 type."""


def bf16(bits: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return a.view(BF16)


def _grad(g):
    if isinstance(g, BF16):
        return 2
    if g.dtype == np.float16:
        return 1
    if g.dtype == np.float32:
        return 0
    raise TypeError("gradients must be float32, float16 or oracle.bf16(bits)")


def words(d: int) -> int:
    return (d + 63) // 64


def _seg(seg, d):
    seg = np.ascontiguousarray(seg, dtype=np.int64)
    if seg.ndim != 1 or len(seg) < 2 or seg[0] != 0 or seg[-1] != d or np.any(np.diff(seg) <= 0):
        raise ValueError("segment table must rise strictly from 0 to d")
    return seg


def bfloat16_to_float(h: int) -> float:
    return lib().oracle_bfloat16_to_double(h)


def half_to_float(h: int) -> float:
    return lib().oracle_half_to_double(int(h) & 0xFFFF)


def adam_warmup_step(g, x, m, v, lr, beta1, beta2, eta, bc1=1.0, bc2=1.0):
    """In place on x, m, v.  g: [n][ld] float32/float16 (ld >= d)."""
    d = x.shape[0]
    n, ld = g.shape
    for a, nm in ((x, "x"), (m, "m"), (v, "v")):
        _chk(a, np.float32, nm)
    lib().oracle_adam_warmup_step(d, n, ld, _p(g), _grad(g), _p(x), _p(m), _p(v), lr, beta1,
                                  beta2, eta, bc1, bc2)


def freeze_variance(v, eta, bc2=1.0):
    _chk(v, np.float32, "v")
    denom = np.empty_like(v)
    lib().oracle_freeze_variance(v.shape[0], _p(v), _p(denom), eta, bc2)
    return denom


def l2norm(v):
    """sqrt(sum v_k^2) in binary64 (the fused variance norm)."""
    _chk(v, np.float32, "v")
    return lib().oracle_l2norm(v.size, _p(v))


def plateau_first(h, window, rtol, min_steps=0):
    """First 1-based step at which the series h has levelled off, or 0."""
    h = np.ascontiguousarray(np.asarray(h, dtype=np.float64))
    return int(lib().oracle_plateau_first(h.size, _p(h), window, rtol, min_steps))


def compensate(beta1, m, g_row, delta_row):
    """c = (b1*m + (1-b1)*g) + delta for one worker row (any length)."""
    c = np.empty(m.shape[0], np.float32)
    lib().oracle_compensate(m.shape[0], beta1, _p(m), _p(g_row), _grad(g_row), 0, _p(delta_row),
                            _p(c))
    return c


def sumsq(c):
    _chk(c, np.float32, "c")
    return lib().oracle_sumsq(c.shape[0], _p(c))


def scale(sumsq_value, length):
    return lib().oracle_scale(float(sumsq_value), int(length))


def pack_signs(c, d=None, bit0=0):
    _chk(c, np.float32, "c")
    d = c.shape[0] + bit0 if d is None else d
    bits = np.zeros(words(d), np.uint64)
    lib().oracle_pack_signs(c.shape[0], _p(c), _p(bits), bit0)
    return bits


def residual(c, s):
    _chk(c, np.float32, "c")
    err = np.empty_like(c)
    lib().oracle_residual(c.shape[0], _p(c), s, _p(err))
    return err


def compress(g, m, delta, wseg, beta1):
    """Worker compression for all n rows.  delta [n][ld] is updated in place.
    Returns (wbits [n][W] uint64, wscale [n][n_wseg] float32)."""
    n, ld = g.shape
    d = m.shape[0]
    _chk(m, np.float32, "m")
    _chk(delta, np.float32, "delta")
    assert delta.shape == (n, ld)
    wseg = _seg(wseg, d)
    wbits = np.zeros((n, words(d)), np.uint64)
    wscale = np.zeros((n, len(wseg) - 1), np.float32)
    lib().oracle_compress(d, n, ld, _p(wseg), len(wseg) - 1, _p(g), _grad(g), _p(m), _p(delta),
                          _p(wbits), _p(wscale), beta1)
    return wbits, wscale


KIND16 = {"f16": 1, "bf16": 2}


def round16(x, kind):
    """binary32 array -> uint16 bit patterns of the nearest binary16 ("f16")
    or bfloat16 ("bf16") values, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_round16(x.size, _p(x), _p(out), KIND16[kind])
    return out


_DECODE16 = {}


def decode16(bits, kind):
    """uint16 bit patterns of binary16 / bfloat16 values -> binary32 (exact),
    through a table of the oracle's decoders over all 65 536 patterns."""
    if kind not in _DECODE16:
        f = half_to_float if kind == "f16" else bfloat16_to_float
        _DECODE16[kind] = np.array([f(h) for h in range(65536)], dtype=np.float64).astype(
            np.float32)
    return _DECODE16[kind][np.asarray(bits, dtype=np.uint16)]


def compress_deferred16(g, m, c16, kind, wscale_prev, wseg, beta1):
    """Worker compression with each worker's compensated momentum held in a
    16-bit format: c16 [n][ld] uint16 (the last compressed vectors) is
    updated in place, wscale_prev [n][n_wseg] holds their scales.  Returns
    (wbits [n][W] uint64, wscale [n][n_wseg] float32)."""
    n, ld = g.shape
    d = m.shape[0]
    _chk(m, np.float32, "m")
    _chk(c16, np.uint16, "c16")
    _chk(wscale_prev, np.float32, "wscale_prev")
    assert c16.shape == (n, ld)
    wseg = _seg(wseg, d)
    assert wscale_prev.shape == (n, len(wseg) - 1)
    wbits = np.zeros((n, words(d)), np.uint64)
    wscale = np.zeros((n, len(wseg) - 1), np.float32)
    lib().oracle_compress_deferred16(d, n, ld, _p(wseg), len(wseg) - 1, _p(g), _grad(g), _p(m),
                                     _p(c16), KIND16[kind], _p(wscale_prev), _p(wbits),
                                     _p(wscale), beta1)
    return wbits, wscale


def compress_local(g, m_local, delta, wseg, beta1):
    """Worker compression with per-worker momentum: m_local and delta [n][ld]
    are updated in place.  Returns (wbits, wscale)."""
    n, ld = g.shape
    _chk(m_local, np.float32, "m_local")
    _chk(delta, np.float32, "delta")
    assert m_local.shape == (n, ld) and delta.shape == (n, ld)
    d = int(wseg[-1])
    wseg = _seg(wseg, d)
    wbits = np.zeros((n, words(d)), np.uint64)
    wscale = np.zeros((n, len(wseg) - 1), np.float32)
    lib().oracle_compress_local(d, n, ld, _p(wseg), len(wseg) - 1, _p(g), _grad(g), _p(m_local),
                                _p(delta), _p(wbits), _p(wscale), beta1)
    return wbits, wscale


def server_average(wbits, wscale, wseg, eps, k0=0, k1=None):
    """a[k] for k in [k0, k1) (other entries of the returned array are 0)."""
    n = wbits.shape[0]
    d = eps.shape[0]
    k1 = d if k1 is None else k1
    wseg = _seg(wseg, d)
    _chk(wbits, np.uint64, "wbits")
    _chk(wscale, np.float32, "wscale")
    a = np.zeros(d, np.float32)
    lib().oracle_server_average(k0, k1, d, n, _p(wseg), len(wseg) - 1, _p(wbits), _p(wscale),
                                _p(eps), _p(a))
    return a


def server_reduce_recompress(wbits, wscale, wseg, sseg, eps):
    """eps [d] updated in place.  Returns (sbits [W] uint64, sscale [n_sseg])."""
    n = wbits.shape[0]
    d = eps.shape[0]
    _chk(eps, np.float32, "eps")
    _chk(wbits, np.uint64, "wbits")
    _chk(wscale, np.float32, "wscale")
    wseg = _seg(wseg, d)
    sseg = _seg(sseg, d)
    sbits = np.zeros(words(d), np.uint64)
    sscale = np.zeros(len(sseg) - 1, np.float32)
    lib().oracle_server_reduce_recompress(d, n, _p(wseg), len(wseg) - 1, _p(sseg), len(sseg) - 1,
                                          _p(wbits), _p(wscale), _p(eps), _p(sbits), _p(sscale))
    return sbits, sscale


def decompress_update(sbits, sscale, sseg, denom, m, x, lr, k0=0, k1=None):
    """m, x updated in place on [k0, k1)."""
    d = x.shape[0]
    k1 = d if k1 is None else k1
    for a, nm in ((denom, "denom"), (m, "m"), (x, "x")):
        _chk(a, np.float32, nm)
    sseg = _seg(sseg, d)
    lib().oracle_decompress_update(k0, k1, _p(sseg), len(sseg) - 1, _p(sbits), _p(sscale),
                                   _p(denom), _p(m), _p(x), lr)


def bit(bits, k):
    return lib().oracle_bit(_p(bits), int(k))


def step(state, g, wseg, sseg, beta1, lr):
    """One compression step on a dict state {m, delta, eps, denom, x}; with
    "m_local" ([n][ld]) in the state, the per-worker-momentum variant (m_hat
    then only moves x).  Returns the messages (wbits, wscale, sbits, sscale)."""
    if "m_local" in state:
        wbits, wscale = compress_local(g, state["m_local"], state["delta"], wseg, beta1)
    else:
        wbits, wscale = compress(g, state["m"], state["delta"], wseg, beta1)
    sbits, sscale = server_reduce_recompress(wbits, wscale, wseg, sseg, state["eps"])
    m_hat = state["m"] if "m" in state else np.zeros_like(state["x"])
    decompress_update(sbits, sscale, sseg, state["denom"], m_hat, state["x"], lr)
    return wbits, wscale, sbits, sscale
