"""Degenerate inputs of the method on the GPU, against the oracle: an
all-zero step (every scale 0, every sign +1, x unchanged), a single nonzero
coordinate, the largest binary16 magnitudes, and argument errors of the
later entry points."""
import ctypes
import sys

import numpy as np
import pytest

import oracle
from gpu_common import B1, B2, ETA, LR, assert_close, assert_words, padded, to_dev, to_host, torch
from communication_compressed_optimizer_02_amd import binding as oba
from communication_compressed_optimizer_02_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def one_step(d, n, g, m, denom, x, wseg, sseg):
    """Teacher-forced explicit step on both sides from zero errors."""
    L = oba.Layout(d, n, wseg, sseg)
    st = dict(x=x.copy(), m=m.copy(), delta=np.zeros((n, d), np.float32),
              eps=np.zeros(d, np.float32), denom=denom)
    wb, ws, sb, ss = oracle.step(st, g, wseg, sseg, B1, LR)
    gdt = "f16" if g.dtype == np.float16 else "f32"
    S = oba.State(L, gdt)
    S.m.copy_(torch().from_numpy(m))
    S.x.copy_(torch().from_numpy(x))
    S.denom.copy_(torch().from_numpy(denom))
    S.step(B1, LR, g=to_dev(padded(g, L.ld)))
    torch().cuda.synchronize()
    assert_words(to_host(S.wbits, np.uint64), wb, "worker words")
    assert_words(to_host(S.sbits, np.uint64), sb, "server words")
    assert_close(to_host(S.wscale), ws, "worker scales")
    assert_close(to_host(S.sscale), ss, "server scales")
    assert_close(to_host(S.x), st["x"], "x")
    assert_close(to_host(S.m), st["m"], "m")
    out = dict(wscale=to_host(S.wscale), sscale=to_host(S.sscale), x=to_host(S.x),
               wbits=to_host(S.wbits, np.uint64), sbits=to_host(S.sbits, np.uint64))
    L.close()
    return out


def test_all_zero_step_keeps_x_and_encodes_plus():
    d, n = 5000, 3
    say(f"[edge] all zero d={d} n={n}")
    z = np.zeros(d, np.float32)
    denom = np.full(d, ETA, np.float32)  # v = 0 at the freeze
    out = one_step(d, n, np.zeros((n, d), np.float32), z, denom, z + 0.5, synth.whole(d),
                   synth.even_shards(d, n))
    assert not out["wscale"].any() and not out["sscale"].any()
    assert not out["wbits"].any() and not out["sbits"].any()
    assert np.all(out["x"] == 0.5)


def test_single_nonzero_coordinate():
    d, n = 3000, 2
    say(f"[edge] one nonzero coordinate d={d} n={n}")
    g = np.zeros((n, d), np.float32)
    g[1, 1234] = -3.0
    z = np.zeros(d, np.float32)
    out = one_step(d, n, g, z, np.full(d, 1e-3, np.float32), z, synth.whole(d),
                   synth.even_shards(d, n))
    # worker 1: c = -0.3 at one coordinate, so s = 0.3/sqrt(d); worker 0 all zero
    assert out["wscale"][0, 0] == 0.0
    assert out["wscale"][1, 0] == np.float32(np.sqrt(np.float64(np.float32(0.1) * np.float32(-3.0)) ** 2 / d))


def test_largest_half_gradients():
    d, n = 4099, 8
    say(f"[edge] binary16 extremes d={d} n={n}")
    rng = np.random.default_rng(3)
    g = np.where(rng.random((n, d)) < 0.5, -65504.0, 65504.0).astype(np.float16)
    g[:, ::5] = np.float16(6e-8)
    m = rng.normal(0, 1.0, d).astype(np.float32)
    one_step(d, n, g, m, np.full(d, 1.0, np.float32), np.zeros(d, np.float32),
             synth.whole(d), synth.even_shards(d, n))


def test_later_entry_points_reject_bad_arguments():
    t = torch()
    L = oba.Layout(100, 2, synth.whole(100), synth.even_shards(100, 2))
    S = oba.State(L)
    lib = oba.lib()
    P = ctypes.c_void_p
    strm = P(t.cuda.current_stream().cuda_stream)
    ws = P(L.ws.data_ptr())
    # per-worker momentum: m_local and c may not be the same buffer
    assert lib.oba_compress_deferred_local(L.handle, P(S.g.data_ptr()), 0, P(S.delta.data_ptr()),
                                           P(S.delta.data_ptr()), P(S.wbits.data_ptr()),
                                           P(S.wscale.data_ptr()), B1, ws, L.ws_bytes,
                                           strm) == -1
    # bad gradient dtype and beta
    assert lib.oba_compress_deferred_local(L.handle, P(S.g.data_ptr()), 7, P(S.m.data_ptr()),
                                           P(S.delta.data_ptr()), P(S.wbits.data_ptr()),
                                           P(S.wscale.data_ptr()), B1, ws, L.ws_bytes,
                                           strm) == -1
    assert lib.oba_compress_deferred_local(L.handle, P(S.g.data_ptr()), 0, P(S.m.data_ptr()),
                                           P(S.delta.data_ptr()), P(S.wbits.data_ptr()),
                                           P(S.wscale.data_ptr()), 1.0, ws, L.ws_bytes,
                                           strm) == -1
    # server momentum: misaligned output, null message
    assert lib.oba_server_momentum(L.handle, P(S.sbits.data_ptr()), P(S.sscale.data_ptr()),
                                   P(S.m.data_ptr() + 4), strm) == -2
    assert lib.oba_server_momentum(L.handle, None, P(S.sscale.data_ptr()), P(S.m.data_ptr()),
                                   strm) == -1
    # update with m = NULL is allowed; a bad lr is not
    assert lib.oba_decompress_update(L.handle, P(S.sbits.data_ptr()), P(S.sscale.data_ptr()),
                                     P(S.denom.data_ptr()), None, P(S.x.data_ptr()),
                                     float("nan"), strm) == -1
    t.cuda.synchronize()
    L.close()
