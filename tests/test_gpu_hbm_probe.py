"""GPU check of the streaming probes behind bench.py's HBM ceiling
(libhbmstream.so): the bytes a probe is credited with are the bytes it moves,
so its stores must land where and as its shape says (every element of every
written row, each value a function of the values loaded), and every row it
loads must reach a stored value (else the compiler may drop that load)."""
import ctypes
import sys

import pytest

import bench
from gpu_common import torch

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name,buf,bpc", [("copy", 0, 0), ("copy", 1, 4), ("worker_g16", 0, 0),
                                          ("worker_g16", 1, 3), ("in_place", 1, 0),
                                          ("write", 0, 8), ("state16", 1, 0),
                                          ("warmup_g16", 0, 0), ("update", 1, 0),
                                          ("worker_g16", 2, 0), ("state16", 3, 3),
                                          ("warmup_g16", 1, 2), ("read", 0, 0),
                                          ("worker_g16_x1", 1, 2), ("worker_g16_x2", 3, 0),
                                          ("worker_g16_x8", 0, 3), ("state16_x1", 1, 0),
                                          ("state16_x1", 2, 3), ("worker_g32_x1", 1, 0)])
def test_probe_stores_what_its_shape_says(name, buf, bpc):
    t = torch()
    lib = bench.probe_lib()
    shape, groups = bench.PROBES[name]
    groups = groups or 2
    info = (ctypes.c_int32 * 5)()
    assert lib.hbm_stream_shape(shape, info) == 0
    na, ab, nb, bb, mode = list(info)
    spans = 5
    ld = spans * 2048 + 8  # rows longer than the spans: the tail must stay untouched
    say(f"[hbm probe] {name} buffer={buf} rows a={groups * na} b={groups * nb}")
    dt = {2: t.float16, 4: t.float32}
    a = (t.rand((max(1, groups * na), ld), device="cuda") + 1.0).to(dt[ab])
    b0 = (t.rand((max(1, groups * nb), ld), device="cuda") + 2.0).to(dt[bb])
    b = b0.clone()
    sink = t.zeros(1, device="cuda")
    st = t.cuda.current_stream()
    rc = lib.hbm_stream_launch(shape, buf, ctypes.c_void_p(a.data_ptr()),
                               ctypes.c_void_p(b.data_ptr()), ld, spans, groups, bpc,
                               ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st.cuda_stream))
    assert rc == 0
    t.cuda.synchronize()
    n = spans * 2048
    af, bf, b0f = a.float(), b.float(), b0.float()
    for gi in range(groups):
        for u in range(nb):
            r = gi * nb + u
            acc = b0f[r, :n].clone() if mode == 2 else t.zeros(n, device="cuda")
            if na == 0:  # element j (0..7) of the lane's two quads: k % 4, +4 in the upper half
                k = t.arange(n, device="cuda")
                acc = acc + (k.remainder(4) + 4 * (k.remainder(2048) >= 1024).long()).float()
            elif u >= na:
                acc = acc + af[gi * na + u % na, :n]
            else:  # every A row reaches a stored row: u, u + nb, u + 2 nb, ... in that order
                for kk in range(u, na, nb):
                    acc = acc + af[gi * na + kk, :n]
            want = (acc + 1.0).to(dt[bb]).float()
            assert t.equal(bf[r, :n], want), f"row {r}"
            assert t.equal(bf[r, n:], b0f[r, n:]), f"row {r}: past the spans"
    assert float(sink.item()) == 0.0
