"""Helpers of the full-size parity tests: a coordinate range followed by the
oracle beside a GPU run over all of d, and the comparison protocol with the
near-zero sign exemption.

Comparison (the method's tolerance): scales and binary32 values within 1e-6
absolute + 1e-5 relative; packed words bit-exact, except at a coordinate whose
encoded value is within 1e-6 of its scale (|c| < 1e-6 s for a worker,
|a| < 1e-6 s_bar for the server).  There the two sides may take different
signs when one scale rounds to the neighbouring binary32 (the scales are
binary64 sums in different orders), and the values computed from that sign
at that coordinate -- the worker's residual, the server average and its sign
and residual, m and x -- are left out of the value comparison, in that step
and the later steps of the same run.
"""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from gpu_common import B1, LR, assert_close


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def h(t):
    return np.ascontiguousarray(t.detach().cpu().numpy())


NEAR_ZERO = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def h(t):
    return np.ascontiguousarray(t.detach().cpu().numpy())


def local_table(seg, lo, hi):
    """Segments of `seg` inside [lo, hi) (which must be a union of them),
    shifted to start at 0, and the index range of those segments."""
    seg = np.asarray(seg, dtype=np.int64)
    j0 = int(np.searchsorted(seg, lo))
    j1 = int(np.searchsorted(seg, hi))
    assert seg[j0] == lo and seg[j1] == hi, "range must be a union of segments"
    return seg[j0:j1 + 1] - lo, j0, j1


def flipped(gw, ow):
    """Coordinates (bit positions) where two packed rows differ."""
    gw, ow = np.asarray(gw).view(np.uint64), np.asarray(ow).view(np.uint64)
    out = []
    for j in np.nonzero(gw != ow)[0]:
        x = int(gw[j]) ^ int(ow[j])
        while x:
            out.append(int(j) * 64 + ((x & -x).bit_length() - 1))
            x &= x - 1
    return np.array(out, dtype=np.int64)


def seg_index(seg, ks):
    return np.searchsorted(seg, ks, side="right") - 1


def close_except(gpu, ora, skip, what):
    """assert_close over the coordinates not in `skip`; bitwise-equal arrays
    (the common case) pass without the elementwise tolerance pass."""
    if skip.size:
        keep = np.ones(ora.shape[0], bool)
        keep[skip] = False
        gpu, ora = gpu[keep], ora[keep]
    if gpu.dtype == ora.dtype == np.float32 and np.array_equal(gpu.view(np.uint32),
                                                               ora.view(np.uint32)):
        return
    assert_close(gpu, ora, what)


class Range:
    """One coordinate range [lo, hi) (a union of worker and of server
    segments, lo a multiple of 64) followed on both sides."""

    def __init__(self, w, lo, hi):
        assert lo % 64 == 0 and (hi % 64 == 0 or hi == w.d)
        self.lo, self.hi = lo, hi
        self.wl, self.j0, self.j1 = local_table(w.wseg, lo, hi)
        self.sl, self.t0, self.t1 = local_table(w.sseg, lo, hi)
        self.w0, self.w1 = lo // 64, (hi + 63) // 64
        # coordinates whose state has diverged at an allowed sign difference
        # of an earlier step: their later values follow different inputs
        self.carry = np.zeros(hi - lo, bool)

    def oracle_step(self, st, g):
        """One oracle step on the range (st updated in place); returns its
        messages and the values it encoded (c per worker, a)."""
        n = g.shape[0]

        def worker(i):  # workers are independent: one oracle call each, in threads
            c_i = oracle.compensate(B1, st["m"], g[i], st["delta"][i])
            wb_i, ws_i = oracle.compress(g[i:i + 1], st["m"], st["delta"][i:i + 1], self.wl, B1)
            return c_i, wb_i[0], ws_i[0]

        with ThreadPoolExecutor(min(n, 8)) as ex:
            res = list(ex.map(worker, range(n)))
        c = np.stack([r[0] for r in res])
        wb = np.stack([r[1] for r in res])
        ws = np.stack([r[2] for r in res])
        del res
        a = oracle.server_average(wb, ws, self.wl, st["eps"])
        sb, ss = oracle.server_reduce_recompress(wb, ws, self.wl, self.sl, st["eps"])
        oracle.decompress_update(sb, ss, self.sl, st["denom"], st["m"], st["x"], LR)
        return dict(wbits=wb, wscale=ws, sbits=sb, sscale=ss, c=c, a=a)

    def compare(self, name, gpu, ora, st):
        """gpu: device tensors of the step's outputs over all of d (delta
        [n][ld] and eps materialised as errors); ora, st: the oracle's step
        outputs and state after it."""
        lo, hi = self.lo, self.hi
        n = ora["wbits"].shape[0]
        assert_close(h(gpu["wscale"][:, self.j0:self.j1]), ora["wscale"], "worker scales")
        assert_close(h(gpu["sscale"][self.t0:self.t1]), ora["sscale"], "server scales")
        carried = self.carry
        exempt = carried.copy()
        flips = 0
        for i in range(n):
            ks = flipped(h(gpu["wbits"][i, self.w0:self.w1]), ora["wbits"][i])
            if ks.size:
                s = ora["wscale"][i][seg_index(self.wl, ks)].astype(np.float64)
                cv = np.abs(ora["c"][i][ks].astype(np.float64))
                bad = ks[~((cv < NEAR_ZERO * s) | carried[ks])]
                assert bad.size == 0, (f"worker {i}: sign differs at {bad[:4] + lo} where "
                                       f"|c| >= {NEAR_ZERO} s")
                exempt[ks] = True
                flips += ks.size
            skip_i = np.union1d(np.nonzero(carried)[0], ks)
            close_except(h(gpu["delta"][i, lo:hi]), st["delta"][i], skip_i,
                         f"worker {i} error delta")
        ks = flipped(h(gpu["sbits"][self.w0:self.w1]), ora["sbits"])
        if ks.size:
            s = ora["sscale"][seg_index(self.sl, ks)].astype(np.float64)
            near = np.abs(ora["a"][ks].astype(np.float64)) < NEAR_ZERO * s
            bad = ks[~(near | exempt[ks])]
            assert bad.size == 0, (f"server sign differs at {bad[:4] + lo} where |a| >= "
                                   f"{NEAR_ZERO} s_bar and every worker sign agrees")
            exempt[ks] = True
        skip = np.nonzero(exempt)[0]
        close_except(h(gpu["eps"][lo:hi]), st["eps"], skip, "server error eps")
        close_except(h(gpu["m"][lo:hi]), st["m"], skip, "momentum m")
        close_except(h(gpu["x"][lo:hi]), st["x"], skip, "parameters x")
        self.carry = exempt
        say(f"  [{name}] [{lo}, {hi}) matches: {flips} worker and {ks.size} server signs "
            f"differ at near-zero values, {skip.size} coordinates exempt")
