"""Benchmark: one 1-bit Adam compression step on one MI355X.

A step is the whole hot path over one gradient set of the workload:
oba_compress (n workers) -> oba_server_reduce_recompress -> oba_decompress_update.
Default workload ``bert_large``: d = 336,000,000 binary32 parameters, n = 8
simulated workers, binary16 gradients 1e-3 * Student-t(3) with a fixed 1 % of
coordinates exactly zero, server error in n equal shards.  The state is
prepared by 10 warm-up steps (the library's Adam kernel) and the freeze;
the timed steps alternate two pre-generated gradient sets, all resident in
HBM.  Prints one JSON line (rank 0, one GPU).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
METRIC = "params updated/sec per 1-bit Adam step + achieved HBM GB/s vs peak"
CSRC = os.path.join(ROOT, "communication_compressed_optimizer_02_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gbytes(w, schedule="deferred"):
    """Algorithmic HBM bytes per parameter of each kernel of a step: every
    buffer a kernel must touch, once per direction."""
    n, gb = w.n, (2 if w.g_dtype == "f16" else 4)
    if schedule == "deferred":
        return {
            # last server bits read (the momentum), g_i and last c_i read;
            # c_i and packed bits written
            "compress_deferred": 1 / 8 + n * (gb + 4) + 4 * n + n / 8,
            # worker bits read, last a read, a written, server bits written
            "server_deferred": n / 8 + 8 + 1 / 8,
            # server bits read, denom read, x read+written (m stays implicit)
            "decompress_update": 1 / 8 + 12,
        }
    if schedule == "state16":
        return {
            # as the deferred pass, with each worker's c read and written as
            # 16-bit values
            "compress_deferred16": 1 / 8 + n * (gb + 2) + 2 * n + n / 8,
            "server_deferred": n / 8 + 8 + 1 / 8,
            "decompress_update": 1 / 8 + 12,
        }
    if schedule == "local":
        return {
            # g_i, m_i and the last c_i read; m_i, c_i and packed bits written
            "compress_deferred_local": n * (gb + 16) + n / 8,
            "server_deferred": n / 8 + 8 + 1 / 8,
            "decompress_update": 1 / 8 + 12,
        }
    reads = 4 + n * (gb + 4)  # m, g_i, delta_i
    return {
        # norm pass: m, g_i, delta_i read
        "compress_p1": reads,
        # apply pass: m, g_i, delta_i read again; delta_i and packed bits written
        "compress_p2": reads + 4 * n + n / 8,
        # worker bits read, eps read, a written over eps, server bits written
        "server_p1": n / 8 + 8 + 1 / 8,
        # a read, eps written
        "server_p2": 8,
        # server bits read, denom read, x read+written, m written
        "decompress_update": 1 / 8 + 16,
    }


def method_bytes(w):
    """Bytes per parameter if every buffer of the method is touched once per
    direction per step, the momentum being carried by the server message:
    g_i read, error read and written, worker bits written and read, server
    error read and written, server bits written and read, denom read, x read
    and written: n(|g| + 8.25) + 20.25."""
    gb = 2 if w.g_dtype == "f16" else 4
    return w.n * (gb + 8.25) + 20.25


def _code_only(text: str) -> str:
    """C++ source without comments and blank lines (a comment edit does not
    change a kernel)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def source_hash():
    """Hash of the code of the kernels and of the code that picks their
    launch grids (everything under csrc/), comments excluded."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload, kernel, field="hbm_bytes_per_launch"):
    """HBM bytes measured by rocprofv3 counters (per launch of the dominant
    kernel, or with field="step_hbm_bytes" per headline step), if the
    committed summary was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    val = re.search(field + r":\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != source_hash():
        return None
    return float(val.group(1))


def trace_from_profiles(workload):
    """The dominant kernel's average launch time (ms) in the committed
    rocprofv3 kernel trace, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    val = re.search(r"trace_avg_us:\s*([0-9.]+)", text)
    if not src or not val or src.group(1) != source_hash():
        return None
    return float(val.group(1)) / 1e3


def make_state(w, torch, oba, synth, warmup_timing=None):
    """The workload's state after its warm-up (Adam steps with the fused
    variance norm, as a run watching for the plateau makes them) and the
    freeze, plus two gradient sets.  warmup_timing (a dict) receives the
    warm-up kernels' mean time per step after the first (gradient generation
    excluded) and the last variance norm."""
    L = oba.Layout(w.d, w.n, w.wseg, w.sseg)
    S = oba.State(L, w.g_dtype)
    gen = synth.device_generator(w.seed)
    zero_idx = synth.device_zero_mask(gen, w.d) if w.name == "bert_large" else None
    S.x.normal_(0.0, 0.02, generator=gen)
    vnorm = torch.zeros(1, dtype=torch.float64, device="cuda")
    log(f"[bench] {w.name}: {w.warmup_steps} warm-up steps")
    for i in range(w.warmup_steps):
        synth.device_grads(gen, w, S.g, zero_idx)
        if i == 1:  # the first step (kernel loading) is not timed
            torch.cuda.synchronize()
            oba.timing_reset()
            oba.timing_enable(True, 64)
        S.warmup(synth.LR, synth.BETA1, synth.BETA2, synth.ETA, vnorm=vnorm)
    torch.cuda.synchronize()
    oba.timing_enable(False, 1)
    tot, cnt = oba.timing_read("adam_warmup")
    oba.timing_reset()
    if warmup_timing is not None and cnt:
        gb = 2 if w.g_dtype == "f16" else 4
        alg = w.n * gb + 24  # g_i read; m, v, x read and written
        warmup_timing.update({
            "avg_ms": round(tot / cnt, 4), "steps": cnt, "alg_bytes_per_param": alg,
            "alg_GBps": round(alg * w.d / (tot / cnt * 1e-3) / 1e9, 1),
            "variance_norm": float(vnorm.item()),
            "note": "Adam warm-up step with the fused variance norm (two kernels)"})
    S.freeze(synth.ETA)
    g_a = S.g
    synth.device_grads(gen, w, g_a, zero_idx)
    g_b = torch.empty_like(g_a)
    synth.device_grads(gen, w, g_b, zero_idx)
    del zero_idx
    torch.cuda.synchronize()
    return L, S, (g_a, g_b)


def host_info():
    """Cores in this process's affinity mask, the CPU model, available RAM."""
    aff = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = None
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    avail = int(line.split()[1]) * 1024
                    break
    except OSError:
        pass
    return aff, model, avail


def oracle_state(w, torch, synth, d, seed):
    """A compression-stage state and one gradient set of workload w at size
    d, drawn with the workload's device generators and copied to the host
    (drawing it with numpy would take longer than the oracle run)."""
    import numpy as np

    import oracle

    ws = synth.scaled(w, d) if w.name != "gpt2_xl" else None
    gen = synth.device_generator(seed)
    zero = synth.device_zero_mask(gen, d) if w.name == "bert_large" else None
    g = torch.empty((w.n, d), dtype=torch.float16 if w.g_dtype == "f16" else torch.float32,
                    device="cuda")
    synth.device_grads(gen, ws, g, zero)
    del zero

    def normal(shape, std):
        return torch.empty(shape, device="cuda").normal_(0.0, std, generator=gen).cpu().numpy()

    st = {"x": normal(d, 0.02), "m": normal(d, 1e-3), "delta": normal((w.n, d), 1e-4),
          "eps": normal(d, 1e-4)}
    v = normal(d, 1e-3) ** 2
    st["denom"] = oracle.freeze_variance(np.ascontiguousarray(v, dtype=np.float32), synth.ETA)
    del v
    g_h = g.cpu().numpy()
    del g
    torch.cuda.empty_cache()
    return ws, st, g_h


def oracle_step_threads(st, g, wseg, sseg, beta1, lr, threads):
    """One oracle step (compress, server, update) with its independent calls
    on `threads` threads: one compression per worker row; when the worker
    scale is one per worker and every server segment starts on a word, one
    server call per server segment; the update over word-aligned ranges.
    The oracle's code is unchanged: each call is the one the single-threaded
    step makes, on its own part of the arrays."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    n, d = g.shape
    with ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(lambda i: oracle.compress(g[i:i + 1], st["m"], st["delta"][i:i + 1],
                                                    wseg, beta1), range(n)))
        wb = np.concatenate([r[0] for r in res])
        ws = np.concatenate([r[1] for r in res])
        del res
        ns = len(sseg) - 1
        if len(wseg) == 2 and all(int(o) % 64 == 0 for o in sseg[:-1]) and threads > 1:
            def server(j):
                lo, hi = int(sseg[j]), int(sseg[j + 1])
                part = np.ascontiguousarray(wb[:, lo // 64:(hi + 63) // 64])
                loc = np.array([0, hi - lo], np.int64)
                return oracle.server_reduce_recompress(part, ws, loc, loc, st["eps"][lo:hi])

            parts = list(ex.map(server, range(ns)))
            sb = np.concatenate([p_[0] for p_ in parts])
            ss = np.concatenate([p_[1] for p_ in parts])
        else:
            sb, ss = oracle.server_reduce_recompress(wb, ws, wseg, sseg, st["eps"])
        cuts = sorted({min(d, (d * k // threads) // 64 * 64) for k in range(threads + 1)} | {d})
        list(ex.map(lambda k: oracle.decompress_update(sb, ss, sseg, st["denom"], st["m"],
                                                       st["x"], lr, cuts[k], cuts[k + 1]),
                    range(len(cuts) - 1)))
    return wb, ws, sb, ss


def cpu_baseline(w, torch, synth, d_cap, single_thread=True):
    """The oracle (plain C) timed on this host's cores: one compression step
    of the workload (compress, server, update) at its full d when host memory
    allows (else the largest d that fits, stated), its independent calls on
    up to 16 threads, median of 3 runs from the same state; then the same
    step at the bert_base shape on one thread, median of 3."""
    import numpy as np

    import oracle

    aff, model, avail = host_info()
    threads = max(1, min(aff, 16))
    gb = 2 if w.g_dtype == "f16" else 4
    per_coord = w.n * (gb + 8) + 24  # g, two copies of delta, m, x, eps, denom (host)
    d = min(w.d, d_cap)
    if avail is not None:
        d = min(d, int(0.5 * avail / per_coord) // 2048 * 2048)
    d = max(d, 1 << 20)
    log(f"[bench] CPU oracle: d={d:,} of {w.d:,}, {threads} threads of {aff}")
    ws, st0, g = oracle_state(w, torch, synth, d, w.seed + 1000)

    # the threaded split computes the single-threaded step exactly (small check)
    k = min(d, 1 << 20)
    small = synth.scaled(w, k)
    a = {nm: np.ascontiguousarray(v[..., :k]) for nm, v in st0.items()}
    b = {nm: v.copy() for nm, v in a.items()}
    gk = np.ascontiguousarray(g[:, :k])
    oracle.step(a, gk, small.wseg, small.sseg, synth.BETA1, synth.LR)
    oracle_step_threads(b, gk, small.wseg, small.sseg, synth.BETA1, synth.LR, threads)
    for nm in ("x", "m", "delta", "eps"):
        assert np.array_equal(a[nm].view(np.uint32), b[nm].view(np.uint32)), nm
    del a, b, gk

    runs = []
    for _ in range(3):
        st = {nm: v.copy() for nm, v in st0.items()}
        t0 = time.perf_counter()
        oracle_step_threads(st, g, ws.wseg, ws.sseg, synth.BETA1, synth.LR, threads)
        runs.append(time.perf_counter() - t0)
        del st
    del st0, g
    med = sorted(runs)[1]
    out = {"value": d / med, "unit": "params/s", "cores": threads, "kind": "oracle",
           "sample": f"one compression step (compress, server, update) of the {w.name} recipe "
                     f"at d={d:,} (the workload's d={w.d:,}"
                     + ("" if d == w.d else f"; params/s measured at d={d:,}") +
                     f"), n={w.n}, {w.g_dtype} gradients; independent oracle calls on "
                     f"{threads} threads; median of 3 runs",
           "threads": threads, "affinity_cores": aff, "cpu_model": model,
           "runs_s": [round(r, 3) for r in runs], "median_s": round(med, 3), "d": d}
    if single_thread:
        wb = synth.workload("bert_base")
        d1 = wb.d if avail is None else min(wb.d, int(0.5 * avail / (wb.n * 12 + 24)))
        log(f"[bench] CPU oracle, one thread: bert_base d={d1:,}")
        ws1, st0, g = oracle_state(wb, torch, synth, d1, wb.seed + 1000)
        runs = []
        for _ in range(3):
            st = {nm: v.copy() for nm, v in st0.items()}
            t0 = time.perf_counter()
            oracle.step(st, g, ws1.wseg, ws1.sseg, synth.BETA1, synth.LR)
            runs.append(time.perf_counter() - t0)
            del st
        med1 = sorted(runs)[1]
        out["single_thread"] = {"workload": wb.name, "d": d1, "n": wb.n, "grad_dtype": wb.g_dtype,
                                "runs_s": [round(r, 3) for r in runs], "median_s": round(med1, 3),
                                "value": d1 / med1, "unit": "params/s", "threads": 1}
        # the same bert_base step on the threads of the main run
        runs = []
        for _ in range(3):
            st = {nm: v.copy() for nm, v in st0.items()}
            t0 = time.perf_counter()
            oracle_step_threads(st, g, ws1.wseg, ws1.sseg, synth.BETA1, synth.LR, threads)
            runs.append(time.perf_counter() - t0)
            del st
        medt = sorted(runs)[1]
        out["bert_base_threads"] = {"workload": wb.name, "d": d1, "threads": threads,
                                    "runs_s": [round(r, 3) for r in runs],
                                    "median_s": round(medt, 3), "value": d1 / medt,
                                    "unit": "params/s"}
        del st0, g
    return out


def run_graph(S, gsets, args, torch, synth):
    """The deferred step captured once per gradient set in a HIP graph
    (torch's graph API) and replayed alternately: the same kernels without
    per-launch host work.  Call after eager deferred steps (implicit m)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(side):
        for g in gsets:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=side):
                S.step_deferred(synth.BETA1, synth.LR, g=g)
            graphs.append(gr)
    torch.cuda.current_stream().wait_stream(side)
    for i in range(max(1, args.warmup)):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    del graphs
    return round(ms, 4)


def run_small(w, S, gsets, args, torch, oba, synth):
    """The deferred step as one launch of one block (oba_step_small), for
    layouts within its limits: W untimed and K timed eager steps from the
    freeze state, then the same step replayed from HIP graphs."""
    L = S.L
    if L.d > 65536 or L.n > 64 or L.n_wseg > 64 or L.n_sseg > 64:
        return None
    S.start_compression()
    log(f"[bench] one-block step: {args.warmup} untimed steps, {args.steps} timed steps")
    S.step_small(synth.BETA1, synth.LR, g=gsets[1])  # the step that reads the warm-up m
    for i in range(args.warmup):
        S.step_small(synth.BETA1, synth.LR, g=gsets[i % 2])
    torch.cuda.synchronize()
    oba.timing_reset()
    oba.timing_enable(True, 16 * max(1, args.steps))
    t0 = time.perf_counter()
    for i in range(args.steps):
        S.step_small(synth.BETA1, synth.LR, g=gsets[i % 2])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    oba.timing_enable(False, 1)
    tot, cnt = oba.timing_read("step_small")
    oba.timing_reset()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(side):
        for g in gsets:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=side):
                S.step_small(synth.BETA1, synth.LR, g=g)
            graphs.append(gr)
    torch.cuda.current_stream().wait_stream(side)
    for i in range(max(1, args.warmup)):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    del graphs
    return {"ms_per_step": round(ms, 4), "value": w.d / (ms * 1e-3),
            "kernel_avg_ms": round(tot / cnt, 4) if cnt else None,
            "graph_replay_ms_per_step": round(graph_ms, 4),
            "graph_replay_value": w.d / (graph_ms * 1e-3)}


def run_listed(w, S, g_flat, args, torch, oba, synth):
    """The deferred step with x and every worker's gradient held as the
    model's separate tensors (copies of the flat buffers), everything else
    flat: W untimed and K timed steps from the freeze state."""
    lengths = [int(k) for k in synth.gpt2_xl_tensor_sizes()]
    L = S.L

    def split(flat):
        out, at = [], 0
        for k in lengths:
            out.append(flat[at:at + k].clone())
            at += k
        return out

    S.start_compression()
    TL = oba.TensorList(L, split(S.x), [split(g_flat[i, :w.d]) for i in range(w.n)])
    log(f"[bench] tensor list ({len(lengths)} tensors): {args.warmup} untimed steps, "
        f"{args.steps} timed steps")
    state = {"implicit": False}

    def step():
        if state["implicit"]:
            oba.compress_deferred_listed(L, TL, None, S.delta, S.wbits, S.wscale, synth.BETA1,
                                         S.sbits, S.sscale)
        else:
            oba.compress_deferred_listed(L, TL, S.m, S.delta, S.wbits, S.wscale, synth.BETA1)
        oba.server_reduce_recompress_deferred(L, S.wbits, S.wscale, S.eps, S.sbits, S.sscale)
        oba.decompress_update_listed(L, TL, S.sbits, S.sscale, S.denom, None, synth.LR)
        state["implicit"] = True

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    oba.timing_reset()
    oba.timing_enable(True, 16 * max(1, args.steps))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    oba.timing_enable(False, 1)
    alg = gbytes(w, "deferred")
    kernels = {}
    for k in list(alg) + ["finalize_scales"]:
        tot, cnt = oba.timing_read(k)
        ent = {"avg_ms": round(tot / cnt, 4) if cnt else 0.0, "launches": cnt}
        if k in alg and cnt:
            ent["alg_GBps"] = round(alg[k] * w.d / (tot / cnt * 1e-3) / 1e9, 1)
        kernels[k] = ent
    oba.timing_reset()
    # the listed warm-up step with the variance norm, on the same tensors
    # (after the deferred steps: it rewrites x, m and v, which they no longer need)
    vnorm = torch.zeros(1, dtype=torch.float64, device="cuda")

    def warm():
        oba.adam_warmup_step_listed(L, TL, S.m, S.v, synth.LR, synth.BETA1, synth.BETA2,
                                    synth.ETA, vnorm=vnorm)

    for _ in range(max(1, args.warmup)):
        warm()
    torch.cuda.synchronize()
    oba.timing_enable(True, 4 * max(1, args.steps))
    for _ in range(args.steps):
        warm()
    torch.cuda.synchronize()
    oba.timing_enable(False, 1)
    tot, cnt = oba.timing_read("adam_warmup")
    oba.timing_reset()
    gb = 2 if w.g_dtype == "f16" else 4
    walg = w.n * gb + 24
    warm_ent = {"avg_ms": round(tot / cnt, 4) if cnt else None, "steps": cnt,
                "alg_bytes_per_param": walg,
                "alg_GBps": round(walg * w.d / (tot / cnt * 1e-3) / 1e9, 1) if cnt else None}
    TL.close()
    del TL
    S.m_implicit = False  # the listed run left S.m stale and sbits/sscale its own
    torch.cuda.empty_cache()
    return {"tensors": len(lengths), "ms_per_step": round(ms, 4), "value": w.d / (ms * 1e-3),
            "step_alg_GBps": round(sum(alg.values()) * w.d / (ms * 1e-3) / 1e9, 1),
            "kernels": kernels, "warmup_step": warm_ent}


def one_gpu_share(w, torch, oba, synth, steps, warmup):
    """The kernels one GPU of an n-GPU job would run per step, at their real
    shapes: its own worker's compression over all d coordinates, the server
    pass over its shard of d/n coordinates (reading the n workers' messages
    for that shard), and the update over d.  The exchanges between GPUs are
    not modelled.  The inputs are the workload's gradient recipe; the shard's
    worker messages are those of n compressions of the same recipe."""
    d, n = w.d, w.n
    ds = d // n
    L1 = oba.Layout(d, 1, synth.whole(d), synth.whole(d))
    Ls = oba.Layout(ds, n, synth.whole(ds), synth.whole(ds))
    S1 = oba.State(L1, w.g_dtype)
    Ss = oba.State(Ls, w.g_dtype)
    gen = synth.device_generator(w.seed + 2000)
    wl1 = synth.Workload(w.name, d, 1, w.g_dtype, w.seed, 0, L1.wseg, L1.sseg, w.grad_std)
    wls = synth.Workload(w.name, ds, n, w.g_dtype, w.seed, 0, Ls.wseg, Ls.sseg, w.grad_std)
    synth.device_grads(gen, wl1, S1.g)
    synth.device_grads(gen, wls, Ss.g)
    S1.x.normal_(0.0, 0.02, generator=gen)
    S1.denom.uniform_(1e-3, 2e-3, generator=gen)
    S1.m.normal_(0.0, 1e-3, generator=gen)
    Ss.denom.fill_(1.0)
    # the shard's n worker messages (and scales) come from n real compressions
    Ss.step_deferred(synth.BETA1, synth.LR)
    S1.step_deferred(synth.BETA1, synth.LR)

    def step():
        oba.compress_deferred(L1, S1.g, None, S1.delta, S1.wbits, S1.wscale, synth.BETA1,
                              S1.sbits, S1.sscale)
        oba.server_reduce_recompress_deferred(Ls, Ss.wbits, Ss.wscale, Ss.eps, Ss.sbits,
                                              Ss.sscale)
        oba.decompress_update(L1, S1.sbits, S1.sscale, S1.denom, None, S1.x, synth.LR)

    for _ in range(max(1, warmup)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gb = 2 if w.g_dtype == "f16" else 4
    alg = d * (1 / 8 + (gb + 4) + 4 + 1 / 8) + ds * (n / 8 + 8 + 1 / 8) + d * (1 / 8 + 12)
    del S1, Ss
    L1.close()
    Ls.close()
    return {"ms_per_step": round(ms, 4), "params_per_s": d / (ms * 1e-3),
            "alg_bytes": alg, "alg_GBps": round(alg / (ms * 1e-3) / 1e9, 1),
            "shape": f"1 worker over d={d:,}, 1 server shard of {ds:,} coordinates with "
                     f"{n} workers' messages, update over d"}


# Streaming probes of libhbmstream.so (calib/hbm_stream.hip): name -> (shape,
# groups).  The worker-pass shapes take the workload's n workers in groups of
# 4, as the deferred worker pass does; the others are fixed row counts.
# name -> (shape, groups); groups None: the workload's n workers in groups of
# PROBE_PER[name] (the probe is skipped when that does not divide n)
PROBES = {"read": (0, 1), "write": (1, 1), "copy": (2, 1), "worker_g16": (3, None),
          "worker_g32": (4, None), "state16": (5, None), "warmup_g16": (6, 1),
          "update": (7, 1), "in_place": (8, 1), "worker_g16_x1": (9, None),
          "worker_g16_x2": (10, None), "worker_g16_x8": (11, None), "state16_x1": (12, None),
          "worker_g32_x1": (13, None)}
PROBE_PER = {"worker_g16_x1": 1, "worker_g16_x2": 2, "worker_g16_x8": 8, "state16_x1": 1,
             "worker_g32_x1": 1}
# the probe of the same access shape as each kernel of the headline step
PROBE_OF = {("compress_deferred", "f16"): "worker_g16_x1",
            ("compress_deferred", "f32"): "worker_g32_x1",
            ("compress_deferred16", "f16"): "state16_x1", ("decompress_update", None): "update",
            ("server_deferred", None): "in_place", ("adam_warmup", "f16"): "warmup_g16"}


def probe_lib():
    import ctypes

    path = os.path.join(ROOT, "communication_compressed_optimizer_02_amd", "libhbmstream.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build first (__graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I, I32, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64
    lib.hbm_stream_shape.restype = I
    lib.hbm_stream_shape.argtypes = [I, ctypes.POINTER(I32)]
    lib.hbm_stream_launch.restype = I
    lib.hbm_stream_launch.argtypes = [I, I, P, P, I64, I64, I32, I32, P, P]
    return lib


PROBE_BPC = (0, 2, 3, 4, 5, 6)  # resident blocks per CU tried (0: as registers allow)


def hbm_ceiling(torch, w, reps=5):
    """What this HBM delivers for each access shape of the method's kernels,
    measured here with the streaming probes (no arithmetic) at the
    workload's size, on random data (constant data streams faster on this
    part): bytes moved per launch / mean launch time (HIP events on the
    launch stream), the best over the global and buffer-resource forms and
    over occupancy caps of PROBE_BPC blocks per CU."""
    import ctypes

    lib = probe_lib()
    spans = w.d // 2048
    ld = spans * 2048
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 3000)
    out = {}
    for name, (shape, groups) in PROBES.items():
        if groups is None:
            per = PROBE_PER.get(name, 4)
            if w.n % per:
                continue
            groups = w.n // per
        na, ab, nb, bb, bmode = _probe_shapes()[name]
        a = torch.empty(max(1, groups * na * ld * ab // 4), device="cuda")
        b = torch.empty(max(1, groups * nb * ld * bb // 4), device="cuda")
        a.uniform_(0.5, 1.0, generator=gen)
        b.uniform_(0.5, 1.0, generator=gen)
        nbytes = groups * ld * (na * ab + nb * bb * (2 if bmode == 2 else 1))
        res = {"bytes_per_launch": nbytes, "GBps": 0.0}
        forms = (0, 1, 2, 3) if (bmode == 2 and na == nb) else (0, 1)
        for buf in forms:
            for bpc in PROBE_BPC:
                def go():
                    return lib.hbm_stream_launch(shape, buf, ctypes.c_void_p(a.data_ptr()),
                                                 ctypes.c_void_p(b.data_ptr()), ld, spans,
                                                 groups, bpc, ctypes.c_void_p(sink.data_ptr()),
                                                 ctypes.c_void_p(stream.cuda_stream))
                if go() != 0:  # an occupancy cap this device cannot express
                    continue
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    go()
                e1.record()
                torch.cuda.synchronize()
                gbs = round(nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)
                form = ("buffer" if buf & 1 else "global") + (", rows alternating" if buf & 2 else "")
                res[f"{form}, bpc{bpc}"] = gbs
                if gbs > res["GBps"]:
                    res["GBps"] = gbs
                    res["best"] = f"{form}, " + (
                        f"{bpc} blocks per CU" if bpc else "occupancy as registers allow")
        out[name] = res
        del a, b
        torch.cuda.empty_cache()
    return {"probes": out, "rows": ld,
            "note": "streaming probes (calib/hbm_stream.hip) in the kernels' lane layout, "
                    "non-temporal, all loads of a block before its stores, random data; GBps = "
                    "the best over load forms, load orders and occupancy caps"}


# ---- profile summaries (profiles/*.md) from raw rocprofv3 output -----------
# The profiled commands, run from the repository root on the GPU machine (each
# counter pass on its own run, as rocprofv3 collects one pass per run).
PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats -d profiles_raw/trace -o run -f csv -- "
             "python3 -u bench.py --steps 5 --warmup 1 --no-cpu-baseline",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex oba:: -d profiles_raw/fetch "
             "-o run -f csv -- python3 -u bench.py --steps 2 --warmup 0 --no-cpu-baseline",
    "write": "rocprofv3 --pmc WRITE_SIZE --kernel-include-regex oba:: -d profiles_raw/write "
             "-o run -f csv -- python3 -u bench.py --steps 2 --warmup 0 --no-cpu-baseline",
    "occ": "rocprofv3 --pmc OccupancyPercent MeanOccupancyPerCU SQ_WAVES --kernel-include-regex "
           "oba:: -d profiles_raw/occ -o run -f csv -- python3 -u bench.py --steps 2 "
           "--warmup 0 --no-cpu-baseline",
}
CU_NUM = 256


def _short(name):
    name = re.sub(r"^void ", "", name)
    name = name.replace("oba::(anonymous namespace)::", "oba::")
    return name.split("(", 1)[0].strip()


_SHAPES = {}


def _probe_shapes():
    """Probe name -> (rows of A, bytes, rows of B, bytes, B mode) per group."""
    if not _SHAPES:
        import ctypes

        lib = probe_lib()
        info = (ctypes.c_int32 * 5)()
        for nm, (shape, _) in PROBES.items():
            assert lib.hbm_stream_shape(shape, info) == 0
            _SHAPES[nm] = tuple(info)
    return _SHAPES


def _role(short, n=None):
    """What a kernel of the bench run is, from its template arguments; with
    the workload's worker count n, a worker or server pass whose group size
    does not fit n (the one-GPU share's single worker) is "other"."""
    m = re.match(r"oba::k_compress(16)?<[^,]+, [^,]+, (\d+), (\d), (true|false)>", short)
    if m:
        mode = int(m.group(3))
        base = {1: "compress_p1", 2: "compress_p2", 3: "compress_deferred (first step, m read)",
                4: "compress_deferred", 5: "compress_deferred_local"}[mode]
        if m.group(1):
            base = base.replace("compress_deferred", "compress_deferred16")
        if not n:
            group = None
        elif m.group(1):  # the 16-bit pass: one worker per block, m-read step groups of 4
            group = 1 if mode == 4 else min(n, 4)
        else:
            group = 1 if mode in (4, 5) else min(n, 8)
        if n and int(m.group(2)) != group:
            return "other (one-GPU share)"
        return base
    m = re.match(r"oba::k_server_p1<(\d+), (true|false)>", short)
    if m:
        if n and int(m.group(1)) != min(n, 8):
            return "other (one-GPU share)"
        return "server_deferred" if m.group(2) == "true" else "server_p1"
    m = re.match(r"oba::k_decompress_update<(true|false), (true|false), (true|false)>", short)
    if m:
        return {("false", "true"): "decompress_update", ("true", "true"):
                "decompress_update (m written)", ("true", "false"): "server_momentum"}.get(
                    (m.group(1), m.group(2)), "")
    m = re.match(r"oba::k_stream<(\d+), [^,]+, [^,]+, \d+, \d+, \d, (true|false), "
                 r"(true|false)>", short)
    if m:  # the first template argument is the probe's shape index
        form = ("buffer" if m.group(2) == "true" else "global") + (
            ", rows alternating" if m.group(3) == "true" else "")
        for nm, (shape, _) in PROBES.items():
            if shape == int(m.group(1)):
                return f"probe {nm} ({form})"
        return "probe"
    for pat, r in (("oba::k_residual", "server_p2"), ("oba::k_adam_warmup", "adam_warmup"),
                   ("oba::k_freeze", "freeze"), ("oba::k_norm_finalize", "variance norm sum"),
                   ("oba::k_finalize_scales", "scale sums"), ("oba::k_sum_items", "scale sums")):
        if short.startswith(pat):
            return r
    return ""


def _alg_bytes(w):
    """Algorithmic bytes per launch of each role at the workload's shape."""
    gb = 2 if w.g_dtype == "f16" else 4
    n, d = w.n, w.d
    per = {}
    for sch in ("deferred", "explicit", "local", "state16"):
        per.update(gbytes(w, sch))
    per["compress_deferred (first step, m read)"] = 4 + n * (gb + 4) + 4 * n + n / 8
    per["compress_deferred16 (first step, m read)"] = 4 + n * (gb + 2) + 2 * n + n / 8
    per["decompress_update (m written)"] = 1 / 8 + 16
    per["server_momentum"] = 1 / 8 + 4
    per["adam_warmup"] = n * gb + 24
    per["freeze"] = 8
    out = {k: v * d for k, v in per.items()}
    ld = (d // 2048) * 2048
    for nm, (shape, groups) in PROBES.items():
        na, ab, nb, bb, mode = _probe_shapes()[nm]
        g = groups if groups is not None else n // PROBE_PER.get(nm, 4)
        for form in ("global", "buffer", "global, rows alternating", "buffer, rows alternating"):
            out[f"probe {nm} ({form})"] = g * ld * (na * ab + nb * bb * (2 if mode == 2 else 1))
    return out


def _per_dispatch(path, counter, n=None):
    """(role, short name, grid) -> list of the counter's values per dispatch."""
    import collections
    import csv

    acc = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or "oba::" not in r["Kernel_Name"]:
                continue
            sh = _short(r["Kernel_Name"])
            acc[(_role(sh, n), sh, int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return acc


def _largest_grids(keys):
    """The grid of each short name's largest launches (the workload's own
    shape; smaller grids of the same kernel are other launches)."""
    big = {}
    for _, sh, g in keys:
        big[sh] = max(big.get(sh, 0), g)
    return big


def summarize_profiles(raw, out_dir, workload="bert_large"):
    """Write the profile summaries from rocprofv3's raw CSVs under `raw`
    (trace/, fetch/, write/, occ/) and the two bench JSON lines there
    (bench.json: the unprofiled default run; trace_bench.json: the traced
    run)."""
    import csv
    import glob

    from communication_compressed_optimizer_02_amd import synth

    w = synth.workload(workload)
    alg = _alg_bytes(w)
    one = lambda pat: sorted(glob.glob(os.path.join(raw, pat)))[0]  # noqa: E731
    src = source_hash()
    written = []

    def jline(name):
        with open(os.path.join(raw, name)) as f:
            return json.loads([x for x in f if x.startswith("{")][-1])

    # ---- traffic: FETCH_SIZE and WRITE_SIZE, calibrated on the copy probe
    fetch = _per_dispatch(one("fetch/*counter_collection.csv"), "FETCH_SIZE", w.n)
    write = _per_dispatch(one("write/*counter_collection.csv"), "WRITE_SIZE", w.n)
    cal = "probe copy (global)"
    cf = [v for k, vs in fetch.items() if k[0] == cal for v in vs]
    cw = [v for k, vs in write.items() if k[0] == cal for v in vs]
    half = alg[cal] / 2  # the copy reads and writes the same bytes
    ff = half / (sum(cf) / len(cf) * 1024)
    fw = half / (sum(cw) / len(cw) * 1024)
    big = _largest_grids(fetch)
    rows, dom, step = [], None, 0.0
    for key in sorted(fetch, key=lambda k: (k[0] or "~", k[1], k[2])):
        role, sh, grid = key
        fv = sum(fetch[key]) / len(fetch[key]) * 1024 * ff
        wl = write.get(key, [0.0])
        wv = sum(wl) / len(wl) * 1024 * fw
        main = grid == big[sh]
        a = alg.get(role) if main else None
        rows.append((sh, grid, role if main else f"{role}, other shape", fv, wv, a))
        if main and role == "compress_deferred":
            dom = fv + wv
        if main and role in ("compress_deferred", "server_deferred", "decompress_update"):
            step += fv + wv
    L = [f"# HBM traffic per launch (rocprofv3 counters), {w.name} workload", "",
         f"Workload: d = {w.d:,}, n = {w.n}, {w.g_dtype} gradients; one MI355X.", "",
         "Commands (repository root, GPU box; one counter per run):", "",
         "    " + PROFILE_CMDS["fetch"], "    " + PROFILE_CMDS["write"], "",
         "Summary written by `python bench.py --summarize-profiles profiles_raw` from those",
         "runs' counter_collection.csv files.", "",
         "Calibration: the copy probe (`k_stream<2, float, float, 4, 4, 1, false, false>`, global form) reads",
         f"and writes {half / 1e9:.3f} GB per launch; it reads FETCH_SIZE = "
         f"{sum(cf) / len(cf) * 1024 / 1e9:.3f} GB and WRITE_SIZE =",
         f"{sum(cw) / len(cw) * 1024 / 1e9:.3f} GB, so FETCH_SIZE is scaled by {ff:.3f} and "
         f"WRITE_SIZE by {fw:.3f}.", "",
         "| kernel | grid (threads) | role | read GB | write GB | traffic GB | algorithmic GB | "
         "traffic / algorithmic |", "|---|---|---|---|---|---|---|---|"]
    for sh, grid, role, fv, wv, a in rows:
        r = f"{(fv + wv) / a:.4f}" if a else "—"
        ag = f"{a / 1e9:.3f}" if a else "—"
        L.append(f"| `{sh}` | {grid} | {role or '—'} | {fv / 1e9:.3f} | {wv / 1e9:.3f} | "
                 f"{(fv + wv) / 1e9:.3f} | {ag} | {r} |")
    L += ["", "Algorithmic bytes: every buffer a kernel must touch, once per direction "
          "(bench.py `gbytes`); a probe's are the rows it streams.  A ratio near 1 means no "
          "re-reads or partial-line waste.", "",
          "Dominant kernel (compress_deferred):", f"hbm_bytes_per_launch: {dom:.0f}",
          "Headline step (three streaming kernels):", f"step_hbm_bytes: {step:.0f}",
          f"kernel_source_sha256: {src}"]
    path = os.path.join(out_dir, f"compress_deferred_{w.name}_pmc.md")
    with open(path, "w") as f:
        f.write("\n".join(L) + "\n")
    written.append(path)

    # ---- occupancy
    occ_files = glob.glob(os.path.join(raw, "occ/*counter_collection.csv"))
    if occ_files:
        occ = {c: _per_dispatch(occ_files[0], c, w.n)
               for c in ("OccupancyPercent", "MeanOccupancyPerCU", "SQ_WAVES")}
        keys = set().union(*[set(v) for v in occ.values()])
        big = _largest_grids(keys)
        L = [f"# Occupancy per kernel (rocprofv3 counters), {w.name} workload", "",
             "Command (repository root, GPU box):", "", "    " + PROFILE_CMDS["occ"], "",
             "Summary written by `python bench.py --summarize-profiles profiles_raw`.",
             "OccupancyPercent = 400 * SQ_WAVE_CYCLES / GRBM_GUI_ACTIVE / CU_NUM / 32 (rocprofv3's",
             "derived counter for gfx950): resident waves as a share of 32 per CU (8 per SIMD);",
             "waves per SIMD below = OccupancyPercent * 8 / 100, the mean over the dispatch,",
             "including its ramp-up and drain.  MeanOccupancyPerCU: the same from SQ_LEVEL_WAVES.",
             "", "| kernel | grid | role | waves per SIMD | OccupancyPercent | MeanOccupancyPerCU "
             "| waves launched |", "|---|---|---|---|---|---|---|"]
        for key in sorted(keys, key=lambda k: (k[0] or "~", k[1], k[2])):
            role, sh, grid = key
            if grid != big[sh]:
                continue
            val = {c: (sum(occ[c][key]) / len(occ[c][key]) if occ[c].get(key) else None)
                   for c in occ}
            op = val["OccupancyPercent"]
            L.append(f"| `{sh}` | {grid} | {role or '—'} | "
                     f"{op * 8 / 100:.2f} | {op:.1f} | " if op is not None else
                     f"| `{sh}` | {grid} | {role or '—'} | — | — | ")
            L[-1] += (f"{val['MeanOccupancyPerCU']:.2f} | " if val["MeanOccupancyPerCU"]
                      is not None else "— | ")
            L[-1] += f"{val['SQ_WAVES']:.0f} |" if val["SQ_WAVES"] is not None else "— |"
        L += ["", f"kernel_source_sha256: {src}"]
        path = os.path.join(out_dir, f"occupancy_{w.name}.md")
        with open(path, "w") as f:
            f.write("\n".join(L) + "\n")
        written.append(path)

    # ---- kernel trace
    stats = []
    with open(one("trace/*kernel_stats.csv")) as f:
        stats = [r for r in csv.DictReader(f) if "oba::" in r["Name"]]
    shapes = {}
    with open(one("trace/*kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            if "oba::" not in r["Kernel_Name"]:
                continue
            sh = _short(r["Kernel_Name"])
            key = (sh, int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]))
            ent = shapes.setdefault(key, {"t": [], "vgpr": r["VGPR_Count"],
                                          "agpr": r["Accum_VGPR_Count"], "sgpr": r["SGPR_Count"],
                                          "lds": r["LDS_Block_Size"],
                                          "scratch": r["Scratch_Size"]})
            ent["t"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    jp, jb = jline("trace_bench.json"), jline("bench.json")
    big = {}
    for sh, g in shapes:
        big[sh] = max(big.get(sh, 0), g)
    T = [f"# Kernel trace: the 1-bit Adam compression step, {w.name} workload", "",
         f"Workload: d = {w.d:,} binary32 parameters, n = {w.n} simulated workers, {w.g_dtype} "
         "gradients, 1 worker segment, n server segments; one MI355X (gfx950).", "",
         "Command (repository root, GPU box):", "", "    " + PROFILE_CMDS["trace"], "",
         "Summary written by `python bench.py --summarize-profiles profiles_raw`.", "",
         "Covers the warm-up and freeze, 1 untimed and 5 timed steps of each schedule "
         "(deferred, explicit, per-worker momentum, 16-bit state), the graph replays, the "
         "one-GPU-share run and the HBM streaming probes.  bench.py's own HIP-event timing of the "
         "dominant kernel (`compress_deferred`): "
         f"{jp['kernels']['compress_deferred']['avg_ms'] * 1e3:.1f} µs in this traced run, "
         f"{jb['kernels']['compress_deferred']['avg_ms'] * 1e3:.1f} µs in the unprofiled "
         "default run on the same box (`python bench.py`).", "",
         "The VGPR column is rocprofv3's: it counts the kernel descriptor's register granules "
         "in units of 4, while gfx950 allocates wave64 VGPRs in granules of 8, so the allocated "
         "count is twice its value rounded up to 8 (84 -> 168).  The compiler's own counts and "
         "occupancy are in kernel_resources_gfx950.md.", "",
         "| kernel | grid (threads) | role | launches | avg µs | min µs | max µs | VGPR (rocprof) "
         "| SGPR | LDS B | scratch B |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    for (sh, g), ent in sorted(shapes.items(), key=lambda kv: -sum(kv[1]["t"])):
        t = ent["t"]
        role = _role(sh, w.n) if g == big[sh] else f"{_role(sh, w.n)}, other shape"
        T.append(f"| `{sh}` | {g} | {role or '—'} | {len(t)} | {sum(t) / len(t):.1f} | "
                 f"{min(t):.1f} | {max(t):.1f} | {ent['vgpr']} | {ent['sgpr']} | {ent['lds']} | "
                 f"{ent['scratch']} |")
    T += ["", "Per kernel name (rocprofv3 --stats):", "",
          "| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        T.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                 f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    dom_t = [v for (sh, g), e in shapes.items() if g == big[sh]
             and _role(sh, w.n) == "compress_deferred" for v in e["t"]]
    T += ["", "Dominant kernel (compress_deferred), trace average per launch:",
          f"trace_avg_us: {sum(dom_t) / len(dom_t):.1f}", f"kernel_source_sha256: {src}"]
    path = os.path.join(out_dir, f"kernel_trace_{w.name}.md")
    with open(path, "w") as f:
        f.write("\n".join(T) + "\n")
    written.append(path)
    return written


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bert_large",
                    choices=["tiny", "bert_base", "bert_large", "gpt2_xl", "quadratic"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tensor-list", action="store_true",
                    help="also time the deferred step with x and the gradients as the model's "
                         "separate tensors (gpt2_xl: its 388 tensors)")
    ap.add_argument("--cpu-sample", type=int, default=336_000_000,
                    help="largest d of the CPU oracle's timed step")
    ap.add_argument("--no-single-thread", action="store_true",
                    help="skip the one-thread oracle run at the bert_base shape")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/*.md from the raw rocprofv3 output under DIR and exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        for p_ in summarize_profiles(args.summarize_profiles, os.path.join(ROOT, "profiles"),
                                     args.workload):
            print(p_)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the n data-parallel workers are simulated as n "
              "buffers on that GPU; a run over several GPUs is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from communication_compressed_optimizer_02_amd import binding as oba
    from communication_compressed_optimizer_02_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = synth.workload(args.workload)
    warm = {}
    L, S, gsets = make_state(w, torch, oba, synth, warm)

    def run(schedule):
        """W untimed + K timed steps of one schedule from the freeze state.
        The deferred schedule's first step, which reads the warm-up's m
        instead of the server message, is never timed."""
        S.start_compression()
        if schedule == "local":
            S.start_local_momentum()
        if schedule == "state16":
            S.start_state16("bf16")
        fn = {"deferred": S.step_deferred, "explicit": S.step, "local": S.step_local,
              "state16": S.step_deferred16}[schedule]
        log(f"[bench] {schedule}: {args.warmup} untimed steps, {args.steps} timed steps")
        if schedule in ("deferred", "state16") and args.warmup == 0:
            fn(synth.BETA1, synth.LR, g=gsets[1])
        for i in range(args.warmup):
            fn(synth.BETA1, synth.LR, g=gsets[i % 2])
        torch.cuda.synchronize()
        oba.timing_reset()
        oba.timing_enable(True, capacity=16 * max(1, args.steps))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(synth.BETA1, synth.LR, g=gsets[i % 2])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        oba.timing_enable(False, 1)
        alg = gbytes(w, schedule)
        kernels = {}
        for k in list(alg) + ["finalize_scales"]:
            tot, cnt = oba.timing_read(k)
            ent = {"avg_ms": round(tot / cnt, 4) if cnt else 0.0, "launches": cnt}
            if k in alg and cnt:
                ent["alg_bytes_per_param"] = alg[k]
                ent["alg_GBps"] = round(alg[k] * w.d / (tot / cnt * 1e-3) / 1e9, 1)
            kernels[k] = ent
        oba.timing_reset()
        return (t1 - t0) * 1e3 / args.steps, alg, kernels

    ms, alg, kernels = run("deferred")
    log("[bench] deferred step replayed from HIP graphs")
    graph_ms = run_graph(S, gsets, args, torch, synth)
    small = run_small(w, S, gsets, args, torch, oba, synth)
    listed = None
    if args.tensor_list:
        if w.name != "gpt2_xl":
            raise SystemExit("--tensor-list needs the tensor-list workload (gpt2_xl)")
        listed = run_listed(w, S, gsets[0], args, torch, oba, synth)
    ms_x, alg_x, kernels_x = run("explicit")
    ms_l, alg_l, kernels_l = run("local")
    del S.m_local
    ms_h, alg_h, kernels_h = run("state16")  # last: it frees the binary32 rows
    # dominant kernel: the largest share of the step's time
    dom = max(alg, key=lambda k: kernels[k]["avg_ms"])
    dom_ms = kernels[dom]["avg_ms"]
    dom_bytes = alg[dom] * w.d
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(w.name, dom)
    step_alg = sum(alg.values()) * w.d
    step_hbm = traffic_from_profiles(w.name, dom, "step_hbm_bytes")  # counters, per step
    out = {
        "metric": METRIC,
        "value": w.d / (ms * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "d": w.d, "n_workers": w.n, "grad_dtype": w.g_dtype,
                   "worker_segments": len(w.wseg) - 1, "server_segments": len(w.sseg) - 1,
                   "parallelism": "dp%d simulated on one GPU" % w.n,
                   "schedule": "deferred-residual state (c, a kept; residuals formed on use; "
                               "momentum rebuilt from the server message)"},
        "step_alg_GBps": round(step_alg / (ms * 1e-3) / 1e9, 1),
        "step_hbm_GBps": (round(step_hbm / (ms * 1e-3) / 1e9, 1) if step_hbm else None),
        "step_alg_bytes_per_param": round(sum(alg.values()), 3),
        "method_bytes_per_param": round(method_bytes(w), 3),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": dom_bytes,
                     "avg_launch_ms": round(dom_ms, 4), "timing": "HIP events on the launch "
                     "stream around each launch of the timed steps",
                     "profile_trace_avg_ms": trace_from_profiles(w.name)},
        "kernels": kernels,
        "graph_replay": {"ms_per_step": graph_ms, "value": w.d / (graph_ms * 1e-3),
                         "note": "the headline step captured in HIP graphs and replayed"},
        "warmup_step": warm,
        "explicit_schedule": {
            "ms_per_step": round(ms_x, 4), "value": w.d / (ms_x * 1e-3),
            "step_alg_bytes_per_param": round(sum(alg_x.values()), 3),
            "step_alg_GBps": round(sum(alg_x.values()) * w.d / (ms_x * 1e-3) / 1e9, 1),
            "kernels": kernels_x},
        "local_momentum_schedule": {
            "ms_per_step": round(ms_l, 4), "value": w.d / (ms_l * 1e-3),
            "step_alg_bytes_per_param": round(sum(alg_l.values()), 3),
            "step_alg_GBps": round(sum(alg_l.values()) * w.d / (ms_l * 1e-3) / 1e9, 1),
            "kernels": kernels_l},
        "state16_schedule": {
            "state": "each worker's compensated momentum c held in bfloat16",
            "ms_per_step": round(ms_h, 4), "value": w.d / (ms_h * 1e-3),
            "step_alg_bytes_per_param": round(sum(alg_h.values()), 3),
            "step_alg_GBps": round(sum(alg_h.values()) * w.d / (ms_h * 1e-3) / 1e9, 1),
            "kernels": kernels_h},
        "tensor_list_schedule": listed,
        "one_block_step": small,
        "kernel_source_sha256": source_hash(),
    }
    del S, gsets
    L.close()
    torch.cuda.empty_cache()
    log("[bench] one-GPU share")
    out["one_gpu_share"] = one_gpu_share(w, torch, oba, synth, args.steps, args.warmup)
    torch.cuda.empty_cache()
    log("[bench] HBM streaming probes")
    ceil = hbm_ceiling(torch, w)
    out["hbm_ceiling"] = ceil
    # the dominant kernel against the probe of its own access shape
    probe = PROBE_OF.get((dom, w.g_dtype)) or PROBE_OF.get((dom, None))
    if probe in ceil["probes"]:
        c = ceil["probes"][probe]["GBps"]
        out["roofline"].update({"ceiling_probe": probe, "ceiling_GBps": c,
                                "frac_of_ceiling": round(achieved / c, 4)})
    for kernels in (out["kernels"], out["state16_schedule"]["kernels"]):
        for k, ent in kernels.items():
            pr = PROBE_OF.get((k, w.g_dtype)) or PROBE_OF.get((k, None))
            if pr in ceil["probes"] and "alg_GBps" in ent:
                ent["frac_of_ceiling"] = round(ent["alg_GBps"] / ceil["probes"][pr]["GBps"], 4)
    pr = PROBE_OF.get(("adam_warmup", w.g_dtype))
    if warm and pr in ceil["probes"] and w.n == 8:
        warm["frac_of_ceiling"] = round(warm["alg_GBps"] / ceil["probes"][pr]["GBps"], 4)
    if not args.no_cpu_baseline and w.name != "gpt2_xl":
        log("[bench] CPU oracle baseline")
        cb = cpu_baseline(w, torch, synth, args.cpu_sample,
                          single_thread=not args.no_single_thread)
        cb["gpu_over_cpu"] = round(out["value"] / cb["value"], 1)
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
