"""Seeded synthetic inputs and workload shapes for the 1-bit Adam step.

This module holds no arithmetic of the method: only sizes, segment tables and
random draws.  Both the GPU path's tests/benchmark and the CPU oracle's tests
take their inputs from here.

Workloads (d parameters, n simulated workers), each named by what it is:
  * ``tiny``      d=4096, n=2, fp32 gradients N(0,1); x0 ~ N(0, 0.02^2);
                  10 warm-up steps, freeze, 10 compression steps; one scale per
                  worker; n equal server shards.
  * ``bert_base`` d=110,000,000, n=4, fp32 gradients N(0, 1e-3^2); 50 warm-up
                  steps; n server shards floor(j*d/n) (not word aligned).
  * ``bert_large``d=336,000,000, n=8, fp16 gradients 1e-3 * Student-t(3) with
                  a fixed 1 % of coordinates exactly zero; n shards of d/n.
  * ``gpt2_xl``   1,556,920,000 parameters as 388 tensors of a 48-layer,
                  hidden-1600 transformer (vocab 50257, 1024 positions),
                  n=4; one scale per chunk of <= 2^24 elements (392 chunks),
                  fp32 gradients N(0, 1e-4^2).
  * ``quadratic`` d=64,000,000, n=8: f(x) = 1/2 sum a_k (x_k - x*_k)^2 with
                  a log-uniform on [1e-3, 1e2], x* ~ N(0,1), gradient noise
                  N(0, 0.1^2) per worker; 300 warm-up + 1700 compression steps.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BETA1 = 0.9
BETA2 = 0.999
ETA = 1e-8
LR = 1e-3
CHUNK = 1 << 24


def even_shards(d: int, n: int) -> np.ndarray:
    """n server shards [floor(j d / n), floor((j+1) d / n))."""
    return np.array([(j * d) // n for j in range(n + 1)], dtype=np.int64)


def whole(d: int) -> np.ndarray:
    return np.array([0, d], dtype=np.int64)


def gpt2_xl_tensor_sizes(layers=48, hidden=1600, vocab=50257, positions=1024):
    """Sizes of the 388 parameter tensors, back to back: token and position
    embeddings, then per layer ln1 (w, b), qkv, out-proj, ln2 (w, b), mlp-in,
    mlp-out (no linear biases), then the final LayerNorm (w, b)."""
    h = hidden
    sizes = [vocab * h, positions * h]
    for _ in range(layers):
        sizes += [h, h, h * 3 * h, h * h, h, h, h * 4 * h, 4 * h * h]
    sizes += [h, h]
    return sizes


def chunk_table(sizes, max_chunk=CHUNK) -> np.ndarray:
    """Segment offsets cutting every tensor into chunks of at most max_chunk."""
    offs = [0]
    pos = 0
    for s in sizes:
        end = pos + s
        while pos < end:
            pos = min(pos + max_chunk, end)
            offs.append(pos)
    return np.array(offs, dtype=np.int64)


@dataclass
class Workload:
    name: str
    d: int
    n: int
    g_dtype: str  # "f32" or "f16"
    seed: int
    warmup_steps: int
    wseg: np.ndarray = field(repr=False)
    sseg: np.ndarray = field(repr=False)
    grad_std: float = 1.0


def workload(name: str) -> Workload:
    if name == "tiny":
        d, n = 4096, 2
        return Workload(name, d, n, "f32", 0, 10, whole(d), even_shards(d, n), 1.0)
    if name == "bert_base":
        d, n = 110_000_000, 4
        return Workload(name, d, n, "f32", 1, 50, whole(d), even_shards(d, n), 1e-3)
    if name == "bert_large":
        d, n = 336_000_000, 8
        return Workload(name, d, n, "f16", 2, 10, whole(d), even_shards(d, n), 1e-3)
    if name == "gpt2_xl":
        t = chunk_table(gpt2_xl_tensor_sizes())
        d = int(t[-1])
        return Workload(name, d, 4, "f32", 3, 10, t, t.copy(), 1e-4)
    if name == "quadratic":
        d, n = 64_000_000, 8
        return Workload(name, d, n, "f32", 4, 300, whole(d), even_shards(d, n), 0.1)
    raise KeyError(name)


def scaled(w: Workload, d: int) -> Workload:
    """The same recipe at a smaller d (segment tables rescaled)."""
    if w.name == "gpt2_xl":
        raise ValueError("use a tensor-list prefix for the tensor-list workload")
    return Workload(w.name, d, w.n, w.g_dtype, w.seed, w.warmup_steps, whole(d),
                    even_shards(d, w.n), w.grad_std)


# --------------------------------------------------------------------------
# host (numpy) generators: small and medium sizes, parity tests
# --------------------------------------------------------------------------

def tiny_inputs(seed=0, d=4096, n=2, steps=20):
    """x0 ~ N(0, 0.02^2) and gradients G[t][i] ~ N(0, 1), float32."""
    rng = np.random.default_rng(seed)
    x0 = rng.normal(0.0, 0.02, d).astype(np.float32)
    G = rng.standard_normal((steps, n, d)).astype(np.float32)
    return x0, G


def student_t3(rng, shape):
    """Student-t with 3 degrees of freedom by definition:
    z0 / sqrt((z1^2 + z2^2 + z3^2) / 3), z ~ N(0, 1)."""
    z = rng.standard_normal((4,) + tuple(shape))
    return z[0] / np.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3.0)


def zero_mask_host(rng, d, frac=0.01):
    """Exactly round(frac*d) distinct coordinates."""
    return np.sort(rng.choice(d, size=int(round(frac * d)), replace=False))


def host_grads(rng, w: Workload, d=None, zero_idx=None):
    """One gradient set [n][d] for workload w on the host."""
    d = w.d if d is None else d
    if w.name == "bert_large":
        g = (1e-3 * student_t3(rng, (w.n, d))).astype(np.float16)
        if zero_idx is not None:
            g[:, zero_idx] = 0
        return g
    return (w.grad_std * rng.standard_normal((w.n, d))).astype(np.float32)


def host_state(rng, d, n, m_std=1e-3, delta_std=1e-4, eps_std=1e-4, v_std=1e-3):
    """A mid-training compression-stage state: x, m, v (positive), delta [n][d],
    eps.  Used for teacher-forced single-call parity."""
    x = rng.normal(0.0, 0.02, d).astype(np.float32)
    m = rng.normal(0.0, m_std, d).astype(np.float32)
    v = (rng.normal(0.0, v_std, d) ** 2).astype(np.float32)
    delta = rng.normal(0.0, delta_std, (n, d)).astype(np.float32)
    eps = rng.normal(0.0, eps_std, d).astype(np.float32)
    return dict(x=x, m=m, v=v, delta=delta, eps=eps)


# --------------------------------------------------------------------------
# device (torch) generators: full-size workloads
# --------------------------------------------------------------------------

def device_generator(seed, device="cuda"):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def device_grads(gen, w: Workload, out, zero_idx=None):
    """Fill out ([n][d] torch tensor, fp32 or fp16) with one gradient set."""
    import torch

    n, d = out.shape
    if w.name == "bert_large":
        chunk = 1 << 26
        for i in range(n):
            for lo in range(0, d, chunk):
                hi = min(d, lo + chunk)
                z = torch.randn((4, hi - lo), generator=gen, device=out.device)
                t = z[0] / torch.sqrt((z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0)
                out[i, lo:hi] = (1e-3 * t).to(out.dtype)
            if zero_idx is not None:
                out[i, zero_idx] = 0
    else:
        out.normal_(0.0, w.grad_std, generator=gen)
    return out


def device_zero_mask(gen, d, frac=0.01, device="cuda"):
    import torch

    k = int(round(frac * d))
    return torch.randperm(d, generator=gen, device=device)[:k]
