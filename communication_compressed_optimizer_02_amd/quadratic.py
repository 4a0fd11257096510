"""End-to-end run of the two-stage method on a synthetic noisy quadratic.

f(x) = 1/2 sum_k a_k (x_k - x*_k)^2 with a_k log-uniform on [1e-3, 1e2] and
x* ~ N(0, 1); each of the n workers sees the gradient a*(x - x*) plus its own
N(0, 0.1^2) noise.  1-bit Adam runs `warmup` plain Adam steps through the
library's warm-up kernel, freezes the variance, then runs compression steps
(deferred-residual layout); the baseline is uncompressed Adam (the same
warm-up kernel, no bias correction) on the identical noise stream.  The loss
is evaluated in binary64 every `every` steps.  The pages claim the
compressed run matches Adam's convergence ([Tang] 1, 7.1, 8) without
numbers, so the ratio is reported, not gated.  Both warm-up variants run:
the bare recurrences of the definition paragraph ([AIMech]) and Kingma-Ba
bias correction; after a short warm-up the bare v is far below its
stationary value, which inflates the frozen step sizes.

    python -m communication_compressed_optimizer_02_amd.quadratic --d 64000000 --n 8
    python -m communication_compressed_optimizer_02_amd.quadratic --auto-freeze 20 0.02
"""
from __future__ import annotations

import argparse
import json
import time

from . import binding as oba
from . import synth


class Problem:
    """The quadratic and its noisy per-worker gradients (harness arithmetic,
    not the method's)."""

    def __init__(self, d, n, seed, device="cuda", noise=0.1):
        import torch

        self.d, self.n, self.noise = d, n, noise
        gen = torch.Generator(device=device)
        gen.manual_seed(int(seed))
        self.a = torch.pow(10.0, torch.empty(d, device=device).uniform_(-3.0, 2.0, generator=gen))
        self.xstar = torch.empty(d, device=device).normal_(0.0, 1.0, generator=gen)
        self.seed = seed
        self.device = device

    def noise_stream(self):
        import torch

        gen = torch.Generator(device=self.device)
        gen.manual_seed(int(self.seed) + 1)
        return gen

    def grads(self, x, xi, out):
        """out[i] = a*(x - x*) + noise*xi[i] (binary32, this order)."""
        base = self.a * (x - self.xstar)
        out.copy_(base.unsqueeze(0) + self.noise * xi)
        return out

    def loss(self, x):
        import torch

        r = (x.double() - self.xstar.double())
        return float(0.5 * torch.sum(self.a.double() * r * r))


def run(d, n, steps, warmup, seed=4, every=10, lr=synth.LR, beta1=synth.BETA1,
        beta2=synth.BETA2, eta=synth.ETA, compressed=True, bias_correction=False, log=None,
        auto_freeze=None, info=None, local_momentum=False, state16=None):
    """Returns (losses {step: f}, optimizer ms per step, gradient ms per step).
    bias_correction: Kingma-Ba factors 1-b^t in the warm-up (and in the
    frozen variance); off = the bare recurrences.  auto_freeze = (window,
    rtol): the warm-up ends when the variance norm ||v/bc2|| levels off
    (library plateau test), at most at step `warmup`; info["freeze_step"]
    receives the last warm-up step.  local_momentum: every worker keeps its
    own momentum in the compression stage (the broadcast only moves x).
    state16 ("f16" or "bf16"): the workers' compensated momenta are held in
    that 16-bit format in the compression stage."""
    import torch

    P = Problem(d, n, seed)
    L = oba.Layout(d, n, synth.whole(d), synth.even_shards(d, n))
    S = oba.State(L)
    xi = torch.empty((n, d), device="cuda")
    gen = P.noise_stream()
    losses = {0: P.loss(S.x)}
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    t_opt = t_grad = 0.0
    vnorm = torch.zeros(1, dtype=torch.float64, device="cuda") if auto_freeze else None
    trig = oba.Plateau(*auto_freeze) if auto_freeze else None
    frozen_at = 0
    for t in range(1, steps + 1):
        e[0].record()
        xi.normal_(0.0, 1.0, generator=gen)
        P.grads(S.x, xi, S.g)
        e[1].record()
        if not compressed or not frozen_at:
            bc1, bc2 = (1 - beta1 ** t, 1 - beta2 ** t) if bias_correction else (1.0, 1.0)
            S.warmup(lr, beta1, beta2, eta, bc1, bc2, vnorm=vnorm)
            stop = t == warmup
            if trig is not None and trig.observe(float(vnorm.item()) / bc2):
                stop = True
            if compressed and stop:
                S.freeze(eta, bc2)
                if local_momentum:
                    S.start_local_momentum()
                if state16:
                    S.start_state16(state16)
                frozen_at = t
        elif local_momentum:
            S.step_local(beta1, lr)
        elif state16:
            S.step_deferred16(beta1, lr)
        else:
            S.step_deferred(beta1, lr)
        e[2].record()
        torch.cuda.synchronize()
        t_grad += e[0].elapsed_time(e[1])
        t_opt += e[1].elapsed_time(e[2])
        if t % every == 0 or t == steps:
            losses[t] = P.loss(S.x)
            if log and t % (every * 50) == 0:
                log(f"  step {t}: f = {losses[t]:.6e}")
    L.close()
    if info is not None:
        info["freeze_step"] = frozen_at
    return losses, t_opt / steps, t_grad / steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--d", type=int, default=64_000_000)
    ap.add_argument("--n", type=int, default=8)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--seed", type=int, default=4)
    ap.add_argument("--local-momentum", action="store_true",
                    help="per-worker momentum in the compression stage")
    ap.add_argument("--state16", choices=["f16", "bf16"],
                    help="hold the workers' compensated momenta in this 16-bit format")
    ap.add_argument("--auto-freeze", nargs=2, type=float, metavar=("WINDOW", "RTOL"),
                    help="end the warm-up when the variance norm levels off (at most at "
                         "--warmup), instead of at --warmup")
    args = ap.parse_args()
    auto = (int(args.auto_freeze[0]), args.auto_freeze[1]) if args.auto_freeze else None
    local = args.local_momentum

    def log(msg):
        print(msg, flush=True)

    marks = [m for m in (args.warmup, 500, 1000, args.steps) if 0 < m <= args.steps]
    out = {"workload": "quadratic", "d": args.d, "n_workers": args.n, "steps": args.steps,
           "warmup": args.warmup, "momentum": "per-worker" if args.local_momentum else "shared",
           "worker_state": args.state16 or "f32"}
    t0 = time.time()
    for name, bc in (("bare", False), ("bias_corrected", True)):
        log(f"[quadratic] {name} warm-up: 1-bit Adam, d={args.d} n={args.n} "
            f"steps={args.steps} warm-up={args.warmup} ({time.time() - t0:.0f} s)")
        info = {}
        f1, opt1, gr1 = run(args.d, args.n, args.steps, args.warmup, args.seed,
                            bias_correction=bc, log=log, auto_freeze=auto, info=info,
                            local_momentum=local, state16=args.state16)
        log(f"[quadratic] {name} warm-up: Adam baseline ({time.time() - t0:.0f} s)")
        fa, opta, _ = run(args.d, args.n, args.steps, args.warmup, args.seed, compressed=False,
                          bias_correction=bc, log=log)
        out[name] = {
            "freeze_step": info["freeze_step"],
            "loss_1bit": {str(m): f1[m] for m in marks if m in f1},
            "loss_adam": {str(m): fa[m] for m in marks if m in fa},
            "ratio_1bit_over_adam": {str(m): f1[m] / fa[m] for m in marks if m in f1},
            "optimizer_ms_per_step": {"1bit_mean_over_run": round(opt1, 4),
                                      "adam": round(opta, 4)},
        }
        out["initial_loss"] = f1[0]
        out["gradient_synthesis_ms_per_step"] = round(gr1, 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
