"""1-bit Adam compression-stage step on AMD MI355X (gfx950).

The method runs in hand-written HIP kernels behind the C ABI of
``include/oba.h`` (liboba.so, built in-tree); ``binding`` is its thin
Python front end and ``synth`` holds the seeded synthetic workloads.
"""
from .binding import (OBA_BF16, OBA_F16, OBA_F32, Layout, ObaError, Plateau, State, TensorList,
                      adam_warmup_step, adam_warmup_step_listed, compress_deferred_listed,
                      decompress_update_listed,
                      adam_warmup_step_vnorm, compress, compress_deferred_local,
                      compress_deferred, decompress_update, deferred_errors, freeze_variance,
                      server_momentum, server_reduce_recompress,
                      server_reduce_recompress_deferred, step_small, timing_enable, timing_read, timing_reset, validate)

__all__ = [
    "OBA_BF16", "OBA_F16", "OBA_F32", "Layout", "ObaError", "Plateau", "State", "TensorList",
    "adam_warmup_step", "adam_warmup_step_listed", "compress_deferred_listed",
    "decompress_update_listed",
    "adam_warmup_step_vnorm", "compress", "compress_deferred_local",
    "compress_deferred", "decompress_update", "deferred_errors", "freeze_variance",
    "server_momentum", "server_reduce_recompress", "server_reduce_recompress_deferred",
    "step_small", "timing_enable",
    "timing_read", "timing_reset", "validate",
]
