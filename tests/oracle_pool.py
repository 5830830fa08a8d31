"""A process pool for the CPU oracle at full workload sizes.  Test
infrastructure.

The oracle's layer (`oracle.moe.forward`) evaluates one MLP term per touched
expert and sums the terms in a fixed order; `map_fn` decides what evaluates the
terms.  At the full sizes (hundreds of 4096 x 1024 experts) the terms and the
oracle's NVFP4 weight quantization take minutes on one core, so the parity tests
hand both to this pool.  The order of the sum, and so every bit of the result,
is that of the builtin map.

Workers are fresh interpreters (spawn start method: nothing of the parent,
GPU state included, is inherited), import only numpy and `oracle`, and run
BLAS on one thread each.  The pool is sized to the host's CPU share, at most 16.
"""
import atexit
import os

import numpy as np

from oracle import moe, nvfp4

_POOL = None
_LIMITS = None


def _init_worker():
    global _LIMITS
    try:
        from threadpoolctl import threadpool_limits
        _LIMITS = threadpool_limits(limits=1)
    except Exception:               # pragma: no cover - threadpoolctl ships with the image
        _LIMITS = None


def workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def pool():
    """The shared pool (created on first use, shut down at exit)."""
    global _POOL
    if _POOL is None:
        import multiprocessing as mp
        from concurrent.futures import ProcessPoolExecutor
        _POOL = ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"),
                                    initializer=_init_worker)
        atexit.register(_POOL.shutdown)
    return _POOL


def pool_map(fn, iterable):
    """Ordered map on the pool (a drop-in for the builtin map)."""
    return pool().map(fn, iterable, chunksize=1)


def bf16_bits_to_f32(bits):
    """uint16 bf16 bit patterns -> exact fp32 values."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_expert_bits(job):
    """(w13 bf16 bits [2F, d], w2 bf16 bits [d, F]) -> the oracle's quantized
    expert dict (the same as tests.oracle_helpers.quantize_expert_oracle)."""
    w13_bits, w2_bits = job
    q13 = nvfp4.quantize_weight(bf16_bits_to_f32(w13_bits))
    q2 = nvfp4.quantize_weight(bf16_bits_to_f32(w2_bits))
    return {"w13": q13["codes"], "w13_scale": q13["scales"], "g13": q13["g"],
            "w2": q2["codes"], "w2_scale": q2["scales"], "g2": q2["g"]}


def forward(*args, **kw):
    """oracle.moe.forward with its expert terms evaluated on the pool."""
    return moe.forward(*args, map_fn=pool_map, **kw)
