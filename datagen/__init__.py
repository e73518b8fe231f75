"""Seeded synthetic layers for GPTQ: weights W and calibration activations X.

This module only draws random numbers and stores them; it holds none of the
quantization method's arithmetic.  Both the fp64 oracle (``oracle/``) and the
GPU library's tests and benchmark read the layers it makes, so the two sides
see the same bytes.

The pages measure GPTQ on real models fed with a few hundred calibration
texts (page "LLM 量化方法原理与实现详解", §3.1 PTQ; page "PTQ 权重量化：从 GPTQ
到 AWQ", section "GPTQ：Hessian 引导的误差补偿").  Neither the models nor the
texts exist here, so every workload is a synthetic stand-in with the shape and
value statistics listed in ``RECIPES``.

Generator recipe (fixed so that any reader can regenerate a layer):

* ``numpy.random.SeedSequence(seed).spawn(4)`` gives four streams:
  0 = W, 1 = X body, 2 = choice of outlier channels, 3 = per-channel sigma.
* X is generated in chunks of ``CHUNK_ROWS`` rows (channels); chunk ``c``
  uses ``Generator(PCG64(stream1.spawn(n_chunks)[c]))`` so chunks can be drawn
  in parallel threads without changing the result.
* ``N(0, s)`` means standard deviation ``s``.  Student-t bodies use
  ``standard_t(3)`` without renormalisation.
* Outlier channels: ``k = round(frac * d_in)`` rows chosen with
  ``choice(d_in, k, replace=False)`` and multiplied after sampling.
* bf16 storage is round-to-nearest-even of the fp32 sample; X is stored
  ``[d_in][n_tok]`` row-major (one row per input channel).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

CHUNK_ROWS = 64

# Workloads.  ``group = 0`` means one group per output row (per-channel grid).
RECIPES = {
    # Tiny layer: both the oracle and exhaustive checks finish in seconds.
    "tiny": dict(d_out=64, d_in=128, n_tok=512, w_std=0.02, body="normal",
                 x_dtype="f32", outliers=("channels", (5, 77), 20.0),
                 bits=4, sym=True, group=32, block=32, damp=0.01, act_order=False),
    # 7B-like attention q projection.
    "q_proj_7b": dict(d_out=4096, d_in=4096, n_tok=262144, w_std=0.02, body="normal",
                      x_dtype="bf16", outliers=("frac", 0.01, 15.0),
                      bits=4, sym=False, group=128, block=128, damp=0.01, act_order=False),
    # 7B-like MLP down projection with heavy-tailed activations.
    "down_proj_7b": dict(d_out=4096, d_in=11008, n_tok=65536, w_std=0.015, body="student_t3",
                         x_dtype="bf16", outliers=("frac", 0.005, 30.0),
                         bits=4, sym=False, group=128, block=128, damp=0.01, act_order=False),
    # 70B-like attention output projection, 3-bit, one scale per output row.
    "o_proj_70b": dict(d_out=8192, d_in=8192, n_tok=131072, w_std=0.01, body="normal",
                       x_dtype="bf16", outliers=("frac", 0.01, 20.0),
                       bits=3, sym=False, group=0, block=128, damp=0.01, act_order=False),
    # 70B-like MLP up projection, per-channel lognormal scales, Hessian order.
    "up_proj_70b": dict(d_out=28672, d_in=8192, n_tok=131072, w_std=0.01, body="lognormal_channels",
                        x_dtype="bf16", outliers=None,
                        bits=4, sym=True, group=128, block=128, damp=0.01, act_order=True),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the raw 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def recipe(name: str, **overrides) -> dict:
    r = dict(RECIPES[name])
    r.update({k: v for k, v in overrides.items() if v is not None})
    r["name"] = name
    return r


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(4)


def make_weight(r: dict, seed: int = 0) -> np.ndarray:
    ss = _streams(seed)
    rng = np.random.Generator(np.random.PCG64(ss[0]))
    w = rng.standard_normal((r["d_out"], r["d_in"]), dtype=np.float32)
    w *= np.float32(r["w_std"])
    return w


def _channel_scales(r: dict, seed: int) -> np.ndarray:
    """Per-channel multiplier of X rows (outliers and lognormal sigmas)."""
    ss = _streams(seed)
    d_in = r["d_in"]
    mult = np.ones(d_in, dtype=np.float32)
    if r["body"] == "lognormal_channels":
        rng3 = np.random.Generator(np.random.PCG64(ss[3]))
        mult *= np.exp(rng3.standard_normal(d_in)).astype(np.float32)
    o = r.get("outliers")
    if o is not None:
        if o[0] == "channels":
            idx = np.array([c for c in o[1] if c < d_in], dtype=np.int64)
        else:
            k = int(round(o[1] * d_in))
            rng2 = np.random.Generator(np.random.PCG64(ss[2]))
            idx = rng2.choice(d_in, k, replace=False)
        mult[idx] *= np.float32(o[2])
    return mult


def make_activations(r: dict, seed: int = 0, threads: int | None = None) -> np.ndarray:
    """X [d_in][n_tok]: uint16 bf16 bit patterns, or float32 when ``x_dtype == 'f32'``."""
    d_in, n = r["d_in"], r["n_tok"]
    ss = _streams(seed)
    n_chunks = (d_in + CHUNK_ROWS - 1) // CHUNK_ROWS
    kids = ss[1].spawn(n_chunks)
    mult = _channel_scales(r, seed)
    bf16 = r["x_dtype"] == "bf16"
    out = np.empty((d_in, n), dtype=np.uint16 if bf16 else np.float32)

    def one(c: int) -> None:
        r0, r1 = c * CHUNK_ROWS, min(d_in, (c + 1) * CHUNK_ROWS)
        rng = np.random.Generator(np.random.PCG64(kids[c]))
        if r["body"] == "student_t3":
            body = rng.standard_t(3, size=(r1 - r0, n)).astype(np.float32)
        else:
            body = rng.standard_normal((r1 - r0, n), dtype=np.float32)
        body *= mult[r0:r1, None]
        out[r0:r1] = f32_to_bf16_bits(body) if bf16 else body

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if n_chunks == 1 or threads <= 1:
        for c in range(n_chunks):
            one(c)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(n_chunks)))
    return out


def make_layer(name: str, seed: int = 0, **overrides) -> dict:
    """Recipe + W (fp32 [d_out][d_in]) + X (see ``make_activations``)."""
    r = recipe(name, **overrides)
    r["W"] = make_weight(r, seed)
    r["X"] = make_activations(r, seed)
    return r
