"""Seeded synthetic inputs for the MoE layer.

This module draws random numbers and nothing else: it holds none of the layer's
arithmetic, so the GPU path and the CPU oracle can both take their inputs from it.

Recipe (one ``numpy.random.default_rng(seed)`` stream, draws in this order):

1. ``x``      [T, d]      N(0, x_std)
2. ``w_gate`` [E, d]      N(0, wg_std)            (router, nn.Linear layout [out, in])
3. ``bias``   [E]         N(0, b_std) if bias == "normal"; -s*ln(e+1) if "zipf"; else absent
4. ``w1``     [E, 2f, d]  N(0, 1/sqrt(d))         (gate rows first, then up rows)
5. ``w2``     [E, d, f]   N(0, 1/sqrt(f))
6. ``dout``   [T, d]      N(0, 1)                 (upstream gradient; only when backward)

Values are drawn as float32 (standard normal times the std, in float32) and, for
bf16 workloads, rounded to bfloat16 with round-to-nearest-even.  ``bias`` stays
float32.  Experts are drawn one at a time, which fixes the stream order.

``redraw_rows`` draws replacement rows of ``x`` from a separate stream
``default_rng([seed, 1, attempt])``: callers that need routing decisions to be
clear of ties use it and decide themselves which rows to replace.

``micro_batch`` draws the ``x`` [T, d] and ``dout`` [T, d] of micro-batch j of a
gradient-accumulation step (the weights stay those of ``generate``) from the
stream ``default_rng([seed, 3, j])``, with ``generate``'s distributions.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable

import numpy as np
import torch

from .configs import MoEConfig


def _cast(a: np.ndarray, act: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if act == "bf16":
        return t.to(torch.bfloat16)  # round-to-nearest-even
    if act == "f32":
        return t
    raise ValueError(f"unknown dtype {act!r}")


def generate(cfg: MoEConfig, seed: int | None = None, with_dout: bool | None = None) -> Dict[str, torch.Tensor]:
    """Draw every input of one layer problem.  Returns CPU tensors."""
    seed = cfg.seed if seed is None else seed
    with_dout = cfg.backward if with_dout is None else with_dout
    rng = np.random.default_rng(seed)
    f32 = np.float32
    out: Dict[str, torch.Tensor] = {}
    out["x"] = _cast(rng.standard_normal((cfg.T, cfg.d), dtype=f32) * f32(cfg.x_std), cfg.act)
    out["w_gate"] = _cast(rng.standard_normal((cfg.E, cfg.d), dtype=f32) * f32(cfg.wg_std), cfg.act)
    if cfg.bias == "normal":
        out["bias"] = torch.from_numpy(rng.standard_normal(cfg.E, dtype=f32) * f32(cfg.b_std))
    elif cfg.bias == "zipf":
        e = np.arange(cfg.E, dtype=np.float64)
        out["bias"] = torch.from_numpy((-cfg.zipf_s * np.log(e + 1.0)).astype(f32))
    elif cfg.bias is not None:
        raise ValueError(f"unknown bias kind {cfg.bias!r}")
    dt = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    w1 = torch.empty((cfg.E, 2 * cfg.f, cfg.d), dtype=dt)
    s1 = f32(1.0 / math.sqrt(cfg.d))
    for e in range(cfg.E):
        w1[e] = _cast(rng.standard_normal((2 * cfg.f, cfg.d), dtype=f32) * s1, cfg.act)
    out["w1"] = w1
    w2 = torch.empty((cfg.E, cfg.d, cfg.f), dtype=dt)
    s2 = f32(1.0 / math.sqrt(cfg.f))
    for e in range(cfg.E):
        w2[e] = _cast(rng.standard_normal((cfg.d, cfg.f), dtype=f32) * s2, cfg.act)
    out["w2"] = w2
    if with_dout:
        out["dout"] = _cast(rng.standard_normal((cfg.T, cfg.d), dtype=f32), cfg.act)
    if cfg.noise_std > 0:
        # routing noise from a stream of its own (the other inputs do not move)
        nrng = np.random.default_rng([seed, 2])
        out["noise"] = torch.from_numpy(nrng.standard_normal((cfg.T, cfg.E), dtype=f32) * f32(cfg.noise_std))
    return out


def redraw_rows(cfg: MoEConfig, x: torch.Tensor, rows: Iterable[int], attempt: int,
                seed: int | None = None) -> torch.Tensor:
    """Replace the given rows of ``x`` (in ascending order) with fresh draws.

    The replacement stream is ``default_rng([seed, 1, attempt])``; the result is a
    new tensor, ``x`` is not modified."""
    seed = cfg.seed if seed is None else seed
    rows = np.unique(np.asarray(list(rows), dtype=np.int64))
    y = x.clone()
    if rows.size == 0:
        return y
    rng = np.random.default_rng([seed, 1, attempt])
    fresh = rng.standard_normal((rows.size, cfg.d), dtype=np.float32) * np.float32(cfg.x_std)
    y[torch.from_numpy(rows)] = _cast(fresh, cfg.act)
    return y


def micro_batch(cfg: MoEConfig, j: int, T: int | None = None, seed: int | None = None) -> Dict[str, torch.Tensor]:
    """x and dout of micro-batch j (T tokens, default cfg.T).  Returns CPU tensors."""
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    rng = np.random.default_rng([seed, 3, j])
    f32 = np.float32
    out = {"x": _cast(rng.standard_normal((T, cfg.d), dtype=f32) * f32(cfg.x_std), cfg.act)}
    if cfg.backward:
        out["dout"] = _cast(rng.standard_normal((T, cfg.d), dtype=f32), cfg.act)
    return out
