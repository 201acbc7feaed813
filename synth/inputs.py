"""Seeded synthetic q/k/v (and upstream gradients) for the VSA workloads.

Shared by the oracle side and the GPU side of every parity test and of the
bench, so both consume identical bits.  It holds none of the method's
arithmetic: it only draws random numbers and shapes them into the value
structure stated per workload.

Recipe (per batch b, head h, with seed s):
  * stream  = numpy Generator(PCG64(SeedSequence([s, b, h])))
  * z_q, z_k, z_v = stream.standard_normal((N, d), float32), in that order
  * structure S, drawn next from the same stream:
      - "offset": one vector o_c ~ N(0,1)^d per 4x4x4 cube; every token of
        cube c gets o_c (so q and k of one cube share a direction and the
        top-K is well separated);
      - "field": a smooth low-frequency field with 4 cosine modes,
        F[t,y,x,ch] = sum_j a[j,ch] cos(2pi(ft_j t/T + fy_j y/Hh + fx_j x/Ww) + phi[j,ch]),
        frequencies (ft,fy,fx) in {0,1,2}^3 minus the zero vector (4 distinct
        draws), a ~ N(0,1), phi ~ U[0, 2pi); each channel then normalised to
        zero mean and unit RMS over the real grid.
  * q = z_q + alpha*S, k = z_k + alpha*S, v = z_v   (float32 arithmetic)
  * bf16 workloads round q, k, v to bfloat16 (round-to-nearest-even, via
    torch.bfloat16); values are returned as float32 arrays holding exactly
    the bf16 values.
  * upstream gradients for the backward use a second stream,
    SeedSequence([s + 1, b, h]): dO_fine then dO_coarse, each N(0,1) (N, d),
    rounded the same way.
Tokens are in raster order r = (t*Hh + y)*Ww + x.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

from .configs import Workload


def _round_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32, copy=False)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return t.to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def _stream(seed: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b, h])))


def _token_coords(w: Workload):
    t, y, x = np.meshgrid(np.arange(w.T), np.arange(w.Hh), np.arange(w.Ww), indexing="ij")
    return t.reshape(-1), y.reshape(-1), x.reshape(-1)


def _offset_structure(w: Workload, rng: np.random.Generator) -> np.ndarray:
    _, ch_n, cw_n = w.cube_grid
    o = rng.standard_normal((w.C, w.d), dtype=np.float32)
    t, y, x = _token_coords(w)
    cube_of_token = ((t // 4) * ch_n + (y // 4)) * cw_n + (x // 4)
    return o[cube_of_token]


_FREQS = np.array([(a, b, c) for a in range(3) for b in range(3) for c in range(3)
                   if (a, b, c) != (0, 0, 0)], dtype=np.float64)


def _field_structure(w: Workload, rng: np.random.Generator) -> np.ndarray:
    modes = rng.choice(len(_FREQS), size=4, replace=False)
    amp = rng.standard_normal((4, w.d))
    phase = rng.uniform(0.0, 2.0 * np.pi, size=(4, w.d))
    t, y, x = _token_coords(w)
    f = _FREQS[modes]                                   # (4, 3)
    theta = 2.0 * np.pi * (np.outer(t / w.T, f[:, 0]) + np.outer(y / w.Hh, f[:, 1])
                           + np.outer(x / w.Ww, f[:, 2]))      # (N, 4)
    # cos(theta + phi) = cos(theta)cos(phi) - sin(theta)sin(phi)
    field = np.cos(theta) @ (amp * np.cos(phase)) - np.sin(theta) @ (amp * np.sin(phase))
    field -= field.mean(axis=0, keepdims=True)
    rms = np.sqrt((field * field).mean(axis=0, keepdims=True))
    field /= np.where(rms > 0, rms, 1.0)
    return field.astype(np.float32)


def make_head(w: Workload, b: int, h: int, seed: int = 0,
              grads: bool = False) -> Dict[str, np.ndarray]:
    """q, k, v (and dO_fine, dO_coarse if grads) for one (b, h), each (N, d) float32."""
    rng = _stream(seed, b, h)
    zq = rng.standard_normal((w.N, w.d), dtype=np.float32)
    zk = rng.standard_normal((w.N, w.d), dtype=np.float32)
    zv = rng.standard_normal((w.N, w.d), dtype=np.float32)
    if w.structure == "offset":
        s = _offset_structure(w, rng)
    elif w.structure == "field":
        s = _field_structure(w, rng)
    else:
        raise ValueError(w.structure)
    a = np.float32(w.alpha)
    out = {
        "q": _round_dtype(zq + a * s, w.dtype),
        "k": _round_dtype(zk + a * s, w.dtype),
        "v": _round_dtype(zv, w.dtype),
    }
    if grads:
        g = _stream(seed + 1, b, h)
        out["do_fine"] = _round_dtype(g.standard_normal((w.N, w.d), dtype=np.float32), w.dtype)
        out["do_coarse"] = _round_dtype(g.standard_normal((w.N, w.d), dtype=np.float32), w.dtype)
    return out


def make_inputs(w: Workload, seed: int = 0, heads: Optional[Sequence[int]] = None,
                grads: bool = False, workers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Arrays of shape (B, len(heads), N, d) float32 (bf16-exact for bf16 workloads)."""
    heads = list(range(w.H)) if heads is None else list(heads)
    names = ["q", "k", "v"] + (["do_fine", "do_coarse"] if grads else [])
    out = {n: np.empty((w.B, len(heads), w.N, w.d), np.float32) for n in names}
    jobs = [(b, hi, h) for b in range(w.B) for hi, h in enumerate(heads)]

    def one(job):
        b, hi, h = job
        res = make_head(w, b, h, seed, grads)
        for n in names:
            out[n][b, hi] = res[n]

    nw = workers or min(8, os.cpu_count() or 1, len(jobs))
    if nw <= 1:
        for j in jobs:
            one(j)
    else:
        with _cf.ThreadPoolExecutor(nw) as ex:
            list(ex.map(one, jobs))
    return out


def sample_plan(w: Workload, seed: int = 1234, n_heads: int = 4, n_qcubes: int = 16):
    """Heads and query cubes the oracle checks on a shape too large for it.

    4 distinct heads; per head the first and last cube (the last is the
    corner cube with the fewest valid tokens) plus n_qcubes-2 distinct random
    others.
    """
    rng = np.random.default_rng(seed)
    heads = sorted(rng.choice(w.H, size=min(n_heads, w.H), replace=False).tolist())
    others = [c for c in range(1, w.C - 1)]
    pick = rng.choice(len(others), size=max(0, min(n_qcubes - 2, len(others))), replace=False)
    qcubes = sorted({0, w.C - 1} | {others[i] for i in pick})
    return heads, qcubes


def as_torch(x: np.ndarray, dtype: str, device=None):
    """Exact conversion of a generated array to a torch tensor of the workload dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device) if device is not None else t
