"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle
checks.  This module only draws numbers: it holds none of the attention or
position arithmetic.

Recipe
  * q, k, v: float32 N(0, 1) drawn by torch.Generator in [B, H, S, d] order
    on the requested device, multiplied by the workload's input scale
    (exact: a power of two) and rounded to the workload dtype (RNE for bf16).
    Streams: q <- seed, k <- seed + 1, v <- seed + 2.
  * sampled query rows: forced rows at chunk and window boundaries and tile
    edges, the rest uniform from numpy.random.default_rng(seed).
  * vertical-slash mask, per query head h (numpy.random.default_rng(seed +
    1000 + h)): verticals are {0..63} plus uniform draws without replacement
    from [64, S); slash offsets are {0..63} plus draws from [64, S); both
    sorted, int32.  The forced entries count toward the budgets.
"""

from __future__ import annotations

import numpy as np
import torch


def gaussian(shape, seed: int, device, scale: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_qkv(w, seed: int = 0, device="cpu", seq: int | None = None):
    """q [B, Hq, S, d], k and v [B, Hkv, S, d] for workload `w` (seq may be
    overridden for reduced-size cases)."""
    S = w.seq if seq is None else seq
    dt = torch_dtype(w.dtype)
    q = gaussian((w.batch, w.n_q_heads, S, w.head_dim), seed, device, w.input_scale, dt)
    k = gaussian((w.batch, w.n_kv_heads, S, w.head_dim), seed + 1, device, w.input_scale, dt)
    v = gaussian((w.batch, w.n_kv_heads, S, w.head_dim), seed + 2, device, w.input_scale, dt)
    return q, k, v


def sample_rows(S: int, C: int, W: int, n: int | None, seed: int = 0) -> np.ndarray:
    """Sorted unique query rows: all rows if n is None or n >= S, else the
    forced boundary rows plus seeded uniform rows up to n."""
    if n is None or n >= S:
        return np.arange(S, dtype=np.int64)
    forced = [0, 1, C - 1, C, C + 1, C + W - 2, C + W - 1, C + W, 2 * C - 1, 2 * C,
              2 * C + W - 2, 3 * C, 3 * C + W - 1, S - 2, S - 1,
              63, 64, 127, 128, 64 * 3 + 31, S // 2, S // 2 - 1]
    forced = sorted({r for r in forced if 0 <= r < S})
    rng = np.random.default_rng(seed)
    rest = set(forced)
    while len(rest) < n:
        rest.update(int(x) for x in rng.integers(0, S, size=n - len(rest)))
    return np.array(sorted(rest), dtype=np.int64)


def vs_mask(n_heads: int, S: int, n_vertical: int, n_slash: int, seed: int = 0, forced: int = 64):
    """Per-head vertical columns [n_heads, n_vertical] and slash offsets
    [n_heads, n_slash], int32, sorted ascending."""
    vert = np.zeros((n_heads, n_vertical), dtype=np.int32)
    slash = np.zeros((n_heads, n_slash), dtype=np.int32)
    for h in range(n_heads):
        rng = np.random.default_rng(seed + 1000 + h)
        fv = min(forced, n_vertical, S)
        fs = min(forced, n_slash, S)
        dv = rng.choice(S - forced, size=n_vertical - fv, replace=False) + forced if n_vertical > fv else []
        ds = rng.choice(S - forced, size=n_slash - fs, replace=False) + forced if n_slash > fs else []
        vert[h] = np.sort(np.concatenate([np.arange(fv), np.asarray(dv, dtype=np.int64)]))
        slash[h] = np.sort(np.concatenate([np.arange(fs), np.asarray(ds, dtype=np.int64)]))
    return vert, slash
