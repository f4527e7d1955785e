"""Independent brute force for pinning the oracle on tiny inputs.

Pure Python / numpy loops in float64 that never form the three rotated query
variants.  The logit of a causal pair is taken in the pairwise-relative form
of RoPE: with z = x[m] + i x[m + d/2] per frequency m,

    < R(a) q, R(b) k > = sum_m Re( z_q(m) * conj(z_k(m)) * exp(i (a - b) theta_m) ),

and the remapped distance a - b is read from the prose of the page
"Qwen2.5-1M 不重训外推 1M" (mizuki-eaf.pages.dev, sections Intra-Chunk,
Successive-Chunk and Inter-Chunk Attention) as a distance, not as a
difference of position indices:

    same chunk                       -> the true distance i - j
    adjacent chunk, row inside W     -> the true distance i - j
    adjacent chunk, row outside W    -> the inter-chunk rule
    chunks two or more apart         -> inter-chunk rule: the pinned query
                                        index C + W - 1 minus the key's
                                        periodic position j mod C
"""

from __future__ import annotations

import cmath
import math

import numpy as np


def dca_distance(i: int, j: int, C: int, W: int) -> int:
    ci, cj = i // C, j // C
    if ci == cj:
        return i - j
    if ci == cj + 1 and (i - ci * C) < W:
        return i - j
    return (C + W - 1) - (j - cj * C)


def theta(d: int, base: float):
    return [base ** (-2.0 * m / d) for m in range(d // 2)]


def pair_logit(q, k, dist: int, th) -> float:
    h = len(q) // 2
    acc = 0.0
    for m in range(h):
        zq = complex(q[m], q[m + h])
        zk = complex(k[m], k[m + h])
        acc += (zq * zk.conjugate() * cmath.exp(1j * dist * th[m])).real
    return acc


def attention(q, k, v, C: int, W: int, base: float, tau: float, dist_fn=dca_distance,
              active=None):
    """q [Hq, S, d], k and v [Hkv, S, d] (numpy float64) -> out [Hq, S, d], lse [Hq, S].
    active(h, i, j) -> bool optionally restricts the causal pairs."""
    Hq, S, d = q.shape
    Hkv = k.shape[0]
    group = Hq // Hkv
    th = theta(d, base)
    scale = tau / math.sqrt(d)
    out = np.zeros((Hq, S, d))
    lse = np.zeros((Hq, S))
    for h in range(Hq):
        kv = h // group
        for i in range(S):
            js = [j for j in range(i + 1) if active is None or active(h, i, j)]
            logits = [scale * pair_logit(q[h, i], k[kv, j], dist_fn(i, j, C, W), th) for j in js]
            mx = max(logits)
            w = [math.exp(s - mx) for s in logits]
            tot = sum(w)
            for wj, j in zip(w, js):
                out[h, i] += (wj / tot) * v[kv, j]
            lse[h, i] = mx + math.log(tot)
    return out, lse


def vs_scores(q_last, rows, k, base: float, tau: float):
    """Column and diagonal sums of the attention of the rows `rows` under
    continuous positions (distance i - j for every pair), from the pairwise
    form of RoPE: q_last [Hq, n, d], k [Hkv, S, d] (numpy float64) ->
    vertical [Hq, S], slash [Hq, S]."""
    Hq, n, d = q_last.shape
    Hkv, S, _ = k.shape
    group = Hq // Hkv
    th = theta(d, base)
    vertical = np.zeros((Hq, S))
    slash = np.zeros((Hq, S))
    for h in range(Hq):
        kv = h // group
        for a, i in enumerate(rows):
            lg = [tau / math.sqrt(d) * pair_logit(q_last[h, a], k[kv, j], i - j, th) for j in range(i + 1)]
            mx = max(lg)
            w = [math.exp(x - mx) for x in lg]
            tot = sum(w)
            for j in range(i + 1):
                vertical[h, j] += w[j] / tot
                slash[h, i - j] += w[j] / tot
    return vertical, slash
