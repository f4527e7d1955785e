"""Dual Chunk Attention (DCA) prefill attention: plain CPU oracle.

TEST INFRASTRUCTURE. Only the test suite, the smoke check of the package entry
file and the CPU-baseline leg of the benchmark may import this module. The
library's compute path never reaches it, and it shares no code, table or
helper with the HIP kernels or their host code.

Everything is computed in float64 on the CPU with plain PyTorch operations,
in the order the definition states. Inputs may be bf16 or fp32 tensors; they
are widened exactly to float64.

Sources (web pages this follows):
  [mizuki]  "Qwen2.5-1M 不重训外推 1M", mizuki-eaf.pages.dev -- the only page that
            states the DCA mapping rules (sections "核心思想", "Intra-Chunk
            Attention", "Successive-Chunk Attention", "Inter-Chunk Attention"),
            DCA + YaRN (section "DCA + YaRN") and MInference vertical-slash
            sparsity (sections "跟 NSA / 其他稀疏注意力的区别",
            "稀疏注意力 + 核优化").
  [yudong]  "Qwen-2.5 explained", yudonglee.me -- section 3 (GQA, RoPE base 1e7)
            and section 4 (DCA narrative).

Readings taken where the pages leave a step open (each is a documented
choice, listed again in the design notes):
  * chunk length C; key j sits at position j mod C            [mizuki, 核心思想 / Inter-Chunk]
  * successive-chunk local window is a query-row window: a row whose
    in-chunk offset r < W sees the previous chunk at true distance, others
    fall back to the pinned inter position: Pq_succ = min(C + r, C + W - 1)
                                                               [mizuki, Successive-Chunk]
  * the pinned inter-chunk query index is C + W - 1, so every remapped
    distance lies in [0, C + W - 1]                            [mizuki, Inter-Chunk]
  * RoPE pairs are half-split (m, m + d/2), rotary dim = d, theta_m =
    base^(-2m/d)                                               [yudong §3; mizuki §1]
  * the YaRN temperature multiplies every logit once, on top of 1/sqrt(d)
                                                               [mizuki, DCA + YaRN]
  * the vertical-slash mask is tile-granular on 64x64 tiles and is defined on
    true indices (key j, offset i - j), not on remapped positions
                                                               [mizuki, 稀疏注意力 + 核优化]
  * causal, self included, positions start at 0; query head h reads KV head
    h // (Hq / Hkv).
  * online vertical-slash selection (the pages only say that key tokens are
    chosen from the attention map's vertical-slash pattern with continuous
    relative positions restored): the last n query rows attend with RoPE at
    their true indices (and the same logit scale as the attention); a key
    column scores the sum of its softmax weights over those rows, a diagonal
    i - j = o the sum along it; each head keeps the first `forced` columns and
    offsets plus the highest-scoring others up to its budgets, ties to the
    smaller index                                              [mizuki, 稀疏注意力 + 核优化]

No function here is "parity unpinned": each is pinned by the CPU tests to
closed forms, brute force, hand-worked fixtures or reductions to vanilla RoPE
attention (see tests/test_oracle_pins.py).
"""

from __future__ import annotations

import math

import torch

F64 = torch.float64

# Region labels of a (query row, key) pair.  [mizuki, 核心思想: the L x L
# attention matrix is split into intra-chunk, successive-chunk and
# inter-chunk parts.]
INTRA, SUCC, INTER = 0, 1, 2

TILE = 64  # the vertical-slash mask's unit: 64 x 64 (query, key) tiles


# ---------------------------------------------------------------------------
# 1. Position-index map  [mizuki, Intra-Chunk / Successive-Chunk / Inter-Chunk]
# ---------------------------------------------------------------------------

def pinned_query_position(C: int, W: int) -> int:
    """The large fixed query index used for inter-chunk pairs: C + W - 1."""
    return C + W - 1


def key_positions(S: int, C: int) -> torch.Tensor:
    """Pk(j) = j mod C: key positions repeat with period C.  int64 [S]."""
    j = torch.arange(S, dtype=torch.int64)
    return j % C


def query_positions(S: int, C: int, W: int):
    """The three query-position variants for rows 0..S-1.

    intra : Pq(i) = i mod C               (original in-chunk position)
    succ  : Pq(i) = min(C + i mod C, C + W - 1)
            (true distance to the previous chunk inside the local window,
             the pinned index outside it)
    inter : Pq(i) = C + W - 1             (pinned, the same for every row)

    Returns (pq_intra [S], pq_succ [S], pq_inter int), int64.
    """
    i = torch.arange(S, dtype=torch.int64)
    r = i % C
    p_inter = pinned_query_position(C, W)
    pq_intra = r
    pq_succ = torch.minimum(C + r, torch.full_like(r, p_inter))
    return pq_intra, pq_succ, p_inter


def pair_region(i: torch.Tensor, j: torch.Tensor, C: int) -> torch.Tensor:
    """Region of the pair (i, j), j <= i, from the chunk distance c(i) - c(j):
    0 -> INTRA, 1 -> SUCC, >= 2 -> INTER."""
    delta = torch.div(i, C, rounding_mode="floor") - torch.div(j, C, rounding_mode="floor")
    return torch.clamp(delta, max=2).to(torch.int64)


def relative_positions(S: int, C: int, W: int) -> torch.Tensor:
    """rel(i, j) = Pq_region(i, j)(i) - Pk(j) for every causal pair (j <= i);
    -1 above the diagonal.  int64 [S, S].  Small S only."""
    pq_intra, pq_succ, p_inter = query_positions(S, C, W)
    pk = key_positions(S, C)
    i = torch.arange(S, dtype=torch.int64)[:, None]
    j = torch.arange(S, dtype=torch.int64)[None, :]
    reg = pair_region(i, j, C)
    pq = torch.where(reg == INTRA, pq_intra[:, None],
                     torch.where(reg == SUCC, pq_succ[:, None],
                                 torch.full_like(reg, p_inter)))
    rel = pq - pk[None, :]
    return torch.where(j <= i, rel, torch.full_like(rel, -1))


# ---------------------------------------------------------------------------
# 2. Rotary position embedding, base 1e7  [yudong §3; mizuki §1]
# ---------------------------------------------------------------------------

def rope_inv_freq(d: int, base: float) -> torch.Tensor:
    """theta_m = base^(-2m/d) for m = 0 .. d/2 - 1, float64."""
    m = torch.arange(d // 2, dtype=F64)
    return torch.pow(torch.tensor(float(base), dtype=F64), -2.0 * m / d)


def rope_rotate(x: torch.Tensor, pos: torch.Tensor, base: float) -> torch.Tensor:
    """Rotate the rows of x (shape [..., n, d]) by their positions pos ([n]).

    Half-split pairs (m, m + d/2), angle pos * theta_m:
        y[m]       = x[m] cos - x[m + d/2] sin
        y[m + d/2] = x[m + d/2] cos + x[m] sin
    """
    x = x.to(F64)
    d = x.shape[-1]
    h = d // 2
    ang = pos.to(F64)[:, None] * rope_inv_freq(d, base)[None, :]   # [n, d/2]
    c, s = torch.cos(ang), torch.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)


# ---------------------------------------------------------------------------
# 3. Vertical-slash block-sparse mask  [mizuki, 稀疏注意力 + 核优化]
# ---------------------------------------------------------------------------

def _any_in_interval(sorted_vals: torch.Tensor, lo: torch.Tensor, hi: torch.Tensor) -> torch.Tensor:
    """For each interval [lo, hi], whether some element of sorted_vals lies in it."""
    a = torch.searchsorted(sorted_vals, lo, right=False)
    b = torch.searchsorted(sorted_vals, hi, right=True)
    return b > a


def vs_tile_active(vertical: torch.Tensor, slash: torch.Tensor,
                   t: torch.Tensor, kt: torch.Tensor) -> torch.Tensor:
    """Whether the 64x64 tile (query tile t, key tile kt), kt <= t, is active
    for one head with vertical key columns `vertical` and slash offsets
    `slash` (both sorted ascending).

    Active iff some vertical column lies in [64 kt, 64 kt + 63], or some
    slash offset lies in [max(0, 64 (t - kt) - 63), 64 (t - kt) + 63] -- the
    offsets i - j that occur inside that tile.
    """
    vertical = vertical.to(torch.int64).contiguous()
    slash = slash.to(torch.int64).contiguous()
    t = t.to(torch.int64)
    kt = kt.to(torch.int64)
    v_hit = _any_in_interval(vertical, TILE * kt, TILE * kt + TILE - 1)
    dlt = t - kt
    lo = torch.clamp(TILE * dlt - (TILE - 1), min=0)
    s_hit = _any_in_interval(slash, lo, TILE * dlt + TILE - 1)
    return v_hit | s_hit


def vs_tile_lists(vertical: torch.Tensor, slash: torch.Tensor, S: int):
    """The per-head tile lists that describe the same mask:
    VT = sorted key tiles kt that hold a vertical column,
    D  = sorted tile distances delta in [0, ceil(S/64)) that hold a slash
         offset, i.e. S_h meets [max(0, 64 delta - 63), 64 delta + 63].
    Tile (t, kt), kt <= t, is active iff kt in VT or t - kt in D."""
    n_tiles = (S + TILE - 1) // TILE
    all_t = torch.arange(n_tiles, dtype=torch.int64)
    vertical = vertical.to(torch.int64).contiguous()
    slash = slash.to(torch.int64).contiguous()
    vt = all_t[_any_in_interval(vertical, TILE * all_t, TILE * all_t + TILE - 1)]
    lo = torch.clamp(TILE * all_t - (TILE - 1), min=0)
    dd = all_t[_any_in_interval(slash, lo, TILE * all_t + TILE - 1)]
    return vt, dd


# ---------------------------------------------------------------------------
# 4. Attention  [mizuki, 核心思想 (one softmax per row over the three parts);
#    DCA + YaRN (temperature on the logits); yudong §3 (GQA)]
# ---------------------------------------------------------------------------

def _softmax_rows(logits: torch.Tensor, allowed: torch.Tensor, vv: torch.Tensor):
    """out_i = sum_j softmax(logits_i)_j v_j over allowed j, and
    lse_i = log sum_j exp(logits_ij).  A row with no allowed key gives
    out = 0, lse = -inf."""
    neg_inf = torch.tensor(-math.inf, dtype=F64)
    s = torch.where(allowed, logits, neg_inf)
    m = s.max(dim=1, keepdim=True).values
    m_safe = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
    p = torch.exp(s - m_safe)
    l = p.sum(dim=1, keepdim=True)
    out = (p @ vv) / torch.where(l > 0, l, torch.ones_like(l))
    lse = (m_safe + torch.log(l)).squeeze(1)
    return out, lse


def _check_shapes(q_rows, rows, k, v):
    assert q_rows.dim() == 4 and k.dim() == 4 and v.shape == k.shape
    B, Hq, R, d = q_rows.shape
    assert k.shape[0] == B and k.shape[3] == d and Hq % k.shape[1] == 0
    assert rows.dim() == 1 and rows.numel() == R
    assert int(rows.min()) >= 0 and int(rows.max()) < k.shape[2]


def dca_prefill_rows(q_rows, rows, k, v, C: int, W: int, rope_base: float,
                     yarn_scale: float, softmax_scale: float | None = None,
                     vertical=None, slash=None, query_pos=None,
                     row_block: int = 32):
    """DCA causal GQA prefill attention on selected query rows.

    q_rows : [B, Hq, R, d]  query vectors of the rows listed in `rows`
    rows   : [R] int        their sequence indices
    k, v   : [B, Hkv, S, d] all keys and values
    vertical, slash : optional [Hq, nv], [Hq, ns] sorted int lists (per query
             head) of the vertical-slash mask; None = dense causal.
    query_pos : optional override (pq_intra [S], pq_succ [S], pq_inter) of the
             query-position variants; the tests pass deliberately wrong maps
             through it to measure how far a wrong mapping moves the output.

    Logit of a causal pair (j <= i) in region X = region(i, j):
        s_ij = tau * sigma * < R(Pq_X(i)) q_i , R(Pk(j)) k_j >
    Output: out_i = sum_j softmax_j(s_i.) v_j, lse_i = log sum_j exp(s_ij).
    Returns out [B, Hq, R, d] float64 and lse [B, Hq, R] float64.
    """
    rows = torch.as_tensor(rows, dtype=torch.int64)
    _check_shapes(q_rows, rows, k, v)
    B, Hq, R, d = q_rows.shape
    Hkv, S = k.shape[1], k.shape[2]
    G = Hq // Hkv
    sigma = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    scale = float(yarn_scale) * sigma

    pq_intra, pq_succ, p_inter = query_positions(S, C, W) if query_pos is None else query_pos
    pk = key_positions(S, C)

    n_keys = int(rows.max()) + 1           # keys beyond the last row are never causal
    keys = torch.arange(n_keys, dtype=torch.int64)
    pq_rows = {
        INTRA: pq_intra[rows],
        SUCC: pq_succ[rows],
        INTER: torch.full((R,), int(p_inter), dtype=torch.int64),
    }

    out = torch.zeros((B, Hq, R, d), dtype=F64)
    lse = torch.zeros((B, Hq, R), dtype=F64)
    for b in range(B):
        for kvh in range(Hkv):
            k_rot = rope_rotate(k[b, kvh, :n_keys], pk[:n_keys], rope_base)   # [n_keys, d]
            vv = v[b, kvh, :n_keys].to(F64)
            for h in range(kvh * G, (kvh + 1) * G):
                q_x = {x: rope_rotate(q_rows[b, h], pq_rows[x], rope_base) for x in (INTRA, SUCC, INTER)}
                if vertical is not None:
                    vh = torch.as_tensor(vertical[h], dtype=torch.int64).contiguous()
                    sh = torch.as_tensor(slash[h], dtype=torch.int64).contiguous()
                for r0 in range(0, R, row_block):
                    rr = rows[r0:r0 + row_block]
                    nk = int(rr.max()) + 1          # keys past the block's last row are never causal
                    kk = keys[:nk]
                    reg = pair_region(rr[:, None], kk[None, :], C)
                    dots = {x: q_x[x][r0:r0 + row_block] @ k_rot[:nk].T for x in (INTRA, SUCC, INTER)}
                    logits = scale * torch.where(reg == INTRA, dots[INTRA],
                                                 torch.where(reg == SUCC, dots[SUCC], dots[INTER]))
                    allowed = kk[None, :] <= rr[:, None]
                    if vertical is not None:
                        # tile activity per (row's query tile, key tile), then
                        # spread to the keys of each tile
                        n_kt = (nk + TILE - 1) // TILE
                        tq = torch.div(rr, TILE, rounding_mode="floor")[:, None].expand(-1, n_kt)
                        tk = torch.arange(n_kt, dtype=torch.int64)[None, :].expand(len(rr), -1)
                        act = vs_tile_active(vh, sh, tq.reshape(-1), tk.reshape(-1)).reshape(len(rr), n_kt)
                        allowed = allowed & act[:, torch.div(kk, TILE, rounding_mode="floor")]
                    o, ls = _softmax_rows(logits, allowed, vv[:nk])
                    out[b, h, r0:r0 + row_block] = o
                    lse[b, h, r0:r0 + row_block] = ls
    return out, lse


def vanilla_prefill_rows(q_rows, rows, k, v, rope_base: float, yarn_scale: float = 1.0,
                         softmax_scale: float | None = None, row_block: int = 32):
    """Plain causal GQA attention with RoPE at the true positions (query at i,
    key at j): the attention DCA changes.  Same shapes and returns as
    dca_prefill_rows."""
    rows = torch.as_tensor(rows, dtype=torch.int64)
    _check_shapes(q_rows, rows, k, v)
    B, Hq, R, d = q_rows.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sigma = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    scale = float(yarn_scale) * sigma
    n_keys = int(rows.max()) + 1
    keys = torch.arange(n_keys, dtype=torch.int64)
    out = torch.zeros((B, Hq, R, d), dtype=F64)
    lse = torch.zeros((B, Hq, R), dtype=F64)
    for b in range(B):
        for kvh in range(Hkv):
            k_rot = rope_rotate(k[b, kvh, :n_keys], keys, rope_base)
            vv = v[b, kvh, :n_keys].to(F64)
            for h in range(kvh * G, (kvh + 1) * G):
                q_rot = rope_rotate(q_rows[b, h], rows, rope_base)
                for r0 in range(0, R, row_block):
                    rr = rows[r0:r0 + row_block]
                    nk = int(rr.max()) + 1
                    logits = scale * (q_rot[r0:r0 + row_block] @ k_rot[:nk].T)
                    allowed = keys[None, :nk] <= rr[:, None]
                    o, ls = _softmax_rows(logits, allowed, vv[:nk])
                    out[b, h, r0:r0 + row_block] = o
                    lse[b, h, r0:r0 + row_block] = ls
    return out, lse



# ---------------------------------------------------------------------------
# 5. Online vertical-slash estimation with continuous positions
#    [mizuki, 稀疏注意力 + 核优化: the key-token selection stage restores
#    continuous relative positions; 跟 NSA / 其他稀疏注意力的区别: a few key
#    tokens draw most of the attention in a vertical-slash pattern]
# ---------------------------------------------------------------------------

def vs_scores(q_last, rows, k, rope_base: float, yarn_scale: float = 1.0, softmax_scale: float | None = None):
    """Attention of the last query rows under continuous positions, summed
    into per-head key-column and diagonal scores.

    q_last [Hq, n, d]: the queries of rows `rows` ([n], ascending, the last n
    rows of the sequence); k [Hkv, S, d] with S = rows[-1] + 1. The logits are
    yarn * sigma * <R(i) q_i, R(j) k_j> -- RoPE at the true indices i and j,
    not the DCA map -- causal (j <= i), one softmax per row. Returns
    vertical [Hq, S] with vertical[h, j] = sum_i p_h[i, j], and slash [Hq, S]
    with slash[h, o] = sum_i p_h[i, i - o] (o = i - j >= 0)."""
    rows = torch.as_tensor(rows, dtype=torch.int64)
    Hq, n, d = q_last.shape
    Hkv, S, _ = k.shape
    G = Hq // Hkv
    sigma = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    scale = float(yarn_scale) * sigma
    keys = torch.arange(S, dtype=torch.int64)
    allowed = keys[None, :] <= rows[:, None]                       # [n, S]
    vertical = torch.zeros((Hq, S), dtype=F64)
    slash = torch.zeros((Hq, S), dtype=F64)
    offs = rows[:, None] - keys[None, :]                           # i - j
    for kvh in range(Hkv):
        k_rot = rope_rotate(k[kvh], keys, rope_base)
        for h in range(kvh * G, (kvh + 1) * G):
            q_rot = rope_rotate(q_last[h], rows, rope_base)
            logits = scale * (q_rot @ k_rot.T)
            logits = torch.where(allowed, logits, torch.tensor(-math.inf, dtype=F64))
            p = torch.softmax(logits, dim=-1)                      # rows sum to 1
            vertical[h] = p.sum(dim=0)
            slash[h].index_add_(0, offs[allowed], p[allowed])
    return vertical, slash


def top_with_forced(score, budget: int, forced: int):
    """The indices [0, forced) (clipped to the array) plus the budget - forced
    highest-scoring other indices, ties to the smaller index; ascending.
    Every index is taken when there are fewer candidates than the budget."""
    n = score.shape[0]
    f = min(forced, budget, n)
    head = torch.arange(f, dtype=torch.int64)
    rest = torch.arange(f, n, dtype=torch.int64)
    take = min(budget - f, rest.numel())
    if take <= 0:
        return head
    # stable sort on the negated score: equal scores keep index order
    order = torch.sort(-score[f:].to(F64), stable=True).indices[:take]
    return torch.sort(torch.cat([head, rest[order]])).values


def vs_estimate(q_last, rows, k, rope_base: float, n_vertical: int, n_slash: int, forced: int = 64,
                yarn_scale: float = 1.0, softmax_scale: float | None = None):
    """Per-head vertical columns and slash offsets for the vertical-slash mask:
    the first `forced` columns and offsets always, the rest by score.
    Returns (vertical [Hq, n_vertical'], slash [Hq, n_slash'], vscore, sscore)
    as int64 / float64 tensors (n' = min(n, S))."""
    vscore, sscore = vs_scores(q_last, rows, k, rope_base, yarn_scale, softmax_scale)
    vert = torch.stack([top_with_forced(vscore[h], n_vertical, forced) for h in range(vscore.shape[0])])
    sl = torch.stack([top_with_forced(sscore[h], n_slash, forced) for h in range(sscore.shape[0])])
    return vert, sl, vscore, sscore
