"""Pins of the CPU oracle to facts that do not come from the oracle itself:
hand-worked fixtures, closed forms, reductions to vanilla RoPE attention,
special cases with known outputs and an independent brute force.

The last test plants plausible mistakes in (a copy of) the oracle and checks
that some pin catches each of them.
"""

from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

from oracle import dca_oracle as O
from tests import brute_force as BF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = torch.float64


def _read_fixture(name):
    rows = {}
    pairs = []
    active = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "pair":
                pairs.append((int(parts[1]), int(parts[2]), parts[3], int(parts[4])))
            elif parts[0] == "active":
                active[int(parts[1])] = [int(x) for x in parts[2:]]
            else:
                rows[parts[0]] = [int(x) for x in parts[1:]]
    return rows, pairs, active


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=F64) * scale


# ---------------------------------------------------------------------------
# position map
# ---------------------------------------------------------------------------

def test_positions_match_hand_worked_fixture():
    rows, pairs, _ = _read_fixture("dca_positions_S20_C8_W3.txt")
    S, C, W = 20, 8, 3
    pq_intra, pq_succ, p_inter = O.query_positions(S, C, W)
    assert pq_intra.tolist() == rows["pq_intra"]
    assert pq_succ.tolist() == rows["pq_succ"]
    assert O.key_positions(S, C).tolist() == rows["pk"]
    assert p_inter == rows["pq_inter"][0]
    rel = O.relative_positions(S, C, W)
    names = {"intra": O.INTRA, "succ": O.SUCC, "inter": O.INTER}
    for i, j, reg, r in pairs:
        assert int(O.pair_region(torch.tensor(i), torch.tensor(j), C)) == names[reg], (i, j)
        assert int(rel[i, j]) == r, (i, j)


@pytest.mark.parametrize("S,C,W", [(64, 16, 4), (100, 16, 0), (257, 32, 32), (300, 64, 7),
                                   (512, 128, 128), (200, 8, 1), (96, 96, 5), (130, 64, 64)])
def test_remapped_distance_matches_prose_rule_and_stays_in_window(S, C, W):
    """rel(i, j) agrees with the distance read from the prose (true distance
    inside a chunk and inside the window, the pinned rule elsewhere), lies in
    [0, C + W - 1], and reaches C + W - 1 once S >= C + W."""
    rel = O.relative_positions(S, C, W)
    for i in range(S):
        for j in range(i + 1):
            assert int(rel[i, j]) == BF.dca_distance(i, j, C, W)
    causal = torch.tril(torch.ones(S, S, dtype=torch.bool))
    r = rel[causal]
    assert int(r.min()) >= 0
    assert int(r.max()) <= C + W - 1
    if S >= C + W and W > 0:
        assert int(r.max()) == C + W - 1


@pytest.mark.parametrize("n,C", [(1, 16), (2, 16), (3, 8), (4, 32), (7, 8)])
def test_region_counts_closed_form(n, C):
    S = n * C
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    reg = O.pair_region(i, j, C)
    causal = j <= i
    assert int(((reg == O.INTRA) & causal).sum()) == n * C * (C + 1) // 2
    assert int(((reg == O.SUCC) & causal).sum()) == (n - 1) * C * C
    assert int(((reg == O.INTER) & causal).sum()) == C * C * (n - 1) * (n - 2) // 2


def test_zero_window_makes_succ_equal_inter():
    pq_intra, pq_succ, p_inter = O.query_positions(300, 64, 0)
    assert torch.all(pq_succ == p_inter)
    assert p_inter == 63


def test_positions_identity_when_chunk_covers_sequence():
    S = 50
    pq_intra, _, _ = O.query_positions(S, 64, 8)
    assert pq_intra.tolist() == list(range(S))
    assert O.key_positions(S, 64).tolist() == list(range(S))


# ---------------------------------------------------------------------------
# rotary embedding
# ---------------------------------------------------------------------------

def test_rope_frequencies():
    th = O.rope_inv_freq(128, 1e7)
    assert th[0].item() == 1.0
    ratio = th[1:] / th[:-1]
    assert torch.allclose(ratio, torch.full_like(ratio, 1e7 ** (-2 / 128)), rtol=1e-13)
    assert math.isclose(th[-1].item(), 1e7 ** (-126 / 128), rel_tol=1e-13)


def test_rope_zero_position_is_identity_bit_exact():
    x = _rand((5, 64), 1)
    y = O.rope_rotate(x, torch.zeros(5, dtype=torch.int64), 1e7)
    assert torch.equal(x, y)


def test_rope_matches_complex_multiplication_and_preserves_norm():
    d = 16
    x = _rand((7, d), 2)
    pos = torch.tensor([0, 1, 5, 100, 9999, 294911, 3])
    y = O.rope_rotate(x, pos, 1e7)
    th = BF.theta(d, 1e7)
    for r in range(7):
        for m in range(d // 2):
            p = int(pos[r])
            z = complex(x[r, m], x[r, m + d // 2]) * complex(math.cos(p * th[m]), math.sin(p * th[m]))
            assert math.isclose(y[r, m].item(), z.real, abs_tol=1e-12)
            assert math.isclose(y[r, m + d // 2].item(), z.imag, abs_tol=1e-12)
    assert torch.allclose(y.norm(dim=1), x.norm(dim=1), rtol=1e-13)


def test_rope_relative_identity():
    d = 32
    q = _rand((1, d), 3)
    k = _rand((1, d), 4)
    for a, b in [(10, 3), (294911, 17), (5, 5), (1000, 999)]:
        lhs = (O.rope_rotate(q, torch.tensor([a]), 1e7) * O.rope_rotate(k, torch.tensor([b]), 1e7)).sum()
        rhs = (O.rope_rotate(q, torch.tensor([a - b]), 1e7) * k).sum()
        assert math.isclose(lhs.item(), rhs.item(), rel_tol=1e-9, abs_tol=1e-10)


# ---------------------------------------------------------------------------
# attention: brute force, reductions, special cases
# ---------------------------------------------------------------------------

def _full(q, k, v, C, W, base, tau, **kw):
    S = q.shape[2]
    return O.dca_prefill_rows(q, torch.arange(S), k, v, C, W, base, tau, **kw)


@pytest.mark.parametrize("Hq,Hkv,d,S,C,W,tau", [(2, 1, 8, 40, 8, 3, 1.0),
                                                 (4, 2, 16, 33, 8, 8, 1.1386294361),
                                                 (3, 3, 8, 27, 4, 0, 1.3)])
def test_oracle_matches_pairwise_brute_force(Hq, Hkv, d, S, C, W, tau):
    base = 1e4   # a smaller base makes rotations at these tiny positions large
    q = _rand((1, Hq, S, d), 10)
    k = _rand((1, Hkv, S, d), 11)
    v = _rand((1, Hkv, S, d), 12)
    out, lse = _full(q, k, v, C, W, base, tau)
    bo, bl = BF.attention(q[0].numpy(), k[0].numpy(), v[0].numpy(), C, W, base, tau)
    np.testing.assert_allclose(out[0].numpy(), bo, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse[0].numpy(), bl, rtol=0, atol=1e-11)


def test_sparse_oracle_matches_pairwise_brute_force():
    Hq, Hkv, d, S, C, W, tau, base = 2, 1, 8, 200, 64, 16, 1.2, 1e4
    q = _rand((1, Hq, S, d), 20)
    k = _rand((1, Hkv, S, d), 21)
    v = _rand((1, Hkv, S, d), 22)
    vert = [np.array([3, 150]), np.array([70])]
    slash = [np.array([0, 1, 80]), np.array([0, 130])]

    def active(h, i, j):
        t, kt = i // 64, j // 64
        vh = any(64 * kt <= x <= 64 * kt + 63 for x in vert[h])
        # a slash offset that some (query, key) pair of the full tile has
        sh = any((i2 - j2) in set(slash[h].tolist())
                 for i2 in range(64 * t, 64 * t + 64) for j2 in range(64 * kt, 64 * kt + 64))
        return vh or sh

    cache = {}

    def active_cached(h, i, j):
        key = (h, i // 64, j // 64)
        if key not in cache:
            cache[key] = active(h, i, j)
        return cache[key]

    out, lse = _full(q, k, v, C, W, base, tau,
                     vertical=[torch.tensor(x) for x in vert], slash=[torch.tensor(x) for x in slash])
    bo, bl = BF.attention(q[0].numpy(), k[0].numpy(), v[0].numpy(), C, W, base, tau, active=active_cached)
    np.testing.assert_allclose(out[0].numpy(), bo, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse[0].numpy(), bl, rtol=0, atol=1e-11)


@pytest.mark.parametrize("S,C,W", [(96, 96, 5), (64, 128, 0), (100, 100, 100)])
def test_dca_reduces_to_vanilla_when_chunk_covers_sequence(S, C, W):
    q = _rand((1, 4, S, 32), 30)
    k = _rand((1, 2, S, 32), 31)
    v = _rand((1, 2, S, 32), 32)
    rows = torch.arange(S)
    a, la = O.dca_prefill_rows(q, rows, k, v, C, W, 1e7, 1.0)
    b, lb = O.vanilla_prefill_rows(q, rows, k, v, 1e7, 1.0)
    assert torch.allclose(a, b, rtol=0, atol=1e-12)
    assert torch.allclose(la, lb, rtol=0, atol=1e-12)


def test_intra_chunk_rows_equal_vanilla_for_long_sequences():
    """Rows of the first chunk only see intra-chunk keys: DCA output equals
    plain causal RoPE attention there whatever the sequence length."""
    S, C, W = 300, 64, 8
    q = _rand((1, 2, S, 16), 40)
    k = _rand((1, 1, S, 16), 41)
    v = _rand((1, 1, S, 16), 42)
    rows = torch.arange(C)
    a, _ = O.dca_prefill_rows(q[:, :, :C], rows, k, v, C, W, 1e7, 1.1)
    b, _ = O.vanilla_prefill_rows(q[:, :, :C], rows, k, v, 1e7, 1.1)
    assert torch.allclose(a, b, rtol=0, atol=1e-12)


def test_dca_differs_from_vanilla_beyond_one_chunk():
    S, C, W = 2048, 512, 128
    q = _rand((1, 2, S, 64), 50)
    k = _rand((1, 1, S, 64), 51)
    v = _rand((1, 1, S, 64), 52)
    rows = torch.arange(C, S, 7)
    a, _ = O.dca_prefill_rows(q[:, :, rows], rows, k, v, C, W, 1e7, 1.0)
    b, _ = O.vanilla_prefill_rows(q[:, :, rows], rows, k, v, 1e7, 1.0)
    assert (a - b).abs().max().item() > 1e-2


def test_special_cases():
    S, C, W = 150, 32, 4
    q = _rand((1, 2, S, 16), 60)
    k = _rand((1, 1, S, 16), 61)
    v = _rand((1, 1, S, 16), 62)
    rows = torch.arange(S)
    out, lse = O.dca_prefill_rows(q, rows, k, v, C, W, 1e7, 1.3)
    # row 0 attends only to itself
    assert torch.allclose(out[0, :, 0], v[0, 0, 0].expand(2, -1), rtol=0, atol=1e-14)
    # constant value rows -> the output is that row
    vc = v[:, :, :1].expand(-1, -1, S, -1).contiguous()
    oc, _ = O.dca_prefill_rows(q, rows, k, vc, C, W, 1e7, 1.3)
    assert torch.allclose(oc, vc[:, [0, 0]], rtol=0, atol=1e-13)
    # zero queries -> uniform weights -> running mean of the values
    oz, lz = O.dca_prefill_rows(torch.zeros_like(q), rows, k, v, C, W, 1e7, 1.3)
    mean = torch.cumsum(v[0, 0], 0) / torch.arange(1, S + 1, dtype=F64)[:, None]
    assert torch.allclose(oz[0, 0], mean, rtol=0, atol=1e-13)
    assert torch.allclose(lz[0, 0], torch.log(torch.arange(1, S + 1, dtype=F64)), rtol=0, atol=1e-13)


def test_sampled_rows_equal_full_rows():
    S, C, W = 200, 32, 8
    q = _rand((1, 4, S, 16), 70)
    k = _rand((1, 2, S, 16), 71)
    v = _rand((1, 2, S, 16), 72)
    full, lf = O.dca_prefill_rows(q, torch.arange(S), k, v, C, W, 1e7, 1.1)
    rows = torch.tensor([199, 0, 64, 33, 31])
    part, lp = O.dca_prefill_rows(q[:, :, rows], rows, k, v, C, W, 1e7, 1.1, row_block=2)
    # equal up to the summation order of the library matmul
    assert torch.allclose(part, full[:, :, rows], rtol=0, atol=1e-14)
    assert torch.allclose(lp, lf[:, :, rows], rtol=0, atol=1e-13)


def test_block_rows_depend_only_on_earlier_keys():
    """[mizuki, Chunked Prefill]: a block of rows [q0, q0 + n) prefilled
    against the keys [0, q0 + n) alone gives the rows of the whole-sequence
    result; later keys, whatever they hold, change nothing (causality)."""
    S, C, W = 240, 32, 8
    q = _rand((1, 2, S, 16), 90)
    k = _rand((1, 1, S, 16), 91)
    v = _rand((1, 1, S, 16), 92)
    full, lf = O.dca_prefill_rows(q, torch.arange(S), k, v, C, W, 1e7, 1.2)
    for q0, n in [(0, 64), (64, 96), (160, 80)]:
        rows = torch.arange(q0, q0 + n)
        kp, vp = k[:, :, :q0 + n].clone(), v[:, :, :q0 + n].clone()
        blk, lb = O.dca_prefill_rows(q[:, :, rows], rows, kp, vp, C, W, 1e7, 1.2)
        assert torch.allclose(blk, full[:, :, rows], rtol=0, atol=1e-14)
        assert torch.allclose(lb, lf[:, :, rows], rtol=0, atol=1e-13)
        # the same rows with the later keys replaced by noise
        kn, vn = k.clone(), v.clone()
        kn[:, :, q0 + n:] = _rand(kn[:, :, q0 + n:].shape, 93, 5.0)
        vn[:, :, q0 + n:] = _rand(vn[:, :, q0 + n:].shape, 94, 5.0)
        bn, _ = O.dca_prefill_rows(q[:, :, rows], rows, kn, vn, C, W, 1e7, 1.2)
        assert torch.allclose(bn, full[:, :, rows], rtol=0, atol=1e-14)


def test_planted_needle_dominates_output():
    """Plant a key whose rotated copy is a multiple of the row's rotated query
    in the pair's region: the output of that row is then almost the needle's
    value row."""
    S, C, W, d = 400, 64, 16, 32
    q = _rand((1, 1, S, d), 80, 0.5)
    k = _rand((1, 1, S, d), 81, 0.5)
    v = _rand((1, 1, S, d), 82, 0.5)
    pq_intra, pq_succ, p_inter = O.query_positions(S, C, W)
    for i, j, pos in [(200, 130, pq_succ), (200, 10, None), (200, 195, pq_intra)]:
        kk = k.clone()
        qpos = torch.tensor([p_inter]) if pos is None else pos[i:i + 1]
        rq = O.rope_rotate(q[0, 0, i:i + 1], qpos, 1e7)
        alpha = 40.0 / (rq.norm() ** 2 / math.sqrt(d))
        kk[0, 0, j] = O.rope_rotate(alpha * rq, -O.key_positions(S, C)[j:j + 1], 1e7)[0]
        out, _ = O.dca_prefill_rows(q[:, :, i:i + 1], torch.tensor([i]), kk, v, C, W, 1e7, 1.0)
        assert torch.allclose(out[0, 0, 0], v[0, 0, j], atol=1e-6)


# ---------------------------------------------------------------------------
# vertical-slash mask
# ---------------------------------------------------------------------------

def test_vs_tiles_match_hand_worked_fixture():
    rows, _, active = _read_fixture("vs_tiles_S512.txt")
    S = rows["S"][0]
    vert = torch.tensor(rows["vertical"])
    slash = torch.tensor(rows["slash"])
    vt, dd = O.vs_tile_lists(vert, slash, S)
    assert vt.tolist() == rows["VT"]
    assert dd.tolist() == rows["D"]
    for t, want in active.items():
        kts = torch.arange(t + 1)
        got = O.vs_tile_active(vert, slash, torch.full_like(kts, t), kts)
        assert kts[got].tolist() == want


def test_vs_tile_activity_matches_pair_enumeration():
    rng = np.random.default_rng(5)
    S = 640
    for trial in range(3):
        vert = np.sort(rng.choice(S, 6, replace=False))
        slash = np.sort(rng.choice(S, 5, replace=False))
        vs, ss = set(vert.tolist()), set(slash.tolist())
        n = S // 64
        for t in range(n):
            for kt in range(t + 1):
                brute = any((j in vs) or ((i - j) in ss)
                            for i in range(64 * t, 64 * t + 64) for j in range(64 * kt, 64 * kt + 64))
                got = bool(O.vs_tile_active(torch.tensor(vert), torch.tensor(slash),
                                            torch.tensor([t]), torch.tensor([kt]))[0])
                assert got == brute, (trial, t, kt)
        vt, dd = O.vs_tile_lists(torch.tensor(vert), torch.tensor(slash), S)
        for t in range(n):
            for kt in range(t + 1):
                merged = (kt in vt.tolist()) or ((t - kt) in dd.tolist())
                got = bool(O.vs_tile_active(torch.tensor(vert), torch.tensor(slash),
                                            torch.tensor([t]), torch.tensor([kt]))[0])
                assert merged == got


def test_vs_first_and_recent_only_closed_form():
    """Verticals {0..63} and slashes {0..63}: query tile t sees key tiles
    {0, t - 1, t} exactly."""
    S = 64 * 12
    vert = torch.arange(64)
    slash = torch.arange(64)
    for t in range(12):
        kts = torch.arange(t + 1)
        got = kts[O.vs_tile_active(vert, slash, torch.full_like(kts, t), kts)].tolist()
        assert got == sorted({0, max(t - 1, 0), t})


def test_all_columns_vertical_equals_dense():
    S, C, W = 256, 64, 8
    q = _rand((1, 2, S, 16), 90)
    k = _rand((1, 1, S, 16), 91)
    v = _rand((1, 1, S, 16), 92)
    rows = torch.arange(0, S, 3)
    dense, _ = O.dca_prefill_rows(q[:, :, rows], rows, k, v, C, W, 1e7, 1.1)
    allv = [torch.arange(0, S, 64)] * 2
    sl = [torch.tensor([S - 1])] * 2
    sparse, _ = O.dca_prefill_rows(q[:, :, rows], rows, k, v, C, W, 1e7, 1.1, vertical=allv, slash=sl)
    assert torch.equal(dense, sparse)


# ---------------------------------------------------------------------------
# the pins catch planted mistakes
# ---------------------------------------------------------------------------

def _pins_pass(mod) -> bool:
    """Run a compact set of the pins above against oracle module `mod`."""
    try:
        S, C, W = 20, 8, 3
        rows, pairs, _ = _read_fixture("dca_positions_S20_C8_W3.txt")
        pq_intra, pq_succ, p_inter = mod.query_positions(S, C, W)
        if pq_succ.tolist() != rows["pq_succ"] or p_inter != rows["pq_inter"][0]:
            return False
        rel = mod.relative_positions(S, C, W)
        if any(int(rel[i, j]) != r for i, j, _, r in pairs):
            return False
        Hq, Hkv, d, S, C, W, tau, base = 4, 2, 8, 30, 8, 3, 1.2, 1e4
        q = _rand((1, Hq, S, d), 10)
        k = _rand((1, Hkv, S, d), 11)
        v = _rand((1, Hkv, S, d), 12)
        out, lse = mod.dca_prefill_rows(q, torch.arange(S), k, v, C, W, base, tau)
        bo, bl = BF.attention(q[0].numpy(), k[0].numpy(), v[0].numpy(), C, W, base, tau)
        return bool(np.allclose(out[0].numpy(), bo, atol=1e-9) and np.allclose(lse[0].numpy(), bl, atol=1e-9))
    except Exception:
        return False


MUTATIONS = {
    "rotation sign": ("torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)",
                      "torch.cat([x1 * c + x2 * s, x2 * c - x1 * s], dim=-1)"),
    "interleaved pairs": ("x1, x2 = x[..., :h], x[..., h:]", "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    "pinned index C + W": ("return C + W - 1", "return C + W"),
    "succ window off by one": ("pq_succ = torch.minimum(C + r, torch.full_like(r, p_inter))",
                               "pq_succ = torch.minimum(C + r + 1, torch.full_like(r, p_inter))"),
    "adjacent chunk as inter": ("return torch.clamp(delta, max=2)", "return torch.clamp(2 * delta, max=2)"),
    "key position not periodic": ("return j % C", "return j"),
    "GQA mapping": ("for h in range(kvh * G, (kvh + 1) * G):\n                q_x",
                    "for h in range(kvh, Hq, Hkv):\n                q_x"),
    "YaRN dropped": ("scale = float(yarn_scale) * sigma\n\n    pq_intra",
                     "scale = sigma\n\n    pq_intra"),
    "causal mask off by one": ("allowed = kk[None, :] <= rr[:, None]", "allowed = kk[None, :] < rr[:, None] + 0 * kk[None, :] + (rr[:, None] == 0)"),
    "lse missing max": ("lse = (m_safe + torch.log(l)).squeeze(1)", "lse = torch.log(l).squeeze(1)"),
    "frequency exponent": ("-2.0 * m / d)", "-1.0 * m / d)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    import importlib.util

    src = open(O.__file__).read()
    old, new = MUTATIONS[name]
    assert old in src, name
    path = tmp_path / "mutant_oracle.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("mutant_oracle", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert _pins_pass(O)
    assert not _pins_pass(mod), f"planted mistake '{name}' not caught"


def _mask_and_estimate_pins_pass(mod) -> bool:
    """A compact set of the mask and estimate pins run against oracle module
    `mod`: the hand-worked tile fixture, tile activity against pair
    enumeration (with offsets on tile-distance edges), the estimate's scores
    against the pairwise brute force, and the selection rule on ties."""
    try:
        rows, _, active = _read_fixture("vs_tiles_S512.txt")
        S = rows["S"][0]
        vert, slash = torch.tensor(rows["vertical"]), torch.tensor(rows["slash"])
        vt, dd = mod.vs_tile_lists(vert, slash, S)
        if vt.tolist() != rows["VT"] or dd.tolist() != rows["D"]:
            return False
        for t, want in active.items():
            kts = torch.arange(t + 1)
            if kts[mod.vs_tile_active(vert, slash, torch.full_like(kts, t), kts)].tolist() != want:
                return False
        # columns and offsets on the edges of tiles and tile distances
        for vv, ss in (([63, 64], [1]), ([], [64]), ([], [63, 127]), ([128], [0])):
            vs_, ss_ = set(vv), set(ss)
            for t in range(4):
                for kt in range(t + 1):
                    brute = any((j in vs_) or ((i - j) in ss_)
                                for i in range(64 * t, 64 * t + 64) for j in range(64 * kt, 64 * kt + 64))
                    got = bool(mod.vs_tile_active(torch.tensor(vv, dtype=torch.int64), torch.tensor(ss),
                                                  torch.tensor([t]), torch.tensor([kt]))[0])
                    if got != brute:
                        return False
        Hq, Hkv, S, d, n = 4, 2, 90, 8, 12
        q = _rand((Hq, n, d), 100)
        k = _rand((Hkv, S, d), 101)
        r = torch.arange(S - n, S)
        vs, ss = mod.vs_scores(q, r, k, 1e4, 1.3)
        bv, bs = BF.vs_scores(q.numpy(), r.tolist(), k.numpy(), 1e4, 1.3)
        if not (np.allclose(vs.numpy(), bv, rtol=0, atol=1e-12) and np.allclose(ss.numpy(), bs, rtol=0, atol=1e-12)):
            return False
        score = torch.tensor([9.0, 1.0, 5.0, 5.0, 0.5, 5.0, 7.0], dtype=torch.float64)
        return (mod.top_with_forced(score, 4, 2).tolist() == [0, 1, 2, 6]
                and mod.top_with_forced(score, 3, 0).tolist() == [0, 2, 6])
    except Exception:
        return False


MASK_MUTATIONS = {
    "slash interval starts one low": ("lo = torch.clamp(TILE * dlt - (TILE - 1), min=0)",
                                      "lo = torch.clamp(TILE * dlt - TILE, min=0)"),
    "vertical interval ends one high": ("v_hit = _any_in_interval(vertical, TILE * kt, TILE * kt + TILE - 1)",
                                        "v_hit = _any_in_interval(vertical, TILE * kt, TILE * kt + TILE)"),
    "estimate sees one key past the row": ("allowed = keys[None, :] <= rows[:, None]   ",
                                           "allowed = keys[None, :] <= rows[:, None] + 1"),
    "estimate diagonal index off by one": ("offs = rows[:, None] - keys[None, :]   ",
                                           "offs = rows[:, None] - keys[None, :] + 1"),
    "estimate logit scale dropped": ("logits = scale * (q_rot @ k_rot.T)", "logits = (q_rot @ k_rot.T)"),
    "forced head dropped": ("f = min(forced, budget, n)", "f = 0"),
    "ties to the larger index": ("order = torch.sort(-score[f:].to(F64), stable=True).indices[:take]",
                                 "order = (rest.numel() - 1 - torch.sort(-score[f:].to(F64).flip(0), "
                                 "stable=True).indices)[:take]"),
}


@pytest.mark.parametrize("name", sorted(MASK_MUTATIONS))
def test_mask_and_estimate_pins_catch_planted_mistake(name, tmp_path):
    import importlib.util

    src = open(O.__file__).read()
    old, new = MASK_MUTATIONS[name]
    assert src.count(old) == 1, name
    path = tmp_path / "mutant_oracle.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("mutant_oracle", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert _mask_and_estimate_pins_pass(O)
    assert not _mask_and_estimate_pins_pass(mod), f"planted mistake '{name}' not caught"


# ---------------------------------------------------------------------------
# online vertical-slash estimation (continuous positions)
# ---------------------------------------------------------------------------

def test_vs_scores_match_pairwise_brute_force():
    Hq, Hkv, S, d, n = 4, 2, 90, 8, 12
    q = _rand((Hq, n, d), 100)
    k = _rand((Hkv, S, d), 101)
    rows = torch.arange(S - n, S)
    vs, ss = O.vs_scores(q, rows, k, 1e4, 1.3)
    bv, bs = BF.vs_scores(q.numpy(), rows.tolist(), k.numpy(), 1e4, 1.3)
    assert np.allclose(vs.numpy(), bv, rtol=0, atol=1e-12)
    assert np.allclose(ss.numpy(), bs, rtol=0, atol=1e-12)
    # every row's softmax sums to one
    assert torch.allclose(vs.sum(1), torch.full((Hq,), float(n), dtype=F64), rtol=0, atol=1e-12)
    assert torch.allclose(ss.sum(1), torch.full((Hq,), float(n), dtype=F64), rtol=0, atol=1e-12)


def test_vs_scores_use_continuous_positions():
    """The selection attention is vanilla RoPE attention: its per-row weights
    reproduce the vanilla oracle's output, and differ from DCA's beyond one
    chunk."""
    Hq, Hkv, S, d, n = 2, 1, 160, 16, 4
    q = _rand((1, Hq, S, d), 102)
    k = _rand((1, Hkv, S, d), 103)
    v = _rand((1, Hkv, S, d), 104)
    rows = torch.arange(S - n, S)

    def weights(run):
        # V = a block of one-hot rows: the outputs are the attention weights
        # of that block of keys
        w = []
        for c in range(S // d):
            v = torch.zeros((1, Hkv, S, d), dtype=F64)
            v[0, 0, c * d:(c + 1) * d] = torch.eye(d, dtype=F64)
            w.append(run(v)[0])
        return torch.cat(w, dim=-1)                                    # [Hq, n, S]

    van = weights(lambda v: O.vanilla_prefill_rows(q[:, :, rows], rows, k, v, 1e4, 1.1)[0])
    vs, _ = O.vs_scores(q[0, :, rows], rows, k[0], 1e4, 1.1)
    assert torch.allclose(vs, van.sum(1), rtol=0, atol=1e-12)
    dca = weights(lambda v: O.dca_prefill_rows(q[:, :, rows], rows, k, v, 32, 8, 1e4, 1.1)[0])
    assert (dca.sum(1) - vs).abs().max() > 1e-3


def test_vs_estimate_finds_planted_column_and_diagonal():
    """Energy only in the slowest RoPE pair (angle below 1e-3 rad over the
    sequence): a key 10x the query wins every row (a vertical), and keys 10x
    the query at one fixed distance o* win along a diagonal (a slash)."""
    S, d, n = 200, 16, 16
    base = 1e7
    rows = torch.arange(S - n, S)
    unit = torch.zeros(d, dtype=F64)
    unit[d // 2 - 1] = 0.3
    q = unit.repeat(2, n, 1)
    k = _rand((1, S, d), 105, 0.01)
    k[0, 37] = 10 * unit
    o_star = 77
    for i in rows.tolist():
        k[0, i - o_star] = 6 * unit
    vert, sl, vs, ss = O.vs_estimate(q, rows, k, base, n_vertical=2, n_slash=2, forced=1)
    assert vert[0].tolist() == [0, 37]
    assert sl[0].tolist() == [0, o_star]


def test_top_with_forced_ties_and_small_inputs():
    score = torch.tensor([9.0, 1.0, 5.0, 5.0, 0.5, 5.0, 7.0], dtype=F64)
    assert O.top_with_forced(score, 4, 2).tolist() == [0, 1, 2, 6]       # 7.0 then 5.0 at the smallest index
    assert O.top_with_forced(score, 5, 2).tolist() == [0, 1, 2, 3, 6]
    assert O.top_with_forced(score, 10, 2).tolist() == list(range(7))     # fewer candidates than the budget
    assert O.top_with_forced(score, 3, 0).tolist() == [0, 2, 6]
    assert O.top_with_forced(score, 1, 3).tolist() == [0]                 # forced clipped to the budget
