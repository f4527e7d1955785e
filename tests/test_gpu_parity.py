"""GPU parity of libdca against the CPU oracle (MI355X).

Every case prints what it runs before touching the GPU. Outputs are compared
element by element with the float64 oracle on the same seeded inputs:
max-abs <= 1e-4 for fp32 and <= 2e-2 for bf16, plus, for bf16, a
discrimination guard (the error must be far below how much a wrong position
mapping would move the output) and planted needles. Position maps, tile
regions and vertical-slash tile lists are compared bit-exactly.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

from oracle import dca_oracle as O
from position_extrapolation_amd import api, synth, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()
    yield
    torch.cuda.synchronize()
    _ONE_M.clear()
    torch.cuda.empty_cache()


def _wl(name, **over):
    w = workloads.get(name)
    return workloads.Workload(**{**w.__dict__, **over})


def _run(q, k, v, w, vertical=None, slash=None, lse=True):
    out, l = api.prefill(q, k, v, w.chunk, w.window, w.rope_base, w.yarn_scale, vertical=vertical,
                         slash=slash, return_lse=True)
    torch.cuda.synchronize()
    return out, l


def _oracle(q, k, v, rows, w, vertical=None, slash=None, query_pos=None):
    rows_t = torch.as_tensor(rows, dtype=torch.int64)
    q_rows = q[:, :, rows_t.to(q.device)].cpu()
    return O.dca_prefill_rows(q_rows, rows_t, k.cpu(), v.cpu(), w.chunk, w.window, w.rope_base,
                              w.yarn_scale, vertical=vertical, slash=slash, query_pos=query_pos)


def _err(gpu_rows, ref):
    return (gpu_rows.double().cpu() - ref).abs().max().item()


def _within_rounding(gpu_rows, ref, v, rows, G):
    """bf16 rounding model, element by element: the output's own rounding,
    plus one bf16 rounding of every weight P (2^-9 relative) times the spread
    of the values the row averages (max over keys j <= i of |v_j - out|),
    doubled for the bf16 rounding of the rotated queries and keys:
    |gpu - ref| <= 2^-8 (|ref| + spread). A fixed absolute term does not
    bound the weight rounding: on rows with few keys the spread reaches 1.4."""
    rows_c = torch.as_tensor(rows, dtype=torch.int64)
    heads = torch.arange(ref.shape[1]) // G
    vv = v.double().cpu()
    hi = torch.cummax(vv, dim=2).values[:, heads][:, :, rows_c]
    lo = torch.cummin(vv, dim=2).values[:, heads][:, :, rows_c]
    spread = torch.maximum(hi - ref, ref - lo)
    return bool(((gpu_rows.double().cpu() - ref).abs() <= (ref.abs() + spread) * 2.0 ** -8 + 1e-6).all())


# ---------------------------------------------------------------------------
# integer stages: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S,C,W", [(2048, 512, 128), (1000, 64, 0), (131072, 32768, 4096),
                                   (1048576, 262144, 32768), (777, 128, 128)])
def test_device_positions_bit_exact(S, C, W):
    say(f"[positions] S={S} C={C} W={W}")
    pqi = torch.empty(S, dtype=torch.int32, device=DEV)
    pqs = torch.empty_like(pqi)
    pk = torch.empty_like(pqi)
    pin = torch.empty(1, dtype=torch.int32, device=DEV)
    api.dca_debug_positions(S, C, W, pqi, pqs, pin, pk)
    torch.cuda.synchronize()
    oi, os_, op = O.query_positions(S, C, W)
    assert torch.equal(pqi.cpu().long(), oi)
    assert torch.equal(pqs.cpu().long(), os_)
    assert int(pin.item()) == op
    assert torch.equal(pk.cpu().long(), O.key_positions(S, C))


@pytest.mark.parametrize("S,C", [(2048, 512), (1000, 64), (4096, 1024), (777, 128)])
def test_device_tile_regions_bit_exact(S, C):
    say(f"[tile regions] S={S} C={C}")
    n = (S + 63) // 64
    out = torch.empty(n * n, dtype=torch.uint8, device=DEV)
    api.dca_debug_tile_regions(S, C, out)
    torch.cuda.synchronize()
    t = torch.arange(n)[:, None].expand(n, n)
    kt = torch.arange(n)[None, :].expand(n, n)
    # every pair of a tile has the region of the tile's first pair
    ref = O.pair_region(64 * t, 64 * kt, C)
    for di, dj in [(63, 0), (0, 63), (63, 63)]:
        ii = torch.clamp(64 * t + di, max=S - 1)
        jj = torch.clamp(64 * kt + dj, max=S - 1)
        other = O.pair_region(ii, jj, C)
        assert torch.equal(other[kt < t], ref[kt < t])
    ref = torch.where(kt > t, torch.full_like(ref, 255), ref)
    assert torch.equal(out.cpu().long().view(n, n), ref)


# ---------------------------------------------------------------------------
# remap pre-pass values
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D,S,C,W", [("bf16", 128, 1000, 256, 64), ("f32", 64, 2048, 512, 128),
                                           ("bf16", 64, 300, 64, 64), ("f32", 128, 513, 128, 0)])
def test_remap_prepass_matches_oracle_rotation(dtype, D, S, C, W):
    say(f"[remap] dtype={dtype} D={D} S={S} C={C} W={W}")
    w = workloads.Workload("t", 1, 4, 2, D, S, C, W, dtype, 0.5 if dtype == "bf16" else 1.0, True)
    q, k, v = synth.make_qkv(w, seed=3, device=DEV)
    shape = api.shape_of(q, k)
    nbytes = api.dca_workspace_size(S, C, W, shape)
    ws = api.alloc_workspace(nbytes, DEV)
    api.dca_remap(q, k, v, S, C, W, w.rope_base, w.yarn_scale, shape, ws, nbytes)
    outs = []
    for which in range(5):
        dst = torch.empty_like(q if which < 3 else k)
        api.dca_debug_unpack(ws, nbytes, which, S, C, W, shape, dst)
        outs.append(dst)
    torch.cuda.synchronize()
    pqi, pqs, pin = O.query_positions(S, C, W)
    ref_q = [O.rope_rotate(q.cpu(), pqi, w.rope_base), O.rope_rotate(q.cpu(), pqs, w.rope_base),
             O.rope_rotate(q.cpu(), torch.full((S,), pin), w.rope_base)]
    # the pre-pass scales the rotated keys by yarn * sigma * log2(e)
    ks = w.yarn_scale / math.sqrt(D) * math.log2(math.e)
    ref_k = O.rope_rotate(k.cpu(), O.key_positions(S, C), w.rope_base) * ks
    for got, ref in zip(outs[:3] + [outs[3]], ref_q + [ref_k]):
        g = got.double().cpu()
        if dtype == "bf16":
            # one bf16 rounding of a float32 result: relative 2^-8 plus fp32 slack
            assert ((g - ref).abs() <= ref.abs() * 2.0 ** -8 + 1e-5).all()
        else:
            assert (g - ref).abs().max().item() <= 1e-5
    assert torch.equal(outs[4], v)


# ---------------------------------------------------------------------------
# attention parity
# ---------------------------------------------------------------------------

def test_parity_tiny_f32_all_rows():
    w = workloads.get("tiny_2k_f32")
    say(f"[parity] {w.name} all rows")
    q, k, v = synth.make_qkv(w, seed=0, device=DEV)
    out, lse = _run(q, k, v, w)
    rows = np.arange(w.seq)
    ref, ref_lse = _oracle(q, k, v, rows, w)
    err = _err(out, ref)
    lerr = _err(lse, ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL["f32"]
    assert lerr <= TOL["f32"]
    van, _ = O.vanilla_prefill_rows(q.cpu(), torch.arange(w.seq), k.cpu(), v.cpu(), w.rope_base, 1.0)
    assert (van - ref).abs().max().item() > 100 * err


@pytest.mark.parametrize("dtype,Hq,Hkv,D,S,C,W", [
    ("bf16", 4, 2, 128, 1000, 256, 64),     # ragged tail, 4 chunks
    ("bf16", 3, 1, 64, 777, 128, 128),      # W = C, d = 64, G = 3
    ("bf16", 2, 2, 128, 640, 64, 0),        # W = 0, C = 64, no GQA
    ("f32", 4, 1, 128, 515, 128, 32),       # fp32, d = 128
    ("f32", 2, 1, 64, 65, 64, 16),          # one row past a chunk
    ("bf16", 2, 1, 128, 1, 64, 8),          # a single row
    ("bf16", 2, 1, 128, 4096, 4096, 100),   # C = S: plain causal RoPE
])
def test_parity_small_all_rows(dtype, Hq, Hkv, D, S, C, W):
    say(f"[parity] dtype={dtype} Hq={Hq} Hkv={Hkv} D={D} S={S} C={C} W={W}")
    w = workloads.Workload("t", 1, Hq, Hkv, D, S, C, W, dtype, 0.5 if dtype == "bf16" else 1.0, True)
    q, k, v = synth.make_qkv(w, seed=11, device=DEV)
    out, lse = _run(q, k, v, w)
    ref, ref_lse = _oracle(q, k, v, np.arange(S), w)
    err, lerr = _err(out, ref), _err(lse, ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL[dtype]
    assert lerr <= (1e-4 if dtype == "f32" else 2e-2)
    if dtype == "bf16":
        # far tighter than the tolerance: the bf16 rounding model
        assert _within_rounding(out, ref, v, np.arange(S), Hq // Hkv)


@pytest.mark.parametrize("S", [64, 130, 192, 300, 320, 383])
def test_parity_every_key_tile_count(S):
    """One to six key tiles per workgroup (ragged or not), with C = 64 so that
    every key tile is its own chunk and the region changes at every tile. The
    two-tile loop's second half of the waves defers the PV of a step's second
    tile past the next barrier: this covers steps with one tile, a deferred
    tile at the end, and waves whose last active tile opens a step. Oracle
    parity on every row, and the fused path bit-identical."""
    say(f"[parity] key tiles per workgroup: S={S} C=64 W=16")
    w = workloads.Workload("t", 1, 2, 1, 128, S, 64, 16, "bf16", 0.5, True)
    q, k, v = synth.make_qkv(w, seed=S, device=DEV)
    out, lse = _run(q, k, v, w)
    ref, ref_lse = _oracle(q, k, v, np.arange(S), w)
    err, lerr = _err(out, ref), _err(lse, ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= 2e-2
    fout, flse = api.prefill(q, k, v, 64, 16, w.rope_base, w.yarn_scale, return_lse=True, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(fout, out) and torch.equal(flse, lse)


@pytest.mark.parametrize("Hq,Hkv", [(32, 1), (40, 1)])
def test_parity_one_kv_head_for_many_query_heads(Hq, Hkv):
    """Group sizes past the decode kernel's 32 columns: the prefill's work
    decode spreads the query heads of one KV head over XCD streams; every
    head's rows must match the oracle."""
    say(f"[parity] Hq={Hq} Hkv={Hkv} (G={Hq // Hkv})")
    w = workloads.Workload("t", 1, Hq, Hkv, 128, 1300, 512, 64, "bf16", 0.5, True)
    q, k, v = synth.make_qkv(w, seed=Hq, device=DEV)
    out, lse = _run(q, k, v, w)
    rows = synth.sample_rows(w.seq, w.chunk, w.window, 96, seed=2)
    ref, ref_lse = _oracle(q, k, v, rows, w)
    rows_t = torch.as_tensor(rows, device=DEV)
    err, lerr = _err(out[:, :, rows_t], ref), _err(lse[:, :, rows_t], ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= 2e-2


def _discrimination(q, k, v, rows, w, ref, gpu_rows):
    """The GPU error must sit far below how far two wrong position mappings
    move the output: vanilla RoPE, and successive-chunk pairs treated as
    inter-chunk. Measured on the rows past the first chunk -- the only rows
    DCA changes -- where outputs are small and the bf16 output rounding does
    not mask a wrong mapping."""
    far = torch.as_tensor(rows >= w.chunk)
    pqi, pqs, pin = O.query_positions(w.seq, w.chunk, w.window)
    wrong_succ, _ = _oracle(q, k, v, rows, w, query_pos=(pqi, torch.full_like(pqs, pin), pin))
    rows_t = torch.as_tensor(rows)
    van, _ = O.vanilla_prefill_rows(q[:, :, rows_t.to(q.device)].cpu(), rows_t, k.cpu(), v.cpu(),
                                    w.rope_base, w.yarn_scale)
    d1 = (van - ref)[:, :, far].abs().max().item()
    d2 = (wrong_succ - ref)[:, :, far].abs().max().item()
    err = (gpu_rows.double().cpu() - ref)[:, :, far].abs().max().item()
    say(f"  rows >= C: wrong-mapping distances vanilla={d1:.3e} succ-as-inter={d2:.3e}; gpu err={err:.3e}")
    assert err <= 0.1 * min(d1, d2)


@pytest.mark.parametrize("name", ["qwen7b_32k", "qwen7b_128k"])
def test_parity_sampled_rows(name):
    w = workloads.get(name)
    rows = synth.sample_rows(w.seq, w.chunk, w.window, w.oracle_rows, seed=0)
    say(f"[parity] {name}: {len(rows)} sampled rows x {w.n_q_heads} heads")
    q, k, v = synth.make_qkv(w, seed=0, device=DEV)
    out, lse = _run(q, k, v, w)
    ref, ref_lse = _oracle(q, k, v, rows, w)
    rows_t = torch.as_tensor(rows, device=DEV)
    err = _err(out[:, :, rows_t], ref)
    lerr = _err(lse[:, :, rows_t], ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= 2e-2
    _discrimination(q, k, v, rows, w, ref, out[:, :, rows_t])


# ---------------------------------------------------------------------------
# the 1M-token Qwen2.5-14B shape (dense and vertical-slash), one seeded input
# ---------------------------------------------------------------------------

_ONE_M = {}


def _one_m():
    """The 1M-token Qwen2.5-14B workload at seed 0, shared by the 1M tests:
    q, k, v on the device, k and v on the host, the 256 sampled rows (the
    forced boundary rows plus seeded ones) and their queries on the host.
    The dense and vertical-slash workloads draw the same q, k, v."""
    if not _ONE_M:
        w = workloads.get("qwen14b_1m")
        q, k, v = synth.make_qkv(w, seed=0, device=DEV)
        rows = synth.sample_rows(w.seq, w.chunk, w.window, w.oracle_rows, seed=0)
        _ONE_M.update(w=w, q=q, k=k, v=v, rows=rows, q_rows=q[:, :, torch.as_tensor(rows, device=DEV)].cpu(),
                      kc=k.cpu(), vc=v.cpu())
    return _ONE_M


def _guard_subset(rows, C, n=48):
    """Indices (into rows) of the rows the wrong-mapping guard re-runs the
    oracle on: rows past the first chunk -- the only rows DCA changes --
    every forced chunk and window boundary there plus evenly spread others,
    n in all, so that the guard's extra oracle passes stay bounded."""
    far = np.nonzero(rows >= C)[0]
    pick = set(far[np.linspace(0, len(far) - 1, n).round().astype(int)].tolist())
    boundary = {C, C + 1, 2 * C - 1, 2 * C, 3 * C, int(rows[-1])}
    pick |= {int(i) for i in far if int(rows[i]) in boundary}
    return np.array(sorted(pick), dtype=np.int64)


def _group_args(m, w, g, idx):
    """Host tensors of KV group g: its query heads' sampled rows idx, its keys
    and values (the oracle's definition restricted to one KV group)."""
    G = w.n_q_heads // w.n_kv_heads
    hs = slice(g * G, (g + 1) * G)
    return hs, m["q_rows"][:, hs][:, :, torch.as_tensor(idx)], m["kc"][:, g:g + 1], m["vc"][:, g:g + 1]


def _oracle_group_rows(m, w, g, idx, **kw):
    hs, qg, kg, vg = _group_args(m, w, g, idx)
    if kw.get("vertical") is not None:
        kw = {**kw, "vertical": kw["vertical"][hs], "slash": kw["slash"][hs]}
    return O.dca_prefill_rows(qg, torch.as_tensor(m["rows"][idx]), kg, vg, w.chunk, w.window, w.rope_base,
                              w.yarn_scale, **kw)


def test_prefill_1m_dense():
    """The 1M-token Qwen2.5-14B prefill in the launch configuration the
    benchmark times; its 256 sampled rows (forced boundary rows plus seeded
    ones) are kept for the per-group oracle checks that follow."""
    m = _one_m()
    w = m["w"]
    say(f"[parity 1M] prefill S={w.seq}; {len(m['rows'])} sampled rows x {w.n_q_heads} heads kept")
    out, lse = _run(m["q"], m["k"], m["v"], w)
    rows_d = torch.as_tensor(m["rows"], device=DEV)
    m["dense_out"], m["dense_lse"] = out[:, :, rows_d].double().cpu(), lse[:, :, rows_d].double().cpu()
    del out, lse
    torch.cuda.empty_cache()
    assert torch.isfinite(m["dense_out"]).all()


@pytest.mark.parametrize("g", range(8))
def test_parity_1m_dense_group(g):
    """One KV group (5 query heads) of the 1M prefill against the oracle on
    the 256 sampled rows: out and lse within the bf16 bound. Then the
    discrimination guard on the rows past the first chunk, the only rows DCA
    changes: the GPU error there must stay below a tenth of how far two wrong
    position mappings (vanilla RoPE, and successive-chunk pairs treated as
    inter-chunk) move the oracle's output, those distances measured on 48 or
    more of those rows including every chunk boundary among them."""
    m = _one_m()
    if "dense_out" not in m:
        pytest.skip("needs test_prefill_1m_dense")
    w, rows = m["w"], m["rows"]
    G = w.n_q_heads // w.n_kv_heads
    hs = slice(g * G, (g + 1) * G)
    say(f"[parity 1M] KV group {g}: oracle on {len(rows)} rows x {G} heads")
    ref, ref_lse = _oracle_group_rows(m, w, g, np.arange(len(rows)))
    m.setdefault("dense_ref", {})[g] = ref
    got, got_lse = m["dense_out"][:, hs], m["dense_lse"][:, hs]
    err, lerr = (got - ref).abs().max().item(), (got_lse - ref_lse).abs().max().item()
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= 2e-2
    far = torch.as_tensor(rows >= w.chunk)
    err_far = (got - ref)[:, :, far].abs().max().item()
    gi = _guard_subset(rows, w.chunk)
    pqi, pqs, pin = O.query_positions(w.seq, w.chunk, w.window)
    wrong_succ, _ = _oracle_group_rows(m, w, g, gi, query_pos=(pqi, torch.full_like(pqs, pin), pin))
    _, qg, kg, vg = _group_args(m, w, g, gi)
    van, _ = O.vanilla_prefill_rows(qg, torch.as_tensor(rows[gi]), kg, vg, w.rope_base, w.yarn_scale)
    ref_g = ref[:, :, torch.as_tensor(gi)]
    d1, d2 = (van - ref_g).abs().max().item(), (wrong_succ - ref_g).abs().max().item()
    say(f"  rows >= C ({int(far.sum())}): gpu err={err_far:.3e}; wrong-mapping distances on {len(gi)} of them: "
        f"vanilla={d1:.3e} succ-as-inter={d2:.3e}; guard ratio err/min={err_far / min(d1, d2):.4f} (bound 0.1)")
    assert err_far <= 0.1 * min(d1, d2)


def test_fused_and_chunked_equal_whole_at_1m():
    """At the 1M-token Qwen2.5-14B shape, in the launch configurations the
    benchmark times: the fused-rotation path and the chunked path (32 blocks
    of 32,768 rows) give the whole-sequence prefill's output and lse bit for
    bit (whose rows the oracle checks in the test above)."""
    m = _one_m()
    w, q, k, v = m["w"], m["q"], m["k"], m["v"]
    say(f"[1M] fused and chunked against the whole prefill, S={w.seq}")
    out, lse = _run(q, k, v, w)
    fout, flse = api.prefill(q, k, v, w.chunk, w.window, w.rope_base, w.yarn_scale, return_lse=True, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(fout, out) and torch.equal(flse, lse)
    del fout, flse
    torch.cuda.empty_cache()
    cout, clse = api.prefill_chunked(q, k, v, w.chunk, w.window, 32768, w.rope_base, w.yarn_scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(cout, out) and torch.equal(clse, lse)
    say("  fused and chunked outputs and lse identical to the whole prefill")


def test_parity_4m_tokens():
    """A 4M-token sequence (2^22; one KV head, d = 64, C = 1M, W = 128K):
    row, tile and byte offsets four times past the benchmark's largest shape.
    The oracle on the forced boundary rows plus seeded rows, and the
    wrong-mapping guard."""
    w = workloads.Workload("t", 1, 2, 1, 64, 1 << 22, 1 << 20, 1 << 17, "bf16", 0.5, True)
    rows = synth.sample_rows(w.seq, w.chunk, w.window, 12, seed=4)
    say(f"[parity 4M] S={w.seq} C={w.chunk} W={w.window}: {len(rows)} sampled rows x {w.n_q_heads} heads")
    q, k, v = synth.make_qkv(w, seed=6, device=DEV)
    out, lse = _run(q, k, v, w)
    rows_t = torch.as_tensor(rows, device=DEV)
    out_rows, lse_rows = out[:, :, rows_t].clone(), lse[:, :, rows_t].clone()
    del out, lse
    ref, ref_lse = _oracle(q, k, v, rows, w)
    err, lerr = _err(out_rows, ref), _err(lse_rows, ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= 2e-2
    _discrimination(q, k, v, rows, w, ref, out_rows)


def test_prefill_1m_vertical_slash():
    """The 1M vertical-slash workload (1000 columns, 2000 offsets per head,
    the dense workload's seed-0 inputs); its 256 sampled rows are kept for
    the per-group checks that follow."""
    m = _one_m()
    w = workloads.get("qwen14b_1m_vs")
    vert, slash = _vs_case(w, seed=0)
    m["vert"], m["slash"] = vert, slash
    say(f"[vs parity 1M] prefill S={w.seq}, {w.n_vertical} columns and {w.n_slash} offsets per head")
    out, lse = _run(m["q"], m["k"], m["v"], w, vertical=vert.to(DEV), slash=slash.to(DEV))
    rows_d = torch.as_tensor(m["rows"], device=DEV)
    m["vs_out"], m["vs_lse"] = out[:, :, rows_d].double().cpu(), lse[:, :, rows_d].double().cpu()
    del out, lse
    torch.cuda.empty_cache()
    assert torch.isfinite(m["vs_out"]).all()


@pytest.mark.parametrize("g", range(8))
def test_vs_parity_1m_group(g):
    """One KV group of the 1M vertical-slash prefill against the oracle on
    the 256 sampled rows: out and lse within the bf16 bound, and two guards
    on the rows past the first chunk, where outputs are small: the GPU error
    must stay below a tenth of (a) the distance between the oracle's dense
    and sparse outputs (a mask-ignoring or all-zero output fails it) and (b)
    how far treating successive-chunk pairs as inter-chunk moves the sparse
    output (on 48 or more of those rows)."""
    m = _one_m()
    if "vs_out" not in m:
        pytest.skip("needs test_prefill_1m_vertical_slash")
    w = workloads.get("qwen14b_1m_vs")
    rows, vert, slash = m["rows"], m["vert"], m["slash"]
    G = w.n_q_heads // w.n_kv_heads
    hs = slice(g * G, (g + 1) * G)
    say(f"[vs parity 1M] KV group {g}: oracle on {len(rows)} rows x {G} heads")
    ref, ref_lse = _oracle_group_rows(m, w, g, np.arange(len(rows)), vertical=vert, slash=slash)
    got, got_lse = m["vs_out"][:, hs], m["vs_lse"][:, hs]
    err, lerr = (got - ref).abs().max().item(), (got_lse - ref_lse).abs().max().item()
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= 2e-2
    dense = m.get("dense_ref", {}).get(g)
    if dense is None:
        dense, _ = _oracle_group_rows(m, w, g, np.arange(len(rows)))
    far = torch.as_tensor(rows >= w.chunk)
    err_far = (got - ref)[:, :, far].abs().max().item()
    dd = (dense - ref)[:, :, far].abs().max().item()
    gi = _guard_subset(rows, w.chunk)
    pqi, pqs, pin = O.query_positions(w.seq, w.chunk, w.window)
    wrong_succ, _ = _oracle_group_rows(m, w, g, gi, vertical=vert, slash=slash,
                                       query_pos=(pqi, torch.full_like(pqs, pin), pin))
    d2 = (wrong_succ - ref[:, :, torch.as_tensor(gi)]).abs().max().item()
    say(f"  rows >= C ({int(far.sum())}): gpu err={err_far:.3e}; dense-vs-sparse distance={dd:.3e} "
        f"(ratio {err_far / dd:.4f}); succ-as-inter distance on {len(gi)} rows={d2:.3e} "
        f"(ratio {err_far / d2:.4f}); bound 0.1")
    assert err_far <= 0.1 * dd
    assert err_far <= 0.1 * d2


def _needle_key(q_row, qpos, kpos, w):
    """A key that, rotated to position kpos, is a multiple of the query row
    rotated to qpos, scaled so that the pair's logit is 20: the needle then
    takes almost all of the row's softmax weight (about 0.998 against a
    million keys of these inputs) under the right position map only."""
    rq = O.rope_rotate(q_row.reshape(1, -1), torch.tensor([int(qpos)]), w.rope_base)
    alpha = 20.0 / (w.yarn_scale * rq.norm().item() ** 2 / math.sqrt(w.head_dim))
    return O.rope_rotate(alpha * rq, torch.tensor([-int(kpos)]), w.rope_base)[0]


def _plant(m, w, cases, h=0):
    """k with one needle key per case (row i, key j, query position of the
    pair's region) for query head h, on the device and (KV head of h only)
    on the host."""
    kvh = h // (w.n_q_heads // w.n_kv_heads)
    k2 = m["k"].clone()
    kh = m["kc"][:, kvh:kvh + 1].clone()
    pk = O.key_positions(w.seq, w.chunk)
    for i, j, qpos in cases:
        key = _needle_key(m["q"][0, h, i].cpu(), qpos, pk[j], w).to(m["k"].dtype)
        k2[0, kvh, j] = key.to(DEV)
        kh[0, 0, j] = key
    return k2, kh


def _oracle_group(m, w, rows, kh, h=0, **kw):
    """The oracle on a few rows of the query heads sharing h's KV head."""
    G = w.n_q_heads // w.n_kv_heads
    kvh = h // G
    rows_t = torch.as_tensor(rows)
    qg = m["q"][:, kvh * G:(kvh + 1) * G][:, :, rows_t.to(DEV)].cpu()
    vh = m["vc"][:, kvh:kvh + 1]
    if "vertical" in kw:
        kw = {**kw, "vertical": kw["vertical"][kvh * G:(kvh + 1) * G], "slash": kw["slash"][kvh * G:(kvh + 1) * G]}
    return O.dca_prefill_rows(qg, rows_t, kh, vh, w.chunk, w.window, w.rope_base, w.yarn_scale, **kw)


def test_planted_needles_1m():
    """Planted needles at the 1M-token shape, one per region: a successive
    pair inside the local window (true distance), a successive pair past it
    (pinned query), an inter-chunk pair and an intra-chunk pair. Each needle
    row's output must be within 0.06 of the needle's value row; a wrong query
    variant turns the needle away and leaves the row near the mean of a
    million values (far from it). The rows of the KV group's five heads are
    checked against the oracle as well."""
    m = _one_m()
    w = m["w"]
    S, C, W = w.seq, w.chunk, w.window
    pqi, pqs, pin = O.query_positions(S, C, W)
    cases = [  # (row, key, query position of the pair's region)
        (C + 3, C - 5, int(pqs[C + 3])),                           # successive, inside the window
        (2 * C + W + 10, C + 7, int(pqs[2 * C + W + 10])),         # successive, pinned
        (3 * C + 5, 100, pin),                                     # inter
        (2 * C + 500, 2 * C + 200, int(pqi[2 * C + 500])),         # intra
    ]
    say(f"[needles 1M] S={S} C={C} W={W}: rows {[c[0] for c in cases]}")
    k2, kh = _plant(m, w, cases)
    out, _ = _run(m["q"], k2, m["v"], w)
    rows = np.array([c[0] for c in cases])
    got = out[:, :5, torch.as_tensor(rows, device=DEV)].double().cpu()
    del out, k2
    torch.cuda.empty_cache()
    ref, _ = _oracle_group(m, w, rows, kh)
    for n, (i, j, _) in enumerate(cases):
        target = m["vc"][0, 0, j].double()
        dg, do = (got[0, 0, n] - target).abs().max().item(), (ref[0, 0, n] - target).abs().max().item()
        say(f"  row {i} key {j}: |gpu - v_j|={dg:.3e} |oracle - v_j|={do:.3e}")
        assert do < 0.05 and dg < 0.06
    err = (got - ref).abs().max().item()
    say(f"  five heads of the group on the needle rows: max abs err {err:.3e}")
    assert err <= TOL["bf16"]


def test_vs_needles_1m():
    """Needles under the 1M vertical-slash mask (head 0's lists): one key in
    a tile active through a vertical column (inter-chunk pair) and one in a
    tile active through a slash distance (successive pair inside the window)
    must each dominate their row; one in a tile the mask leaves out
    (successive pair, pinned query) must not move its row at all: that row is
    bit-identical to the sparse prefill without the needles, and far from the
    needle's value row (where a dense, mask-ignoring kernel would put it)."""
    m = _one_m()
    w = workloads.get("qwen14b_1m_vs")
    S, C, W = w.seq, w.chunk, w.window
    vert, slash = _vs_case(w, seed=0)
    vt, dl = O.vs_tile_lists(vert[0], slash[0], S)
    vt_set, dl_set = set(vt.tolist()), set(dl.tolist())
    pqs, pin = O.query_positions(S, C, W)[1:]
    tpc = C // 64
    i_a = 3 * C + 5                                   # inter: key tile with a vertical column, chunk 0
    kt_a = next(int(t) for t in vt.tolist() if 4 <= t < tpc - 4)
    i_s = C + 3                                       # successive inside the window: slash-active tile of chunk 0
    t_s = i_s // 64
    kt_s = next(t_s - d for d in sorted(dl_set, reverse=True) if 0 < t_s - d < tpc - 1 and t_s - d not in vt_set
                and t_s - d != kt_a)
    i_n = 2 * C + W + 10                              # successive, pinned: an inactive tile of chunk 1
    t_n = i_n // 64
    kt_n = next(kt for kt in range(tpc + 8, 2 * tpc - 8) if kt not in vt_set and t_n - kt not in dl_set)
    cases = [(i_a, 64 * kt_a + 7, pin), (i_s, 64 * kt_s + 9, int(pqs[i_s])), (i_n, 64 * kt_n + 11, int(pqs[i_n]))]
    for i, j, _ in cases:
        say(f"[vs needles 1M] row {i} key {j}: tile ({i // 64}, {j // 64}) "
            f"active={bool(O.vs_tile_active(vert[0], slash[0], torch.tensor([i // 64]), torch.tensor([j // 64]))[0])}")
    vd, sd = vert.to(DEV), slash.to(DEV)
    G = w.n_q_heads // w.n_kv_heads
    # the two active needles together; the inactive one alone (a vertical
    # needle is visible to every later query tile, the inactive row's too)
    active, inactive = cases[:2], cases[2:]
    rows = np.array([c[0] for c in active])
    k2, kh = _plant(m, w, active)
    out, _ = _run(m["q"], k2, m["v"], w, vertical=vd, slash=sd)
    got = out[:, :G, torch.as_tensor(rows, device=DEV)].double().cpu()
    del out, k2
    torch.cuda.empty_cache()
    ref, _ = _oracle_group(m, w, rows, kh, vertical=vert, slash=slash)
    for n, (i, j, _) in enumerate(active):
        target = m["vc"][0, 0, j].double()
        dg, do = (got[0, 0, n] - target).abs().max().item(), (ref[0, 0, n] - target).abs().max().item()
        say(f"  active: row {i} key {j}: |gpu - v_j|={dg:.3e} |oracle - v_j|={do:.3e}")
        assert do < 0.05 and dg < 0.06
    err = (got - ref).abs().max().item()
    say(f"  {G} heads of the group on the active needles' rows: max abs err {err:.3e}")
    assert err <= TOL["bf16"]
    i, j, _ = inactive[0]
    base, _ = _run(m["q"], m["k"], m["v"], w, vertical=vd, slash=sd)
    base_row = base[0, 0, i].clone()
    del base
    k3, _ = _plant(m, w, inactive)
    out, _ = _run(m["q"], k3, m["v"], w, vertical=vd, slash=sd)
    got_row = out[0, 0, i].clone()
    del out, k3
    torch.cuda.empty_cache()
    far = (got_row.double().cpu() - m["vc"][0, 0, j].double()).abs().max().item()
    same = torch.equal(got_row, base_row)
    say(f"  inactive: row {i} key {j}: identical to the prefill without the needle: {same}; |gpu - v_j|={far:.3e}")
    assert same and far > 0.2


@pytest.mark.parametrize("g", [0, 7])
def test_vs_estimate_1m_group(g):
    """The online vertical-slash estimate at the 1M shape with the benchmark's
    budgets (1000 columns, 2000 offsets, the first 64 of each forced, the last
    64 rows), on the shared seed-0 input: for the five query heads of KV group
    g, the column and diagonal scores against the oracle's, the lists exactly
    the selection rule applied to the kernel's own scores, and differing from
    the oracle's lists only at the budget's edge, within twice the measured
    score error."""
    m = _one_m()
    w = m["w"]
    S, n_last, nv, ns, forced = w.seq, 64, 1000, 2000, 64
    say(f"[vs estimate 1M] KV group {g}: S={S} n_last={n_last} nv={nv} ns={ns} forced={forced}")
    if "estimate" not in m:
        vert, slash, vs, ss = api.vs_estimate(m["q"], m["k"], nv, ns, forced, n_last, w.rope_base, w.yarn_scale,
                                              return_scores=True)
        torch.cuda.synchronize()
        m["estimate"] = (vert.cpu(), slash.cpu(), vs.cpu(), ss.cpu())
    vert, slash, vs, ss = m["estimate"]
    G = w.n_q_heads // w.n_kv_heads
    hs = range(g * G, (g + 1) * G)
    rows = torch.arange(S - n_last, S)
    q_last = m["q"][0, g * G:(g + 1) * G, S - n_last:].cpu()
    ref_vs, ref_ss = O.vs_scores(q_last, rows, m["kc"][0, g:g + 1], w.rope_base, w.yarn_scale)
    ev = (vs[g * G:(g + 1) * G].double() - ref_vs).abs().max().item()
    es = (ss[g * G:(g + 1) * G].double() - ref_ss).abs().max().item()
    say(f"  score err vertical={ev:.3e} slash={es:.3e} (largest scores {ref_vs.max().item():.3e}, "
        f"{ref_ss.max().item():.3e})")
    # on iid inputs every column and diagonal scores about 64 / S, so the
    # bound is relative to the largest score: 2^-9, one bf16 rounding of the
    # rotated keys and queries (measured: 4.4e-4 of it)
    assert ev <= 2e-3 * ref_vs.abs().max().item() and es <= 2e-3 * ref_ss.abs().max().item()
    for j, h in enumerate(hs):
        assert vert[h].long().tolist() == O.top_with_forced(vs[h].double(), nv, forced).tolist()
        assert slash[h].long().tolist() == O.top_with_forced(ss[h].double(), ns, forced).tolist()
        for got, sc, budget, err in ((vert[h], ref_vs[j], nv, ev), (slash[h], ref_ss[j], ns, es)):
            a, b = set(got.tolist()), set(O.top_with_forced(sc, budget, forced).tolist())
            if a == b:
                continue
            edge = min(float(sc[i]) for i in b if i >= forced)
            for i in a ^ b:
                assert abs(float(sc[i]) - edge) <= 2 * err + 1e-12, (h, i)
    say(f"  lists of heads {hs.start}..{hs.stop - 1}: the rule on the kernel's scores; oracle's up to edge ties")


def test_planted_needles_bf16():
    """For chosen rows, overwrite one key so that its rotated copy is a large
    multiple of the row's rotated query under the pair's region; the output of
    that row must then be close to the needle's value row."""
    w = _wl("qwen7b_32k", n_q_heads=4, n_kv_heads=1)
    say(f"[needles] S={w.seq} C={w.chunk} W={w.window}")
    q, k, v = synth.make_qkv(w, seed=5, device=DEV)
    S, C, W = w.seq, w.chunk, w.window
    pqi, pqs, pin = O.query_positions(S, C, W)
    pk = O.key_positions(S, C)
    cases = [  # (row, key, position variant of the pair)
        (C + 3, C - 5, pqs),            # successive, inside the window
        (2 * C + W + 10, C + 7, pqs),   # successive, pinned
        (3 * C + 5, 100, None),         # inter
        (2 * C + 500, 2 * C + 200, pqi),  # intra
    ]
    kc = k.cpu().clone()
    h = 0
    for i, j, var in cases:
        qpos = torch.tensor([pin]) if var is None else var[i:i + 1]
        rq = O.rope_rotate(q[0, h, i:i + 1].cpu(), qpos, w.rope_base)
        alpha = 20.0 / (w.yarn_scale * rq.norm().item() ** 2 / math.sqrt(w.head_dim))
        kc[0, 0, j] = O.rope_rotate(alpha * rq, -pk[j:j + 1], w.rope_base)[0].to(k.dtype)
    k2 = kc.to(DEV)
    out, _ = _run(q, k2, v, w)
    rows = np.array([c[0] for c in cases])
    ref, _ = _oracle(q, k2, v, rows, w)
    for n, (i, j, _) in enumerate(cases):
        got = out[0, h, i].double().cpu()
        target = v[0, 0, j].double().cpu()
        say(f"  row {i} key {j}: |gpu - v_j|={(got - target).abs().max():.3e} "
            f"|oracle - v_j|={(ref[0, h, n] - target).abs().max():.3e}")
        assert (ref[0, h, n] - target).abs().max() < 0.05
        assert (got - target).abs().max() < 0.06
    err = _err(out[:, :, torch.as_tensor(rows, device=DEV)], ref)
    assert err <= TOL["bf16"]


def test_deterministic_and_writes_every_output():
    w = _wl("qwen7b_32k", seq=5000, chunk=1024, window=128)
    say(f"[determinism] S={w.seq}")
    q, k, v = synth.make_qkv(w, seed=2, device=DEV)
    shape = api.shape_of(q, k)
    nbytes = api.dca_workspace_size(w.seq, w.chunk, w.window, shape)
    ws = api.alloc_workspace(nbytes, DEV)
    outs = []
    for _ in range(2):
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), device=DEV)
        api.dca_prefill(q, k, v, out, lse, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, None,
                        shape, ws, nbytes)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any() and not torch.isnan(lse).any()
        outs.append((out, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_workspace_too_small_leaves_output_untouched():
    w = _wl("qwen7b_32k", seq=1024, chunk=256, window=64)
    q, k, v = synth.make_qkv(w, seed=2, device=DEV)
    shape = api.shape_of(q, k)
    nbytes = api.dca_workspace_size(w.seq, w.chunk, w.window, shape)
    ws = api.alloc_workspace(nbytes, DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(api.DcaError) as e:
        api.dca_prefill(q, k, v, out, None, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, None,
                        shape, ws, nbytes - 1)
    assert e.value.status == api.DCA_E_WORKSPACE
    torch.cuda.synchronize()
    assert (out == 7.0).all()


def test_stages_equal_prefill():
    w = _wl("qwen7b_32k", seq=3000, chunk=512, window=64)
    q, k, v = synth.make_qkv(w, seed=4, device=DEV)
    ref = _run(q, k, v, w)[0]
    shape = api.shape_of(q, k)
    nbytes = api.dca_workspace_size(w.seq, w.chunk, w.window, shape)
    ws = api.alloc_workspace(nbytes, DEV)
    out = torch.empty_like(q)
    api.dca_remap(q, k, v, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, shape, ws, nbytes)
    api.dca_attention(out, None, w.seq, w.chunk, w.window, None, shape, ws, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


# ---------------------------------------------------------------------------
# vertical-slash sparse path
# ---------------------------------------------------------------------------

def _vs_case(w, seed=0):
    vert, slash = synth.vs_mask(w.n_q_heads, w.seq, w.n_vertical, w.n_slash, seed=seed)
    return torch.from_numpy(vert), torch.from_numpy(slash)


@pytest.mark.parametrize("S,nv,ns", [(4096, 40, 60), (1000, 70, 70), (131072, 1000, 2000)])
def test_vs_index_lists_bit_exact(S, nv, ns):
    say(f"[vs index] S={S} nv={nv} ns={ns}")
    w = _wl("qwen14b_1m_vs", seq=S, chunk=1024 if S >= 1024 else 64, window=64, n_vertical=nv, n_slash=ns,
            n_q_heads=8, n_kv_heads=2)
    vert, slash = _vs_case(w, seed=9)
    shape = api.make_shape(1, w.n_q_heads, w.n_kv_heads, w.head_dim, torch.bfloat16)
    vd, sd = vert.to(DEV), slash.to(DEV)
    mask = api.make_mask(vd, sd)
    nbytes = api.dca_workspace_size(S, w.chunk, w.window, shape, mask)
    ws = api.alloc_workspace(nbytes, DEV)
    api.dca_vs_index(S, w.chunk, w.window, mask, shape, ws, nbytes)
    nt = (S + 63) // 64
    vt = torch.empty((w.n_q_heads, nt), dtype=torch.int32, device=DEV)
    dl = torch.empty_like(vt)
    vn = torch.empty(w.n_q_heads, dtype=torch.int32, device=DEV)
    dn = torch.empty_like(vn)
    api.dca_debug_vs_lists(ws, nbytes, S, w.chunk, w.window, mask, shape, vt, vn, dl, dn)
    torch.cuda.synchronize()
    for h in range(w.n_q_heads):
        rvt, rdl = O.vs_tile_lists(vert[h], slash[h], S)
        assert int(vn[h]) == len(rvt) and int(dn[h]) == len(rdl)
        assert torch.equal(vt[h, :len(rvt)].cpu().long(), rvt)
        assert torch.equal(dl[h, :len(rdl)].cpu().long(), rdl)


@pytest.mark.parametrize("S,nv,ns,heads,q_tiles", [
    (4096, 40, 60, range(8), None),                # every query tile
    (1000, 70, 70, range(8), None),                # ragged: an odd tile count, a half-empty pair
    (1048576, 1000, 2000, (0, 17, 39), 48),        # the 1M shape: sampled and boundary query tiles
])
def test_vs_tile_order_bit_exact(S, nv, ns, heads, q_tiles):
    """The key tiles the attention kernel's own iterator visits, merged on the
    device from the per-head lists, against the tile mask defined directly
    from the columns and offsets (oracle): for one query tile the active
    tiles kt <= t ascending; for the kernel's two-tile workgroup their union,
    each with the bit of every query tile it is active for."""
    say(f"[vs tiles] S={S} nv={nv} ns={ns}")
    hq = 40 if S >= (1 << 20) else 8
    w = _wl("qwen14b_1m_vs", seq=S, chunk=1024 if S >= 1024 else 64, window=64, n_vertical=nv, n_slash=ns,
            n_q_heads=hq, n_kv_heads=hq // 5 if hq == 40 else 2)
    vert, slash = _vs_case(w, seed=21)
    shape = api.make_shape(1, w.n_q_heads, w.n_kv_heads, w.head_dim, torch.bfloat16)
    vd, sd = vert.to(DEV), slash.to(DEV)
    mask = api.make_mask(vd, sd)
    nbytes = api.dca_workspace_size(S, w.chunk, w.window, shape, mask)
    ws = api.alloc_workspace(nbytes, DEV)
    api.dca_vs_index(S, w.chunk, w.window, mask, shape, ws, nbytes)
    nt = (S + 63) // 64
    kt_out = torch.empty(nt, dtype=torch.int32, device=DEV)
    m_out = torch.empty(nt, dtype=torch.int32, device=DEV)
    n_out = torch.empty(1, dtype=torch.int32, device=DEV)
    if q_tiles is None:
        tiles = list(range(nt))
    else:
        rng = np.random.default_rng(3)
        tiles = sorted(set([0, 1, 2, 3, nt - 2, nt - 1, nt // 2, nt // 2 + 1]
                           + [int(x) for x in rng.integers(0, nt, q_tiles)]))
    checked = 0
    for h in heads:
        def active(t):
            kt = torch.arange(t + 1)
            return kt[O.vs_tile_active(vert[h], slash[h], torch.full_like(kt, t), kt)]
        for group in (1, 2):
            for t0 in sorted(set(t - t % group for t in tiles)):
                api.dca_debug_vs_tiles(ws, nbytes, S, w.chunk, w.window, mask, shape, h, t0, group,
                                       kt_out, m_out, n_out)
                n = int(n_out.item())
                assert n <= nt
                got_kt = kt_out[:n].cpu().long()
                got_m = m_out[:n].cpu().long()
                per_q = [active(t0 + q) if t0 + q < nt else torch.empty(0, dtype=torch.long) for q in range(group)]
                union = torch.unique(torch.cat(per_q))
                assert torch.equal(got_kt, union), (h, t0, group)
                for q in range(group):
                    assert torch.equal(got_kt[(got_m >> q) & 1 == 1], per_q[q]), (h, t0, group, q)
                assert ((got_m >> group) == 0).all()
                checked += 1
    say(f"  {checked} tile lists identical")


@pytest.mark.parametrize("S,C,W,nv,ns", [(4096, 1024, 128, 40, 60), (1000, 256, 64, 10, 12),
                                         (32768, 8192, 1024, 300, 600)])
def test_vs_parity(S, C, W, nv, ns):
    say(f"[vs parity] S={S} C={C} W={W} nv={nv} ns={ns}")
    w = _wl("qwen14b_1m_vs", seq=S, chunk=C, window=W, n_vertical=nv, n_slash=ns, n_q_heads=4,
            n_kv_heads=1)
    q, k, v = synth.make_qkv(w, seed=1, device=DEV)
    vert, slash = _vs_case(w, seed=1)
    out, lse = _run(q, k, v, w, vertical=vert.to(DEV), slash=slash.to(DEV))
    rows = synth.sample_rows(S, C, W, None if S <= 4096 else 512, seed=1)
    ref, ref_lse = _oracle(q, k, v, rows, w, vertical=vert, slash=slash)
    rows_t = torch.as_tensor(rows, device=DEV)
    err, lerr = _err(out[:, :, rows_t], ref), _err(lse[:, :, rows_t], ref_lse)
    dense, _ = _oracle(q, k, v, rows, w)
    dd = (dense - ref).abs().max().item()
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}; dense-vs-sparse distance {dd:.3e}")
    assert err <= TOL["bf16"] and lerr <= 2e-2
    assert err <= 0.1 * dd


@pytest.mark.parametrize("dtype,D,S,C,W,nv,ns", [
    ("bf16", 64, 2000, 512, 64, 12, 20),     # the d = 64 kernel instance
    ("f32", 64, 1500, 256, 32, 10, 16),      # fp32 instances, all rows
    ("f32", 128, 900, 128, 128, 8, 12),
])
def test_vs_parity_other_instances(dtype, D, S, C, W, nv, ns):
    """Vertical-slash parity for the kernel instances other than bf16 d = 128
    (which the cases above cover): all rows against the oracle."""
    say(f"[vs parity] dtype={dtype} D={D} S={S} C={C} W={W} nv={nv} ns={ns}")
    w = workloads.Workload("t", 1, 4, 2, D, S, C, W, dtype, 0.5 if dtype == "bf16" else 1.0, True,
                           n_vertical=nv, n_slash=ns)
    q, k, v = synth.make_qkv(w, seed=81, device=DEV)
    vert, slash = _vs_case(w, seed=81)
    out, lse = _run(q, k, v, w, vertical=vert.to(DEV), slash=slash.to(DEV))
    rows = np.arange(S)
    ref, ref_lse = _oracle(q, k, v, rows, w, vertical=vert, slash=slash)
    err, lerr = _err(out, ref), _err(lse, ref_lse)
    dense, _ = _oracle(q, k, v, rows, w)
    dd = (dense - ref).abs().max().item()
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}; dense-vs-sparse distance {dd:.3e}")
    assert err <= TOL[dtype] and lerr <= (1e-4 if dtype == "f32" else 2e-2)
    assert err <= 0.1 * dd


# ---------------------------------------------------------------------------
# chunked prefill: rows [q0, q0 + n) against keys [0, q0 + n), one workspace
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,Hq,Hkv,D,S,C,W,chunk", [
    ("bf16", 4, 2, 128, 8292, 2048, 512, 1536),   # blocks not a multiple of 256, ragged last block
    ("bf16", 3, 1, 64, 1000, 128, 128, 64),       # 64-row blocks
    ("f32", 2, 1, 64, 2048, 512, 128, 320),       # fp32, blocks straddle chunk boundaries
    ("bf16", 2, 1, 128, 4096, 4096, 100, 4096),   # one block = the whole sequence
    ("f32", 2, 1, 128, 700, 256, 64, 192),        # fp32, d = 128, ragged last block
])
def test_chunked_equals_whole_prefill(dtype, Hq, Hkv, D, S, C, W, chunk):
    say(f"[chunked] dtype={dtype} Hq={Hq} Hkv={Hkv} D={D} S={S} C={C} W={W} chunk={chunk}")
    w = workloads.Workload("t", 1, Hq, Hkv, D, S, C, W, dtype, 0.5 if dtype == "bf16" else 1.0, True)
    q, k, v = synth.make_qkv(w, seed=21, device=DEV)
    full, full_lse = _run(q, k, v, w)
    out, lse = api.prefill_chunked(q, k, v, C, W, chunk, w.rope_base, w.yarn_scale, return_lse=True)
    torch.cuda.synchronize()
    # every wave sees the same rows, keys and tile order either way
    assert torch.equal(out, full)
    assert torch.equal(lse, full_lse)
    rows = synth.sample_rows(S, C, W, 96, seed=3)
    ref, ref_lse = _oracle(q, k, v, rows, w)
    rows_t = torch.as_tensor(rows, device=DEV)
    err = _err(out[:, :, rows_t], ref)
    say(f"  bit-identical to the whole-sequence call; max abs err vs oracle {err:.3e}")
    assert err <= TOL[dtype]


def test_chunked_vertical_slash_equals_whole():
    say("[chunked vs] S=8192 C=2048 W=256 chunk=2048 nv=80 ns=120")
    w = _wl("qwen14b_1m_vs", seq=8192, chunk=2048, window=256, n_vertical=80, n_slash=120, n_q_heads=4,
            n_kv_heads=2)
    q, k, v = synth.make_qkv(w, seed=4, device=DEV)
    vert, slash = _vs_case(w, seed=4)
    vd, sd = vert.to(DEV), slash.to(DEV)
    full, full_lse = _run(q, k, v, w, vertical=vd, slash=sd)
    out, lse = api.prefill_chunked(q, k, v, w.chunk, w.window, 2048, w.rope_base, w.yarn_scale, vertical=vd,
                                   slash=sd, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, full)
    assert torch.equal(lse, full_lse)


def test_chunk_reads_only_earlier_blocks():
    """A block's output does not depend on keys past its last row: the same
    block computed with the later rows of q, k and v replaced by noise."""
    say("[chunk causality] bf16 S=4096 C=1024 W=128, block [1024, 2048)")
    w = workloads.Workload("t", 1, 2, 1, 128, 4096, 1024, 128, "bf16", 0.5, True)
    q, k, v = synth.make_qkv(w, seed=5, device=DEV)
    shape = api.shape_of(q, k)
    nbytes = api.dca_chunk_workspace_size(4096, 1024, w.chunk, w.window, shape)
    outs = []
    for noise in (False, True):
        ws = api.alloc_workspace(nbytes, DEV)
        k2, v2 = k.clone(), v.clone()
        if noise:
            k2[:, :, 2048:] = torch.randn_like(k2[:, :, 2048:].float()).to(k2.dtype) * 4
            v2[:, :, 2048:] = torch.randn_like(v2[:, :, 2048:].float()).to(v2.dtype) * 4
            # a later block written first must not leak into an earlier one
            o = torch.empty_like(q[:, :, 2048:3072])
            api.dca_prefill_chunk(q[:, :, 2048:3072].contiguous(), k2[:, :, 2048:3072].contiguous(),
                                  v2[:, :, 2048:3072].contiguous(), o, None, 2048, 1024, 4096, w.chunk, w.window,
                                  w.rope_base, w.yarn_scale, None, shape, ws, nbytes)
        for q0 in (0, 1024):
            o = torch.empty_like(q[:, :, q0:q0 + 1024])
            api.dca_prefill_chunk(q[:, :, q0:q0 + 1024].contiguous(), k2[:, :, q0:q0 + 1024].contiguous(),
                                  v2[:, :, q0:q0 + 1024].contiguous(), o, None, q0, 1024, 4096, w.chunk, w.window,
                                  w.rope_base, w.yarn_scale, None, shape, ws, nbytes)
        torch.cuda.synchronize()
        outs.append(o)
    assert torch.equal(outs[0], outs[1])


# ---------------------------------------------------------------------------
# decode: one new token at index pos against the cache a prefill left behind
# ---------------------------------------------------------------------------

def _decode_run(q, k, v, w, prompt, steps, yarn=None):
    """Prefill rows [0, prompt) as one block (when prompt > 0), then decode the
    tokens prompt .. prompt + steps - 1 one at a time on the same workspace
    (YaRN temperature: the workload's, unless given)."""
    yarn = w.yarn_scale if yarn is None else yarn
    shape = api.shape_of(q, k)
    S = w.seq
    nbytes = api.dca_chunk_workspace_size(S, max(prompt, 1), w.chunk, w.window, shape)
    ws = api.alloc_workspace(nbytes, DEV)
    if prompt > 0:
        o = torch.empty_like(q[:, :, :prompt])
        api.dca_prefill_chunk(q[:, :, :prompt].contiguous(), k[:, :, :prompt].contiguous(),
                              v[:, :, :prompt].contiguous(), o, None, 0, prompt, S, w.chunk, w.window, w.rope_base,
                              yarn, None, shape, ws, nbytes)
    outs, lses = [], []
    for pos in range(prompt, prompt + steps):
        o = torch.empty_like(q[:, :, pos])
        l = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
        api.dca_decode(q[:, :, pos].contiguous(), k[:, :, pos].contiguous(), v[:, :, pos].contiguous(), o, l, pos, S,
                       w.chunk, w.window, w.rope_base, yarn, shape, ws, nbytes)
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    return torch.stack(outs, 2), torch.stack(lses, 2)


@pytest.mark.parametrize("dtype,Hq,Hkv,D,S,C,W,prompt", [
    ("bf16", 8, 2, 128, 2200, 512, 64, 2040),    # decode crosses a 64-key tile (2048) and keeps going
    ("bf16", 5, 1, 128, 1100, 1024, 128, 1020),  # crosses the chunk boundary at 1024: intra -> new chunk
    ("f32", 4, 2, 64, 700, 128, 32, 600),        # fp32, d = 64, G = 2
    ("bf16", 7, 1, 64, 40, 64, 8, 0),            # no prompt: decode from pos 0 on a fresh workspace
    ("f32", 4, 1, 128, 300, 128, 16, 250),       # fp32, d = 128, G = 4
])
def test_decode_matches_oracle(dtype, Hq, Hkv, D, S, C, W, prompt):
    steps = min(S - prompt, 40)
    say(f"[decode] dtype={dtype} Hq={Hq} Hkv={Hkv} D={D} S={S} C={C} W={W} prompt={prompt} steps={steps}")
    w = workloads.Workload("t", 1, Hq, Hkv, D, S, C, W, dtype, 0.5 if dtype == "bf16" else 1.0, True)
    q, k, v = synth.make_qkv(w, seed=31, device=DEV)
    out, lse = _decode_run(q, k, v, w, prompt, steps)
    rows = np.arange(prompt, prompt + steps)
    ref, ref_lse = _oracle(q, k, v, rows, w)
    err, lerr = _err(out, ref), _err(lse, ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL[dtype]
    assert lerr <= (1e-4 if dtype == "f32" else 2e-2)
    if dtype == "bf16":
        assert _within_rounding(out, ref, v, rows, Hq // Hkv)


def test_decode_long_context():
    """Decode at a ~100K-token context (7B shape): the oracle on every decoded
    row, the discrimination guard against wrong position maps, and agreement
    with the prefill of the same rows."""
    # rows just past the start of the fourth 32K chunk: row offset < W, where
    # the successive-chunk position differs from the inter-chunk one
    prompt, steps = 3 * 32768 + 100, 6
    w = _wl("qwen7b_128k", seq=prompt + steps)
    say(f"[decode ~100K] prompt={prompt} steps={steps}")
    q, k, v = synth.make_qkv(w, seed=2, device=DEV)
    out, lse = _decode_run(q, k, v, w, prompt, steps)
    rows = np.arange(prompt, prompt + steps)
    ref, _ = _oracle(q, k, v, rows, w)
    err = _err(out, ref)
    _discrimination(q, k, v, rows, w, ref, out)
    pre, _ = _run(q, k, v, w)
    dp = (out.float() - pre[:, :, rows.tolist()].float()).abs().max().item()
    say(f"  max abs err {err:.3e}; decode vs prefill rows {dp:.3e}")
    assert err <= TOL["bf16"]
    assert dp <= TOL["bf16"]


def test_decode_at_1m_context():
    """Decode the last four tokens of the 1M-token Qwen2.5-14B shape after a
    chunk-call prefill of the rest, as the benchmark does: the oracle on every
    decoded row of all 40 heads, and the error far below the distance of
    vanilla RoPE from the DCA result. (These rows sit at the end of a chunk,
    past the window, where the successive and inter positions coincide, so
    the other wrong mapping of the long-context test is no wrong mapping
    here.)"""
    w = workloads.get("qwen14b_1m")
    steps = 4
    prompt = w.seq - steps
    say(f"[decode 1M] prompt={prompt} steps={steps}")
    q, k, v = synth.make_qkv(w, seed=4, device=DEV)
    out, lse = _decode_run(q, k, v, w, prompt, steps)
    rows = np.arange(prompt, prompt + steps)
    ref, ref_lse = _oracle(q, k, v, rows, w)
    err, lerr = _err(out, ref), _err(lse, ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= 2e-2
    rows_t = torch.as_tensor(rows)
    van, _ = O.vanilla_prefill_rows(q[:, :, rows_t.to(q.device)].cpu(), rows_t, k.cpu(), v.cpu(), w.rope_base,
                                    w.yarn_scale)
    dv = (van - ref).abs().max().item()
    say(f"  vanilla RoPE distance {dv:.3e}")
    assert err <= 0.1 * dv


# ---------------------------------------------------------------------------
# fused query rotation: identical to the path with materialized variants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,Hq,Hkv,D,S,C,W", [
    ("bf16", 4, 2, 128, 3000, 1024, 256),   # ragged tail, three chunks
    ("bf16", 3, 1, 64, 777, 128, 128),      # W = C, d = 64
    ("f32", 2, 1, 64, 2048, 512, 128),
    ("f32", 4, 1, 128, 515, 128, 32),
])
def test_fused_rotation_equals_materialized(dtype, Hq, Hkv, D, S, C, W):
    say(f"[fused] dtype={dtype} Hq={Hq} Hkv={Hkv} D={D} S={S} C={C} W={W}")
    w = workloads.Workload("t", 1, Hq, Hkv, D, S, C, W, dtype, 0.5 if dtype == "bf16" else 1.0, True)
    q, k, v = synth.make_qkv(w, seed=41, device=DEV)
    ref_out, ref_lse = _run(q, k, v, w)
    out, lse = api.prefill(q, k, v, C, W, w.rope_base, w.yarn_scale, return_lse=True, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    assert torch.equal(lse, ref_lse)
    rows = synth.sample_rows(S, C, W, 64, seed=5)
    ref, _ = _oracle(q, k, v, rows, w)
    err = _err(out[:, :, torch.as_tensor(rows, device=DEV)], ref)
    say(f"  bit-identical to the materialized path; max abs err vs oracle {err:.3e}")
    assert err <= TOL[dtype]


def test_fused_rotation_vertical_slash():
    say("[fused vs] S=8192 C=2048 W=256 nv=80 ns=120")
    w = _wl("qwen14b_1m_vs", seq=8192, chunk=2048, window=256, n_vertical=80, n_slash=120, n_q_heads=4,
            n_kv_heads=2)
    q, k, v = synth.make_qkv(w, seed=6, device=DEV)
    vert, slash = _vs_case(w, seed=6)
    vd, sd = vert.to(DEV), slash.to(DEV)
    ref_out, ref_lse = _run(q, k, v, w, vertical=vd, slash=sd)
    out, lse = api.prefill(q, k, v, w.chunk, w.window, w.rope_base, w.yarn_scale, vertical=vd, slash=sd,
                           return_lse=True, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    assert torch.equal(lse, ref_lse)


# ---------------------------------------------------------------------------
# batch > 1: each sequence of the batch against the oracle, and bit for bit
# against its own single-sequence call
# ---------------------------------------------------------------------------

def _one(t, b):
    return t[b:b + 1].contiguous()


@pytest.mark.parametrize("dtype,B,Hq,Hkv,D,S,C,W", [
    ("bf16", 3, 4, 2, 64, 700, 128, 32),     # ragged tail, G = 2
    ("f32", 2, 2, 1, 128, 300, 64, 64),      # fp32, W = C
])
def test_batched_prefill(dtype, B, Hq, Hkv, D, S, C, W):
    say(f"[batched] dtype={dtype} B={B} Hq={Hq} Hkv={Hkv} D={D} S={S} C={C} W={W}")
    w = workloads.Workload("t", B, Hq, Hkv, D, S, C, W, dtype, 0.5 if dtype == "bf16" else 1.0, True)
    q, k, v = synth.make_qkv(w, seed=61, device=DEV)
    out, lse = _run(q, k, v, w)
    ref, ref_lse = _oracle(q, k, v, np.arange(S), w)
    err, lerr = _err(out, ref), _err(lse, ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL[dtype] and lerr <= (1e-4 if dtype == "f32" else 2e-2)
    w1 = workloads.Workload("t", 1, Hq, Hkv, D, S, C, W, dtype, w.input_scale, True)
    for b in range(B):
        o1, l1 = _run(_one(q, b), _one(k, b), _one(v, b), w1)
        assert torch.equal(o1[0], out[b]) and torch.equal(l1[0], lse[b])


def test_batched_vertical_slash():
    w = _wl("qwen14b_1m_vs", batch=2, seq=3000, chunk=1024, window=128, n_vertical=40, n_slash=60, n_q_heads=4,
            n_kv_heads=2)
    say(f"[batched vs] B=2 S={w.seq} C={w.chunk} W={w.window} nv=40 ns=60")
    q, k, v = synth.make_qkv(w, seed=62, device=DEV)
    vert, slash = _vs_case(w, seed=62)
    vd, sd = vert.to(DEV), slash.to(DEV)
    out, lse = _run(q, k, v, w, vertical=vd, slash=sd)
    rows = synth.sample_rows(w.seq, w.chunk, w.window, 400, seed=2)
    ref, ref_lse = _oracle(q, k, v, rows, w, vertical=vert, slash=slash)
    rows_t = torch.as_tensor(rows, device=DEV)
    err, lerr = _err(out[:, :, rows_t], ref), _err(lse[:, :, rows_t], ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= 2e-2
    w1 = _wl("qwen14b_1m_vs", batch=1, seq=3000, chunk=1024, window=128, n_vertical=40, n_slash=60, n_q_heads=4,
             n_kv_heads=2)
    for b in range(2):
        o1, l1 = _run(_one(q, b), _one(k, b), _one(v, b), w1, vertical=vd, slash=sd)
        assert torch.equal(o1[0], out[b]) and torch.equal(l1[0], lse[b])


def test_batched_chunked_and_fused_equal_whole():
    w = workloads.Workload("t", 2, 4, 2, 128, 2500, 512, 64, "bf16", 0.5, True)
    say(f"[batched chunked/fused] B=2 S={w.seq} C={w.chunk} W={w.window} block=768")
    q, k, v = synth.make_qkv(w, seed=63, device=DEV)
    full, full_lse = _run(q, k, v, w)
    out, lse = api.prefill_chunked(q, k, v, w.chunk, w.window, 768, w.rope_base, w.yarn_scale, return_lse=True)
    fo, fl = api.prefill(q, k, v, w.chunk, w.window, w.rope_base, w.yarn_scale, return_lse=True, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(out, full) and torch.equal(lse, full_lse)
    assert torch.equal(fo, full) and torch.equal(fl, full_lse)


def test_batched_decode():
    w = workloads.Workload("t", 2, 8, 2, 128, 1200, 512, 64, "bf16", 0.5, True)
    prompt, steps = 1100, 20
    say(f"[batched decode] B=2 S={w.seq} C={w.chunk} W={w.window} prompt={prompt} steps={steps}")
    q, k, v = synth.make_qkv(w, seed=64, device=DEV)
    out, lse = _decode_run(q, k, v, w, prompt, steps)
    rows = np.arange(prompt, prompt + steps)
    ref, ref_lse = _oracle(q, k, v, rows, w)
    err, lerr = _err(out, ref), _err(lse, ref_lse)
    say(f"  max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL["bf16"] and lerr <= 2e-2


# ---------------------------------------------------------------------------
# HIP graph capture: the library records only kernel launches on the
# caller's stream (no allocation, memset or synchronization), so a call can
# be captured and replayed
# ---------------------------------------------------------------------------

def _replays_match(capture, outputs, refs, replays=3):
    """Capture `capture()` in a graph after one eager warm-up on a side
    stream, then replay it several times with eager work in between; every
    replay must reproduce `refs` bit for bit."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        capture()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    for r in range(replays):
        for o in outputs:
            o.fill_(float("nan"))                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outputs, refs):
            assert torch.equal(o, ref), f"replay {r}"


def test_graph_capture_prefill_and_decode():
    w = workloads.Workload("t", 1, 4, 2, 128, 3000, 1024, 128, "bf16", 0.5, True)
    say(f"[graph] S={w.seq} C={w.chunk} W={w.window}: dense, vertical-slash, decode")
    q, k, v = synth.make_qkv(w, seed=71, device=DEV)
    shape = api.shape_of(q, k)
    S, C, W = w.seq, w.chunk, w.window
    # dense prefill
    ref_out, ref_lse = _run(q, k, v, w)
    nbytes = api.dca_workspace_size(S, C, W, shape)
    ws = api.alloc_workspace(nbytes, DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    _replays_match(lambda: api.dca_prefill(q, k, v, out, lse, S, C, W, w.rope_base, w.yarn_scale, None, shape, ws,
                                           nbytes), [out, lse], [ref_out, ref_lse])
    # vertical-slash prefill
    wv = _wl("qwen14b_1m_vs", seq=S, chunk=C, window=W, n_vertical=40, n_slash=60, n_q_heads=4, n_kv_heads=2)
    vert, slash = _vs_case(wv, seed=71)
    vd, sd = vert.to(DEV), slash.to(DEV)
    ref_vo, ref_vl = _run(q, k, v, w, vertical=vd, slash=sd)
    mask = api.make_mask(vd, sd)
    vbytes = api.dca_workspace_size(S, C, W, shape, mask)
    vws = api.alloc_workspace(vbytes, DEV)
    _replays_match(lambda: api.dca_prefill(q, k, v, out, lse, S, C, W, w.rope_base, w.yarn_scale, mask, shape, vws,
                                           vbytes), [out, lse], [ref_vo, ref_vl])
    # one decode step after a 2900-row prompt (it rewrites the same cache slot)
    prompt = 2900
    dbytes = api.dca_chunk_workspace_size(S, prompt, C, W, shape)
    dws = api.alloc_workspace(dbytes, DEV)
    po = torch.empty_like(q[:, :, :prompt])
    api.dca_prefill_chunk(q[:, :, :prompt].contiguous(), k[:, :, :prompt].contiguous(),
                          v[:, :, :prompt].contiguous(), po, None, 0, prompt, S, C, W, w.rope_base, w.yarn_scale,
                          None, shape, dws, dbytes)
    qt, kt, vt = (t[:, :, prompt].contiguous() for t in (q, k, v))
    do = torch.empty_like(qt)
    dl = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)

    def dec():
        api.dca_decode(qt, kt, vt, do, dl, prompt, S, C, W, w.rope_base, w.yarn_scale, shape, dws, dbytes)

    dec()
    torch.cuda.synchronize()
    ref_do, ref_dl = do.clone(), dl.clone()
    _replays_match(dec, [do, dl], [ref_do, ref_dl])


def test_graph_capture_fused_and_chunked():
    """The fused-rotation prefill, and a chunked prefill of two blocks in one
    graph (the second block reads the keys the first wrote into the
    workspace), replayed with eager work in between: every replay equals the
    eager whole-sequence call bit for bit."""
    w = workloads.Workload("t", 1, 4, 2, 128, 3000, 1024, 128, "bf16", 0.5, True)
    say(f"[graph] S={w.seq} C={w.chunk} W={w.window}: fused, chunked in two blocks")
    q, k, v = synth.make_qkv(w, seed=72, device=DEV)
    shape = api.shape_of(q, k)
    S, C, W = w.seq, w.chunk, w.window
    ref_out, ref_lse = _run(q, k, v, w)
    fbytes = api.dca_fused_workspace_size(S, C, W, shape)
    fws = api.alloc_workspace(fbytes, DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    _replays_match(lambda: api.dca_prefill_fused(q, k, v, out, lse, S, C, W, w.rope_base, w.yarn_scale, None, shape,
                                                 fws, fbytes), [out, lse], [ref_out, ref_lse])
    blk = 1536
    cbytes = api.dca_chunk_workspace_size(S, blk, C, W, shape)
    cws = api.alloc_workspace(cbytes, DEV)
    blocks = []
    for q0 in (0, blk):
        n = min(blk, S - q0)
        ins = tuple(t[:, :, q0:q0 + n].contiguous() for t in (q, k, v))
        blocks.append((q0, n, ins, torch.empty_like(ins[0]),
                       torch.empty(q.shape[:2] + (n,), dtype=torch.float32, device=DEV)))

    def chunks():
        for q0, n, (qb, kb, vb), ob, lb in blocks:
            api.dca_prefill_chunk(qb, kb, vb, ob, lb, q0, n, S, C, W, w.rope_base, w.yarn_scale, None, shape, cws,
                                  cbytes)

    outs = [x for b in blocks for x in (b[3], b[4])]
    refs = [x for q0, n, *_ in blocks for x in (ref_out[:, :, q0:q0 + n], ref_lse[:, :, q0:q0 + n])]
    _replays_match(chunks, outs, refs)


# ---------------------------------------------------------------------------
# a plain C consumer of the ABI (tests/c_abi_example.c, built by build())
# ---------------------------------------------------------------------------

def _splitmix_bf16(seed, n):
    """The C example's inputs: splitmix64(seed + i) -> 24 bits in [-0.5, 0.5),
    rounded to bf16 (nearest even) with the same integer steps."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + np.arange(n, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z ^= z >> np.uint64(31)
    f = (z >> np.uint64(40)).astype(np.float32) * np.float32(1.0 / 16777216.0) - np.float32(0.5)
    u = f.view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return torch.from_numpy(u.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16)


def test_plain_c_consumer(tmp_path):
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_example")
    if not os.path.exists(exe):
        pytest.fail("tests/c_abi_example is missing: build it with __graft_entry__.build()")
    B, Hq, Hkv, D, S, C, W = 1, 4, 2, 128, 3000, 1024, 128
    say(f"[c consumer] {exe}: bf16 B={B} Hq={Hq} Hkv={Hkv} D={D} S={S} C={C} W={W}")
    dst = str(tmp_path / "c_out.bin")
    r = subprocess.run([exe, dst], capture_output=True, text=True, timeout=120)
    say("  " + (r.stdout + r.stderr).strip())
    assert r.returncode == 0
    raw = open(dst, "rb").read()
    nq, nl = B * Hq * S * D, B * Hq * S
    c_out = torch.frombuffer(bytearray(raw[:2 * nq]), dtype=torch.bfloat16).view(B, Hq, S, D)
    c_lse = torch.frombuffer(bytearray(raw[2 * nq:]), dtype=torch.float32).view(B, Hq, S)
    q = _splitmix_bf16(1, nq).view(B, Hq, S, D).to(DEV)
    k = _splitmix_bf16(2, B * Hkv * S * D).view(B, Hkv, S, D).to(DEV)
    v = _splitmix_bf16(3, B * Hkv * S * D).view(B, Hkv, S, D).to(DEV)
    yarn = float(np.float32(0.1 * math.log(S / C) + 1.0))
    out, lse = api.prefill(q, k, v, C, W, 1e7, yarn, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), c_out) and torch.equal(lse.cpu(), c_lse)


# ---------------------------------------------------------------------------
# online vertical-slash estimation (continuous positions)
# ---------------------------------------------------------------------------

def _est_case(dtype, Hq, Hkv, D, S, seed):
    w = workloads.Workload("t", 1, Hq, Hkv, D, S, 64, 0, dtype, 0.5 if dtype == "bf16" else 1.0, True)
    return w, synth.make_qkv(w, seed=seed, device=DEV)


@pytest.mark.parametrize("dtype,Hq,Hkv,D,S,n_last,nv,ns,forced", [
    ("bf16", 4, 2, 128, 3000, 64, 100, 200, 64),
    ("f32", 3, 1, 64, 1000, 64, 50, 80, 16),
    ("bf16", 2, 1, 64, 333, 20, 40, 333, 8),       # fewer rows, every offset kept
    ("bf16", 5, 1, 128, 70, 64, 70, 10, 0),        # short sequence, no forced head
    ("f32", 2, 1, 128, 900, 64, 60, 90, 16),       # fp32, d = 128
])
def test_vs_estimate_matches_oracle(dtype, Hq, Hkv, D, S, n_last, nv, ns, forced):
    say(f"[vs estimate] dtype={dtype} Hq={Hq} Hkv={Hkv} D={D} S={S} n_last={n_last} nv={nv} ns={ns} forced={forced}")
    w, (q, k, v) = _est_case(dtype, Hq, Hkv, D, S, seed=51)
    tau = 1.1386294361
    vert, slash, vs, ss = api.vs_estimate(q, k, nv, ns, forced, n_last, 1e7, tau, return_scores=True)
    torch.cuda.synchronize()
    rows = torch.arange(S - n_last, S)
    ref_v, ref_s, ref_vs, ref_ss = O.vs_estimate(q[0, :, rows].cpu(), rows, k[0].cpu(), 1e7, nv, ns, forced, tau)
    ev = (vs.double().cpu() - ref_vs).abs().max().item()
    es = (ss.double().cpu() - ref_ss).abs().max().item()
    say(f"  score err vertical={ev:.3e} slash={es:.3e}")
    tol = TOL[dtype]
    assert ev <= tol and es <= tol
    # the lists are exactly the selection the rule makes on the kernel's own scores
    for h in range(Hq):
        assert vert[h].cpu().long().tolist() == O.top_with_forced(vs[h].double().cpu(), nv, forced).tolist()
        assert slash[h].cpu().long().tolist() == O.top_with_forced(ss[h].double().cpu(), ns, forced).tolist()
        # and differ from the oracle's only on near-ties at the budget's edge
        for got, ref, sc in ((vert[h], ref_v[h], ref_vs[h]), (slash[h], ref_s[h], ref_ss[h])):
            a, b = set(got.cpu().tolist()), set(ref.tolist())
            if a == b:
                continue
            edge = min(float(sc[i]) for i in b if i >= forced)
            for i in a ^ b:
                assert abs(float(sc[i]) - edge) <= 2 * tol, (h, i)


def test_vs_estimate_ties_across_compaction_steps():
    """A 50K-token sequence (the selection compacts several 8192-score steps)
    with ~13K zeroed keys: their columns score exactly alike, and the
    vertical budget is set so that its edge falls inside that run of ties.
    The lists must be exactly the selection rule on the kernel's own scores
    (ties to the smaller index), and the scores match the oracle's."""
    S, Hq, Hkv, D, n_last, forced = 50000, 2, 1, 64, 64, 64
    say(f"[vs estimate ties] S={S}")
    w, (q, k, v) = _est_case("bf16", Hq, Hkv, D, S, seed=53)
    k[0, 0, 1000:40000:3] = 0
    tied = torch.arange(1000, 40000, 3)
    _, _, vs, _ = api.vs_estimate(q, k, 100, 100, forced, n_last, 1e7, 1.0, return_scores=True)
    torch.cuda.synchronize()
    vsc = vs.double().cpu()
    # the zeroed columns share one score per head; budget = forced + (columns
    # above it) + half of the tied run
    nvs = []
    for h in range(Hq):
        c0 = vsc[h, tied]
        assert torch.equal(c0, c0[:1].expand_as(c0)), "zeroed keys must tie exactly"
        above = int((vsc[h, forced:] > c0[0]).sum())
        nvs.append(forced + above + tied.numel() // 2)
    nv = max(nvs)
    vert, slash, vs2, ss2 = api.vs_estimate(q, k, nv, 3000, forced, n_last, 1e7, 1.0, return_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(vs2, vs)
    for h in range(Hq):
        assert vert[h].cpu().long().tolist() == O.top_with_forced(vs2[h].double().cpu(), nv, forced).tolist()
        assert slash[h].cpu().long().tolist() == O.top_with_forced(ss2[h].double().cpu(), 3000, forced).tolist()
    rows = torch.arange(S - n_last, S)
    _, _, ref_vs, ref_ss = O.vs_estimate(q[0, :, rows].cpu(), rows, k[0].cpu(), 1e7, nv, 3000, forced, 1.0)
    ev = (vs2.double().cpu() - ref_vs).abs().max().item()
    es = (ss2.double().cpu() - ref_ss).abs().max().item()
    say(f"  score err vertical={ev:.3e} slash={es:.3e}; budget {nv}")
    assert ev <= TOL["bf16"] and es <= TOL["bf16"]


def test_vs_estimate_finds_planted_pattern_and_drives_sparse_prefill():
    """Keys planted along a column and along a diagonal are found at a
    16K-token sequence, and the lists drive the sparse prefill."""
    S, Hq, Hkv, D = 16384, 2, 1, 128
    say(f"[vs estimate planted] S={S}")
    w = workloads.Workload("t", 1, Hq, Hkv, D, S, 4096, 512, "bf16", 0.5, True)
    q, k, v = synth.make_qkv(w, seed=52, device=DEV)
    # energy only in the slowest RoPE pair: the logits are nearly position-free
    unit = torch.zeros(D, device=DEV)
    unit[D // 2 - 1] = 1.0
    q[:, :, S - 64:] = (unit * 0.5).to(q.dtype)
    k[0, 0, 5000] = (unit * 12).to(k.dtype)
    o_star = 9000
    for i in range(S - 64, S):
        k[0, 0, i - o_star] = (unit * 8).to(k.dtype)
    vert, slash = api.vs_estimate(q, k, 200, 400, 64)
    torch.cuda.synchronize()
    for h in range(Hq):
        assert 5000 in vert[h].tolist()
        assert o_star in slash[h].tolist()
    out = api.prefill(q, k, v, w.chunk, w.window, w.rope_base, w.yarn_scale, vertical=vert, slash=slash)
    torch.cuda.synchronize()
    rows = np.array([S - 1, S - 30, 12000, 700])
    ref, _ = _oracle(q, k, v, rows, w, vertical=vert.cpu().long(), slash=slash.cpu().long())
    assert _err(out[:, :, torch.as_tensor(rows, device=DEV)], ref) <= TOL["bf16"]


# ---------------------------------------------------------------------------
# seeded random configurations: every entry point over the supported domain
# ---------------------------------------------------------------------------

_N_RANDOM = 64


def _random_case(i):
    """One seeded draw over the supported domain: dtype, head_dim, batch, GQA
    ratio, chunk C (a multiple of 64), window W (0, 1, C - 1, C or between),
    sequence length (from a single row to a few thousand, ragged, or on a
    chunk boundary give or take one), YaRN temperature,
    entry point (whole-sequence, fused rotation, chunked with a random block,
    decode) and, for the prefill entry points, sometimes a vertical-slash
    mask with small random budgets."""
    rng = np.random.default_rng(7000 + i)
    c = {}
    c["dtype"] = "bf16" if rng.random() < 0.7 else "f32"
    c["D"] = int(rng.choice([64, 128]))
    c["B"] = 1 if rng.random() < 0.75 else 2
    c["Hkv"] = int(rng.choice([1, 2]))
    c["G"] = int(rng.choice([1, 2, 3, 5, 8]))
    c["C"] = 64 * int(rng.integers(1, 10))
    u = rng.random()
    if u < 0.15:
        c["S"] = int(rng.integers(1, 65))                       # inside the first key tile
    elif u < 0.3:
        # on a chunk boundary, one short of it or one past it
        c["S"] = max(1, c["C"] * int(rng.integers(1, 5)) + int(rng.integers(-1, 2)))
    else:
        c["S"] = int(rng.integers(65, 2600))
    c["W"] = int(rng.choice([0, 1, c["C"] - 1, c["C"], int(rng.integers(0, c["C"] + 1))]))
    c["yarn"] = float(rng.choice([1.0, 1.1386294361]))
    c["mode"] = str(rng.choice(["prefill", "fused", "chunked", "decode"]))
    c["block"] = 64 * int(rng.integers(1, 9))
    c["steps"] = min(c["S"], int(rng.integers(1, 9)))
    c["mask"] = c["mode"] != "decode" and rng.random() < 0.35
    c["nv"] = int(rng.integers(1, min(c["S"], 48) + 1))
    c["ns"] = int(rng.integers(1, min(c["S"], 48) + 1))
    c["forced"] = int(rng.integers(1, min(c["nv"], c["ns"], 8) + 1))
    return c


@pytest.mark.parametrize("i", range(_N_RANDOM))
def test_random_configuration(i):
    c = _random_case(i)
    say(f"[random {i}] {c}")
    dtype, S, C, W = c["dtype"], c["S"], c["C"], c["W"]
    Hq = c["Hkv"] * c["G"]
    w = workloads.Workload("t", c["B"], Hq, c["Hkv"], c["D"], S, C, W, dtype, 0.5 if dtype == "bf16" else 1.0,
                           False)
    q, k, v = synth.make_qkv(w, seed=7000 + i, device=DEV)
    yarn = c["yarn"]
    vert = slash = vd = sd = None
    if c["mask"]:
        # a few forced entries (offset 0 keeps every row's diagonal tile), the
        # rest drawn from the whole sequence
        vn, sn = synth.vs_mask(Hq, S, c["nv"], c["ns"], seed=7000 + i, forced=c["forced"])
        vert, slash = torch.from_numpy(vn), torch.from_numpy(sn)
        vd, sd = vert.to(DEV), slash.to(DEV)
    if c["mode"] == "decode":
        prompt = S - c["steps"]
        out, lse = _decode_run(q, k, v, w, prompt, c["steps"], yarn=yarn)
        rows = np.arange(prompt, S)
        got, got_lse = out, lse
    else:
        if c["mode"] == "chunked":
            out, lse = api.prefill_chunked(q, k, v, C, W, c["block"], w.rope_base, yarn, vertical=vd, slash=sd,
                                           return_lse=True)
        else:
            out, lse = api.prefill(q, k, v, C, W, w.rope_base, yarn, vertical=vd, slash=sd, return_lse=True,
                                   fused=c["mode"] == "fused")
        torch.cuda.synchronize()
        rows = np.arange(S) if S <= 700 else synth.sample_rows(S, C, W, 96, seed=i)
        rows_t = torch.as_tensor(rows, device=DEV)
        got, got_lse = out[:, :, rows_t], lse[:, :, rows_t]
    rows_c = torch.as_tensor(rows, dtype=torch.int64)
    ref, ref_lse = O.dca_prefill_rows(q[:, :, rows_c.to(DEV)].cpu(), rows_c, k.cpu(), v.cpu(), C, W, w.rope_base,
                                      yarn, vertical=vert, slash=slash)
    err, lerr = _err(got, ref), _err(got_lse, ref_lse)
    say(f"  {len(rows)} rows x {c['B'] * Hq} heads: max abs err out={err:.3e} lse={lerr:.3e}")
    assert err <= TOL[dtype]
    assert lerr <= (1e-4 if dtype == "f32" else 2e-2)
    if dtype == "bf16":
        assert _within_rounding(got, ref, v, rows, c["G"])


_N_RANDOM_EST = 32


def _random_estimate_case(i):
    """One seeded draw over the online estimate's domain: dtype, head_dim, GQA
    ratio, sequence length (inside one key tile, one off a multiple of the
    8192 scores the selection stages at a time, or up to 12K), the number of
    scored rows (1 to 64), both budgets (1 to the whole sequence), the forced
    head (0 to the smaller budget, at most 64) and the YaRN temperature."""
    rng = np.random.default_rng(9000 + i)
    c = {"dtype": "bf16" if rng.random() < 0.7 else "f32", "D": int(rng.choice([64, 128])),
         "Hkv": int(rng.choice([1, 2])), "G": int(rng.choice([1, 2, 3, 5]))}
    u = rng.random()
    if u < 0.15:
        c["S"] = int(rng.integers(1, 65))
    elif u < 0.35:
        c["S"] = max(1, 8192 * int(rng.integers(1, 3)) + int(rng.integers(-1, 2)))
    else:
        c["S"] = int(rng.integers(65, 12000))
    S = c["S"]
    c["n_last"] = int(rng.integers(1, min(64, S) + 1))
    c["nv"] = S if rng.random() < 0.1 else int(rng.integers(1, min(S, 3000) + 1))
    c["ns"] = S if rng.random() < 0.1 else int(rng.integers(1, min(S, 3000) + 1))
    c["forced"] = int(rng.integers(0, min(c["nv"], c["ns"], 64) + 1))
    c["yarn"] = float(rng.choice([1.0, 1.1386294361]))
    return c


@pytest.mark.parametrize("i", range(_N_RANDOM_EST))
def test_random_estimate(i):
    c = _random_estimate_case(i)
    say(f"[random estimate {i}] {c}")
    dtype, S, n_last, nv, ns, forced = c["dtype"], c["S"], c["n_last"], c["nv"], c["ns"], c["forced"]
    Hq = c["Hkv"] * c["G"]
    w, (q, k, v) = _est_case(dtype, Hq, c["Hkv"], c["D"], S, seed=9000 + i)
    vert, slash, vs, ss = api.vs_estimate(q, k, nv, ns, forced, n_last, 1e7, c["yarn"], return_scores=True)
    torch.cuda.synchronize()
    rows = torch.arange(S - n_last, S)
    ref_v, ref_s, ref_vs, ref_ss = O.vs_estimate(q[0, :, rows].cpu(), rows, k[0].cpu(), 1e7, nv, ns, forced,
                                                 c["yarn"])
    ev = (vs.double().cpu() - ref_vs).abs().max().item()
    es = (ss.double().cpu() - ref_ss).abs().max().item()
    # relative to the largest score (a score is about n_last / S on iid
    # inputs): one bf16 rounding of the rotated queries and keys, or fp32
    # sums over up to 12K keys
    rel = 2e-3 if dtype == "bf16" else 1e-4
    say(f"  score err vertical={ev:.3e} slash={es:.3e} (largest {ref_vs.max().item():.3e}, {ref_ss.max().item():.3e})")
    assert ev <= rel * ref_vs.abs().max().item() and es <= rel * ref_ss.abs().max().item()
    vsc, ssc = vs.double().cpu(), ss.double().cpu()
    for h in range(Hq):
        assert vert[h].cpu().long().tolist() == O.top_with_forced(vsc[h], nv, forced).tolist()
        assert slash[h].cpu().long().tolist() == O.top_with_forced(ssc[h], ns, forced).tolist()
        for got, ref, sc, err in ((vert[h], ref_v[h], ref_vs[h], ev), (slash[h], ref_s[h], ref_ss[h], es)):
            a, b = set(got.cpu().tolist()), set(ref.tolist())
            if a == b:
                continue
            edge = min(float(sc[j]) for j in b if j >= forced)
            for j in a ^ b:
                assert abs(float(sc[j]) - edge) <= 2 * err + 1e-12, (h, j)
