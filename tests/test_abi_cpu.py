"""The C-ABI library on a host without a GPU: it loads, exports every entry
point include/dca.h declares, computes the host position map bit-exactly
against the oracle, sizes the workspace, and rejects bad arguments before any
HIP call."""

from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

from oracle import dca_oracle as O
from position_extrapolation_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dca.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dca_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_entry_point():
    names = _declared()
    assert len(names) >= 12
    L = api.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(api.EXPORTS) == names


@pytest.mark.parametrize("S,C,W", [(20, 8, 3), (2048, 512, 128), (1000, 64, 0), (777, 128, 128),
                                   (131072, 32768, 4096)])
def test_host_positions_bit_exact(S, C, W):
    pqi, pqs, pinter, pk = api.dca_remap_positions(S, C, W)
    oi, os_, op = O.query_positions(S, C, W)
    assert torch.equal(pqi.to(torch.int64), oi)
    assert torch.equal(pqs.to(torch.int64), os_)
    assert pinter == op
    assert torch.equal(pk.to(torch.int64), O.key_positions(S, C))


def test_workspace_size_formula():
    sh = api.make_shape(1, 28, 4, 128, torch.bfloat16)
    S, C, W = 32768, 8192, 1024
    n = api.dca_workspace_size(S, C, W, sh)
    q = 28 * S * 128 * 2
    kv = 4 * S * 128 * 2
    table = (C + W) * 64 * 8
    assert n >= 3 * q + 2 * kv + table
    assert n <= 3 * q + 2 * kv + table + 6 * 256
    m = api.dca_vs_mask(None, None, 0, 0)
    assert api.dca_workspace_size(S, C, W, sh, m) > n


def _call_prefill(**over):
    sh = over.pop("shape", api.make_shape(1, 2, 1, 64, torch.float32))
    args = dict(q=0x10000000, k=0x20000000, v=0x30000000, out=0x40000000, lse=None, seq=2048, C=512,
                W=128, base=1e7, yarn=1.0, mask=None, ws=0x50000000, ws_bytes=1 << 30)
    args.update(over)
    L = api.lib()
    return L.dca_prefill(args["q"], args["k"], args["v"], args["out"], args["lse"], args["seq"], args["C"],
                         args["W"], args["base"], args["yarn"],
                         None if args["mask"] is None else ctypes.byref(args["mask"]), ctypes.byref(sh),
                         args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(q=None), api.DCA_E_INVALID),
    (dict(out=None), api.DCA_E_INVALID),
    (dict(seq=0), api.DCA_E_INVALID),
    (dict(C=100), api.DCA_E_UNSUPPORTED),
    (dict(C=0), api.DCA_E_INVALID),
    (dict(W=-1), api.DCA_E_INVALID),
    (dict(W=600), api.DCA_E_UNSUPPORTED),
    (dict(base=1.0), api.DCA_E_INVALID),
    (dict(base=float("nan")), api.DCA_E_INVALID),
    (dict(yarn=0.0), api.DCA_E_INVALID),
    (dict(yarn=float("inf")), api.DCA_E_INVALID),
    (dict(ws=None), api.DCA_E_INVALID),
    (dict(ws=0x50000010), api.DCA_E_INVALID),
    (dict(ws_bytes=1000), api.DCA_E_WORKSPACE),
    (dict(out=0x10000000), api.DCA_E_INVALID),            # out aliases q
    (dict(out=0x50000000 + 4096), api.DCA_E_INVALID),     # out inside the workspace
    (dict(lse=0x40000000 + 100), api.DCA_E_INVALID),      # lse inside out
    (dict(q=0x50000000 + 4096), api.DCA_E_INVALID),       # q inside the workspace
    (dict(k=0x50000000 + (1 << 29)), api.DCA_E_INVALID),  # k inside the workspace
    (dict(v=0x50000000 - 4096), api.DCA_E_INVALID),       # v runs into the workspace
    (dict(shape=api.make_shape(1, 3, 2, 64, torch.float32)), api.DCA_E_INVALID),
    (dict(shape=api.make_shape(1, 2, 1, 96, torch.float32)), api.DCA_E_UNSUPPORTED),
    (dict(shape=api.make_shape(0, 2, 1, 64, torch.float32)), api.DCA_E_INVALID),
    (dict(shape=api.dca_shape(1, 2, 1, 64, 7, 0.0)), api.DCA_E_INVALID),
    (dict(shape=api.dca_shape(1, 2, 1, 64, 0, -1.0)), api.DCA_E_INVALID),
    (dict(mask=api.dca_vs_mask(None, None, 5, 0)), api.DCA_E_INVALID),
    (dict(mask=api.dca_vs_mask(None, None, -1, 0)), api.DCA_E_INVALID),
    (dict(mask=api.dca_vs_mask(0x50000000 + 4096, 0xA1000000, 10, 10)), api.DCA_E_INVALID),  # list in the workspace
    (dict(mask=api.dca_vs_mask(0xA0000000, 0x40000000 + 64, 10, 10)), api.DCA_E_INVALID),    # list inside out
    (dict(mask=api.dca_vs_mask(0xA0000000, 0xB0000000, 10, 10), lse=0xB0000000 - 16),
     api.DCA_E_INVALID),                                                                    # list inside lse
    (dict(seq=1 << 31), api.DCA_E_UNSUPPORTED),
])
def test_invalid_arguments_rejected_before_any_hip_call(over, status):
    assert _call_prefill(**over) == status
    assert api.dca_last_error() != ""


def test_valid_call_without_gpu_reports_device_error():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call_prefill() == api.DCA_E_DEVICE
    assert "HIP error" in api.dca_last_error()


def test_chunk_workspace_size():
    sh = api.make_shape(1, 28, 4, 128, torch.bfloat16)
    S, C, W = 32768, 8192, 1024
    whole = api.dca_workspace_size(S, C, W, sh)
    assert api.dca_chunk_workspace_size(S, S, C, W, sh) == whole
    small = api.dca_chunk_workspace_size(S, 4096, C, W, sh)
    # three query variants of 4096 rows instead of 32768
    assert whole - small == 3 * 28 * (S - 4096) * 128 * 2
    for bad in (0, S + 1):
        with pytest.raises(api.DcaError):
            api.dca_chunk_workspace_size(S, bad, C, W, sh)


def test_fused_workspace_size():
    sh = api.make_shape(1, 28, 4, 128, torch.bfloat16)
    S, C, W = 32768, 8192, 1024
    whole = api.dca_workspace_size(S, C, W, sh)
    fused = api.dca_fused_workspace_size(S, C, W, sh)
    # no query variants: three query-sized sections less
    assert whole - fused == 3 * 28 * S * 128 * 2
    L = api.lib()
    bad = L.dca_prefill_fused(0x10000000, 0x20000000, 0x30000000, 0x40000000, None, S, C, W, 1e7, 1.0, None,
                              ctypes.byref(sh), 0x50000000, fused - 256, None)
    assert bad == api.DCA_E_WORKSPACE


def _call_chunk(**over):
    sh = api.make_shape(1, 2, 1, 64, torch.float32)
    args = dict(q=0x10000000, k=0x20000000, v=0x30000000, out=0x40000000, lse=None, q_offset=512, n_rows=256,
                seq=2048, C=512, W=128, base=1e7, yarn=1.0, mask=None, ws=0x50000000, ws_bytes=1 << 30)
    args.update(over)
    return api.lib().dca_prefill_chunk(args["q"], args["k"], args["v"], args["out"], args["lse"], args["q_offset"],
                                       args["n_rows"], args["seq"], args["C"], args["W"], args["base"],
                                       args["yarn"], None if args["mask"] is None else ctypes.byref(args["mask"]),
                                       ctypes.byref(sh), args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(q_offset=100), api.DCA_E_UNSUPPORTED),          # not a multiple of 64
    (dict(q_offset=-64), api.DCA_E_INVALID),
    (dict(n_rows=0), api.DCA_E_INVALID),
    (dict(q_offset=1920, n_rows=256), api.DCA_E_INVALID),  # past the sequence
    (dict(ws_bytes=1 << 20), api.DCA_E_WORKSPACE),
    (dict(out=0x10000000 + 4096), api.DCA_E_INVALID),     # out overlaps q
    (dict(k=None), api.DCA_E_INVALID),
    (dict(v=0x50000000 + 256), api.DCA_E_INVALID),        # v inside the workspace
    (dict(mask=api.dca_vs_mask(0xA0000000, 0x50000000 + 256, 10, 10)), api.DCA_E_INVALID),   # list in the workspace
    (dict(mask=api.dca_vs_mask(0x40000000 + 512, 0xA1000000, 10, 10)), api.DCA_E_INVALID),   # list inside out
])
def test_chunk_arguments_rejected_before_any_hip_call(over, status):
    assert _call_chunk(**over) == status
    assert api.dca_last_error() != ""


def test_valid_chunk_call_without_gpu_reports_device_error():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call_chunk() == api.DCA_E_DEVICE


def _call_decode(**over):
    sh = over.pop("shape", api.make_shape(1, 4, 2, 64, torch.float32))
    args = dict(q=0x10000000, k=0x20000000, v=0x30000000, out=0x40000000, lse=None, pos=700, seq=2048, C=512,
                W=128, base=1e7, yarn=1.0, ws=0x50000000, ws_bytes=1 << 30)
    args.update(over)
    return api.lib().dca_decode(args["q"], args["k"], args["v"], args["out"], args["lse"], args["pos"], args["seq"],
                                args["C"], args["W"], args["base"], args["yarn"], ctypes.byref(sh), args["ws"],
                                args["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(pos=-1), api.DCA_E_INVALID),
    (dict(pos=2048), api.DCA_E_INVALID),
    (dict(v=None), api.DCA_E_INVALID),
    (dict(ws_bytes=1 << 16), api.DCA_E_WORKSPACE),
    (dict(shape=api.make_shape(1, 66, 2, 64, torch.float32)), api.DCA_E_UNSUPPORTED),   # 33 heads per group
    (dict(out=0x30000000), api.DCA_E_INVALID),            # out aliases v
    (dict(yarn=-1.0), api.DCA_E_INVALID),
    (dict(q=0x50000000 + 4096), api.DCA_E_INVALID),       # the new query inside the cache workspace
])
def test_decode_arguments_rejected_before_any_hip_call(over, status):
    assert _call_decode(**over) == status
    assert api.dca_last_error() != ""


def test_valid_decode_call_without_gpu_reports_device_error():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call_decode() == api.DCA_E_DEVICE


def _call_estimate(**over):
    sh = over.pop("shape", api.make_shape(1, 4, 2, 64, torch.float32))
    args = dict(q=0x10000000, k=0x20000000, seq=2048, n_last=64, base=1e7, yarn=1.0, nv=100, ns=200, nf=64,
                vert=0x30000000, slash=0x31000000, vs=None, ss=None, ws=0x50000000, ws_bytes=1 << 30)
    args.update(over)
    return api.lib().dca_vs_estimate(args["q"], args["k"], args["seq"], args["n_last"], args["base"], args["yarn"],
                                     args["nv"], args["ns"], args["nf"], ctypes.byref(sh), args["vert"],
                                     args["slash"], args["vs"], args["ss"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(n_last=0), api.DCA_E_INVALID),
    (dict(n_last=65), api.DCA_E_INVALID),
    (dict(nv=0), api.DCA_E_INVALID),
    (dict(ns=4096), api.DCA_E_INVALID),                   # budget past the sequence
    (dict(nf=101), api.DCA_E_INVALID),                    # forced past a budget
    (dict(vert=None), api.DCA_E_INVALID),
    (dict(shape=api.make_shape(2, 4, 2, 64, torch.float32)), api.DCA_E_UNSUPPORTED),   # batch 2
    (dict(ws_bytes=1 << 20), api.DCA_E_WORKSPACE),
    (dict(slash=0x30000000 + 64), api.DCA_E_INVALID),     # lists overlap
    (dict(k=0x50000000 + 4096), api.DCA_E_INVALID),       # k inside the workspace
    (dict(vs=0x50000000 + 4096), api.DCA_E_INVALID),      # a score output inside the workspace
    (dict(vs=0xA0000000, ss=0xA0000000 + 64), api.DCA_E_INVALID),   # the score outputs overlap
    (dict(ss=0x30000000 - 64), api.DCA_E_INVALID),        # a score output runs into the vertical list
    (dict(ss=0x10000000 + 4096), api.DCA_E_INVALID),      # a score output inside q
    (dict(vert=0x20000000 + 128), api.DCA_E_INVALID),     # a list inside k
])
def test_estimate_arguments_rejected_before_any_hip_call(over, status):
    assert _call_estimate(**over) == status
    assert api.dca_last_error() != ""


def test_valid_masked_and_scored_calls_without_gpu_report_device_error():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    # the fake workspace spans [0x50000000, 0x90000000): lists and scores above it
    assert _call_prefill(mask=api.dca_vs_mask(0xA0000000, 0xA1000000, 10, 10)) == api.DCA_E_DEVICE
    assert _call_chunk(mask=api.dca_vs_mask(0xA0000000, 0xA1000000, 10, 10)) == api.DCA_E_DEVICE
    assert _call_estimate(vs=0xA0000000, ss=0xA1000000) == api.DCA_E_DEVICE


def test_index_and_fused_reject_mask_lists_in_the_workspace():
    sh = api.make_shape(1, 2, 1, 64, torch.float32)
    L = api.lib()
    inside = api.dca_vs_mask(0x50000000 + 4096, 0xA1000000, 10, 10)
    st = L.dca_vs_index(2048, 512, 128, ctypes.byref(inside), ctypes.byref(sh), 0x50000000, 1 << 30, None)
    assert st == api.DCA_E_INVALID and "mask list" in api.dca_last_error()
    st = L.dca_prefill_fused(0x10000000, 0x20000000, 0x30000000, 0x40000000, None, 2048, 512, 128, 1e7, 1.0,
                             ctypes.byref(inside), ctypes.byref(sh), 0x50000000, 1 << 30, None)
    assert st == api.DCA_E_INVALID and "mask list" in api.dca_last_error()


def test_estimate_workspace_size():
    sh = api.make_shape(1, 40, 8, 128, torch.bfloat16)
    S = 1 << 20
    n = api.dca_vs_estimate_workspace_size(S, sh)
    keys = 8 * S * 128 * 2
    table = S * 64 * 8
    scores = 2 * 40 * S * 4
    assert keys + table + scores < n < keys + table + scores + (8 << 20)


def _call_vs_tiles(**over):
    sh = over.pop("shape", api.make_shape(1, 4, 2, 128, torch.bfloat16))
    mask = over.pop("mask", api.dca_vs_mask(0x30000000, 0x31000000, 40, 60))
    args = dict(ws=0x50000000, ws_bytes=1 << 30, seq=4096, C=1024, W=128, head=1, q_tile=4, group=2,
                kt=0x60000000, m=0x61000000, cap=64, n=0x62000000)
    args.update(over)
    return api.lib().dca_debug_vs_tiles(args["ws"], args["ws_bytes"], args["seq"], args["C"], args["W"],
                                        None if mask is None else ctypes.byref(mask), ctypes.byref(sh),
                                        args["head"], args["q_tile"], args["group"], args["kt"], args["m"],
                                        args["cap"], args["n"], None)


@pytest.mark.parametrize("over,status", [
    (dict(mask=None), api.DCA_E_INVALID),
    (dict(head=4), api.DCA_E_INVALID),
    (dict(head=-1), api.DCA_E_INVALID),
    (dict(group=3), api.DCA_E_INVALID),
    (dict(q_tile=5), api.DCA_E_INVALID),                 # not a multiple of the group
    (dict(q_tile=64), api.DCA_E_INVALID),                # past ceil(seq / 64)
    (dict(cap=0), api.DCA_E_INVALID),
    (dict(n=None), api.DCA_E_INVALID),
    (dict(ws_bytes=1 << 16), api.DCA_E_WORKSPACE),
])
def test_vs_tiles_arguments_rejected_before_any_hip_call(over, status):
    assert _call_vs_tiles(**over) == status
    assert api.dca_last_error() != ""


def test_valid_vs_tiles_call_without_gpu_reports_device_error():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call_vs_tiles() == api.DCA_E_DEVICE


def test_status_strings():
    for s in range(5):
        assert api.dca_status_str(s).startswith("DCA_")
    assert api.dca_status_str(99) == "unknown dca_status"


def _included_files(path, seen):
    """Every repository file a source pulls in through #include "..." (recursively)."""
    seen.add(path)
    for name in re.findall(r'^#include "([^"]+)"', open(path).read(), flags=re.M):
        for d in (os.path.dirname(path), os.path.join(ROOT, "include")):
            cand = os.path.normpath(os.path.join(d, name))
            if os.path.exists(cand):
                if cand not in seen:
                    _included_files(cand, seen)
                break
    return seen


def test_stored_traffic_is_keyed_on_every_kernel_source():
    """The bench reports stored HBM traffic only while the kernel's sources are
    unchanged: the digest must cover the .hip file and every header it includes."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for kernel, files in bench.KERNEL_SOURCES.items():
        listed = {os.path.normpath(os.path.join(ROOT, f)) for f in files}
        reached = _included_files(os.path.normpath(os.path.join(ROOT, files[0])), set())
        assert reached == listed, (kernel, sorted(reached ^ listed))
        assert re.fullmatch(r"[0-9a-f]{16}", bench.kernel_source_digest(kernel))


def test_traffic_digest_ignores_comments_but_not_code():
    """Comments and whitespace do not invalidate stored counters; code does,
    including the text of inline asm strings."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    base = 'int a = 1;  // a note\nasm volatile("s_nop 0 // kept");\n'
    assert bench.code_text(base) == bench.code_text('/* header */ int a = 1;\n\n  asm volatile("s_nop 0 // kept");')
    assert bench.code_text(base) != bench.code_text(base.replace("a = 1", "a = 2"))
    assert bench.code_text(base) != bench.code_text(base.replace("s_nop 0 //", "s_nop 1 //"))


@pytest.mark.parametrize("S,nv,ns", [(1000, 20, 30), (4096, 40, 60), (3001, 200, 100)])
def test_bench_sparse_work_count_equals_enumeration(S, nv, ns):
    """The vertical-slash workload's work (bench.vs_active_pairs, a
    convolution over the tile lists) equals the causal pairs of every active
    64x64 tile, enumerated tile by tile with the oracle's activity rule."""
    import importlib.util

    import numpy as np

    from oracle import dca_oracle as O
    from position_extrapolation_amd import synth, workloads

    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    w0 = workloads.get("qwen14b_1m_vs")
    w = workloads.Workload(**{**w0.__dict__, "seq": S, "n_q_heads": 3, "n_kv_heads": 1,
                              "n_vertical": nv, "n_slash": ns})
    vert, slash = synth.vs_mask(w.n_q_heads, S, nv, ns, seed=5)
    n = (S + 63) // 64
    brute = 0
    for h in range(w.n_q_heads):
        for t in range(n):
            kt = torch.arange(t + 1)
            act = O.vs_tile_active(torch.from_numpy(vert[h]), torch.from_numpy(slash[h]),
                                   torch.full_like(kt, t), kt)
            rows = min(64, S - 64 * t)
            for j in kt[act].tolist():
                brute += rows * (rows + 1) // 2 if j == t else rows * 64
    assert bench.vs_active_pairs(w, vert, slash) == brute


@pytest.mark.parametrize("over,status", [
    (dict(), api.DCA_E_DEVICE),                           # valid: reaches the first HIP call
    (dict(q=0x50000000 + 4096), api.DCA_E_INVALID),       # q inside the workspace
    (dict(v=0x50000000 + (1 << 20)), api.DCA_E_INVALID),  # v inside the workspace
])
def test_remap_rejects_inputs_inside_the_workspace(over, status):
    if status == api.DCA_E_DEVICE and torch.cuda.is_available():
        pytest.skip("a GPU is present")
    sh = api.make_shape(1, 2, 1, 64, torch.float32)
    args = dict(q=0x10000000, k=0x20000000, v=0x30000000, ws=0x50000000, ws_bytes=1 << 30)
    args.update(over)
    st = api.lib().dca_remap(args["q"], args["k"], args["v"], 2048, 512, 128, 1e7, 1.0, ctypes.byref(sh),
                             args["ws"], args["ws_bytes"], None)
    assert st == status
    assert api.dca_last_error() != ""


def _call_decode_static(**over):
    sh = over.pop("shape", api.make_shape(1, 4, 2, 64, torch.float32))
    args = dict(q=0x10000000, k=0x20000000, v=0x30000000, out=0x40000000, lse=None, pos=700, seq=2048, C=512,
                W=128, base=1e7, yarn=1.0, ws=0x50000000, ws_bytes=None)
    args.update(over)
    if args["ws_bytes"] is None:     # the key/value cache alone
        args["ws_bytes"] = api.dca_fused_workspace_size(args["seq"], args["C"], args["W"], sh)
    return api.lib().dca_decode_static(args["q"], args["k"], args["v"], args["out"], args["lse"], args["pos"],
                                       args["seq"], args["C"], args["W"], args["base"], args["yarn"],
                                       ctypes.byref(sh), args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(pos=2048), api.DCA_E_INVALID),
    (dict(q=None), api.DCA_E_INVALID),
    (dict(ws_bytes=1 << 12), api.DCA_E_WORKSPACE),         # smaller than the key/value cache
    (dict(out=0x10000000), api.DCA_E_INVALID),             # out aliases q
    # 4 x 64 query heads of d = 128: about 34 MB of scratch, past the 16 MiB array
    (dict(shape=api.make_shape(4, 64, 8, 128, torch.bfloat16)), api.DCA_E_UNSUPPORTED),
])
def test_decode_static_arguments_rejected_before_any_hip_call(over, status):
    assert _call_decode_static(**over) == status
    assert api.dca_last_error() != ""


def test_decode_static_takes_a_cache_only_workspace():
    """Without a GPU a valid call reaches the scratch lookup (the first HIP
    call) and reports DCA_E_DEVICE; dca_decode rejects the same workspace,
    which has no room for its scratch."""
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call_decode_static() == api.DCA_E_DEVICE
    sh = api.make_shape(1, 4, 2, 64, torch.float32)
    nb = api.dca_fused_workspace_size(2048, 512, 128, sh)
    assert _call_decode(ws_bytes=nb) == api.DCA_E_WORKSPACE
