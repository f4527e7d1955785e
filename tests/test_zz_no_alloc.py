"""dca_decode_static, the decode entry point that allocates nothing (its
scratch lives in the library's static device array), against dca_decode
through the C ABI: bit-identical outputs on two calls in a row, the second
with a smaller problem, so that whatever the first call left in the shared
array cannot leak into the second. Also: a problem whose scratch exceeds the
array is rejected before any launch, and the call captured in a HIP graph
replays bit for bit while a smaller eager call overwrites the array between
replays."""

from __future__ import annotations

import sys

import pytest
import torch

from position_extrapolation_amd import api, synth, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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


def _cache(w, prompt, q, k, v):
    """A workspace whose key/value cache holds the rotated keys and values of
    rows [0, prompt), written by a chunked prefill of those rows."""
    shape = api.shape_of(q, k)
    nbytes = api.dca_chunk_workspace_size(w.seq, prompt, w.chunk, w.window, shape)
    ws = api.alloc_workspace(nbytes, DEV)
    o = torch.empty_like(q[:, :, :prompt])
    api.dca_prefill_chunk(q[:, :, :prompt].contiguous(), k[:, :, :prompt].contiguous(),
                          v[:, :, :prompt].contiguous(), o, None, 0, prompt, w.seq, w.chunk, w.window, w.rope_base,
                          w.yarn_scale, None, shape, ws, nbytes)
    return shape, ws, nbytes


def _both(w, pos, q, k, v, shape, ws, nbytes):
    """Decode token pos with dca_decode, then again with dca_decode_static
    on the same cache (the second call stores the same key and value again)."""
    args = (q[:, :, pos].contiguous(), k[:, :, pos].contiguous(), v[:, :, pos].contiguous())
    out_ref = torch.empty_like(args[0])
    lse_ref = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
    out = torch.full_like(args[0], float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    api.dca_decode(*args, out_ref, lse_ref, pos, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, shape, ws,
                   nbytes)
    api.dca_decode_static(*args, out, lse, pos, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, shape, ws,
                          nbytes)
    torch.cuda.synchronize()
    return out, lse, out_ref, lse_ref


@pytest.mark.parametrize("dtype,first,second", [
    # (Hq, Hkv, D, S, C, W, prompt): the second call is smaller in heads, head size and context
    ("bf16", (40, 8, 128, 9000, 2048, 256, 8990), (8, 2, 64, 3000, 1024, 128, 2500)),
    ("f32", (16, 4, 128, 5000, 1024, 128, 4900), (4, 1, 64, 700, 128, 32, 600)),
])
def test_decode_static_equals_decode(dtype, first, second):
    for n, (Hq, Hkv, D, S, C, W, prompt) in enumerate((first, second)):
        say(f"[decode static] call {n + 1}: dtype={dtype} Hq={Hq} Hkv={Hkv} D={D} S={S} C={C} W={W} pos={prompt}")
        w = workloads.Workload("t", 1, Hq, Hkv, D, S, C, W, dtype, 0.5 if dtype == "bf16" else 1.0, True)
        q, k, v = synth.make_qkv(w, seed=40 + n, device=DEV)
        shape, ws, nbytes = _cache(w, prompt, q, k, v)
        out, lse, out_ref, lse_ref = _both(w, prompt, q, k, v, shape, ws, nbytes)
        assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
        say(f"  identical to dca_decode (max |out| {out.abs().max().item():.3e})")


def test_decode_static_needs_only_the_cache():
    """A workspace sized for the keys and values alone (no query section) is
    enough for the static variant; dca_decode needs room for its scratch."""
    w = workloads.Workload("t", 1, 8, 2, 128, 3000, 1024, 128, "bf16", 0.5, True)
    q, k, v = synth.make_qkv(w, seed=44, device=DEV)
    shape = api.shape_of(q, k)
    cache_bytes = api.dca_fused_workspace_size(w.seq, w.chunk, w.window, shape)
    big, ws_big, nb_big = _cache(w, 2999, q, k, v)
    ws = api.alloc_workspace(cache_bytes, DEV)
    ws.copy_(ws_big[:cache_bytes])
    pos = 2999
    args = (q[:, :, pos].contiguous(), k[:, :, pos].contiguous(), v[:, :, pos].contiguous())
    out = torch.empty_like(args[0])
    api.dca_decode_static(*args, out, None, pos, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, shape, ws,
                          cache_bytes)
    out_ref = torch.empty_like(out)
    api.dca_decode(*args, out_ref, None, pos, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, shape, ws_big,
                   nb_big)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    with pytest.raises(api.DcaError) as e:
        api.dca_decode(*args, out_ref, None, pos, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, shape, ws,
                       cache_bytes)
    assert e.value.status == api.DCA_E_WORKSPACE


def test_decode_static_rejects_scratch_past_the_array():
    """4 x 64 query heads of d = 128 need about 34 MB of scratch, more than the
    16 MiB array: DCA_E_UNSUPPORTED before any launch."""
    shape = api.make_shape(4, 64, 8, 128, torch.bfloat16)
    S, C, W = 1024, 256, 64
    nbytes = api.dca_fused_workspace_size(S, C, W, shape)
    ws = api.alloc_workspace(nbytes, DEV)
    q = torch.zeros((4, 64, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((4, 8, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(api.DcaError) as e:
        api.dca_decode_static(q, kv, kv.clone(), out, None, 10, S, C, W, 1e7, 1.0, shape, ws, nbytes)
    assert e.value.status == api.DCA_E_UNSUPPORTED
    assert "static array" in str(e.value)


def _decode_case(Hq, Hkv, D, S, C, W, prompt, seed):
    w = workloads.Workload("t", 1, Hq, Hkv, D, S, C, W, "bf16", 0.5, True)
    q, k, v = synth.make_qkv(w, seed=seed, device=DEV)
    shape = api.shape_of(q, k)
    nbytes = api.dca_chunk_workspace_size(S, prompt, C, W, shape)
    ws = api.alloc_workspace(nbytes, DEV)
    o = torch.empty_like(q[:, :, :prompt])
    api.dca_prefill_chunk(q[:, :, :prompt].contiguous(), k[:, :, :prompt].contiguous(),
                          v[:, :, :prompt].contiguous(), o, None, 0, prompt, S, C, W, w.rope_base, w.yarn_scale,
                          None, shape, ws, nbytes)
    tok = tuple(t[:, :, prompt].contiguous() for t in (q, k, v))
    out = torch.empty_like(tok[0])
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)

    def call():
        api.dca_decode_static(*tok, out, lse, prompt, S, C, W, w.rope_base, w.yarn_scale, shape, ws, nbytes)

    return call, out, lse


def test_decode_static_in_a_graph():
    say("[decode static graph] 40/8 heads, d = 128, pos 8000; between replays an eager 8/2-head, d = 64 call")
    call, out, lse = _decode_case(40, 8, 128, 9000, 2048, 256, 8000, seed=90)
    other, oo, ol = _decode_case(8, 2, 64, 3000, 1024, 128, 2500, seed=91)
    call()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    other()
    torch.cuda.synchronize()
    ref_oo = oo.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        other()                                  # overwrites the shared scratch
        torch.cuda.synchronize()
        assert torch.equal(oo, ref_oo)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {r}"
    say("  three replays identical to the eager call")
