#!/usr/bin/env python3
"""Benchmark of DCA prefill attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra] [--no-cpu]

A step is one pass of the whole path over one batch of synthetic input:
the remap pre-pass (cos/sin table + rotated query variants, rotated keys and
value re-layout), the vertical-slash tile index for sparse workloads, and the
attention kernel -- the same launches dca_prefill makes, issued through its
stage entry points so that HIP events on the launch stream time each kernel.

Prints ONE JSON line. `value` is whole-step TFLOP/s on the 1M-token Qwen2.5-14B
layer shape (dense causal work 4 d Hq S(S+1)/2); `roofline` reports the
attention kernel against the bf16 dense MFMA peak; `step_ms_median` and
`step_ms_min` are the median and fastest step by the stream events (the mean,
`ms_per_step`, is the host clock over the timed steps); `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload; `extra` holds the other
measured workloads: 128K dense, 1M vertical-slash, the 1M sequence as a
chunked prefill in 32,768-row blocks, decode at a 1M context, the 1M path
with the query rotation fused into the attention kernel, the online
vertical-slash estimate at 1M, and the online flow end to end (estimate,
then the sparse prefill with the estimated mask) beside the dense step.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from position_extrapolation_amd import api, synth, workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 matrix (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def remap_bytes(w) -> float:
    """Algorithmic bytes of the RoPE/DCA pre-pass: read q and k once, write the
    three rotated query variants and the rotated keys,
    S B (Hq + Hkv) d e + S B (3 Hq + Hkv) d e (45,056 B per token at the 1M
    Qwen2.5-14B shape)."""
    e = 2 if w.dtype == "bf16" else 4
    per_tok = (w.n_q_heads + w.n_kv_heads) * w.head_dim * e               # read
    per_tok += (3 * w.n_q_heads + w.n_kv_heads) * w.head_dim * e          # write
    return float(per_tok * w.seq * w.batch)


def remap_extra_bytes(w) -> dict:
    """Bytes the pre-pass moves beyond the algorithmic ones, by design: the
    value re-layout into the attention kernel's operand order (read and write
    v once) and the float32 cos/sin table for positions [0, C + W)."""
    e = 2 if w.dtype == "bf16" else 4
    return {"value_relayout": float(2 * w.n_kv_heads * w.head_dim * e * w.seq * w.batch),
            "cos_sin_table": float((w.chunk + w.window) * (w.head_dim // 2) * 8)}


class ClockSampler:
    """The GPU's graphics clock (MHz), sampled every `period` seconds by a
    host thread while a timed region runs: from amdsmi, else from the sysfs
    DPM table (the level marked current). stop() returns the summary, or a
    record of why no clock could be read."""

    def __init__(self, period: float = 0.05):
        import threading

        self.period = period
        self.samples = []
        self.power = []
        self.source = None
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._read = self._open()

    def _open(self):
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            h = handles[0] if len(handles) == 1 else self._match(amdsmi, handles)
            if h is None:
                raise RuntimeError(f"{len(handles)} GPUs listed, none matched cuda:0's PCI address")
            amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
            self.source = "amdsmi gfx clock"

            def read():
                clk = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"]
                try:
                    pw = amdsmi.amdsmi_get_power_info(h).get("current_socket_power")
                except Exception:
                    pw = None
                return clk, pw
            return read
        except Exception as e:              # no amdsmi, no permission, no match
            self.error = f"amdsmi: {e}"
        import glob

        for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            try:
                open(path).read()
            except OSError:
                continue
            self.source = f"sysfs {path}"

            def read(path=path):
                for line in open(path):
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz")), None
                return None, None
            return read
        return None

    @staticmethod
    def _match(amdsmi, handles):
        props = torch.cuda.get_device_properties(0)
        bus = getattr(props, "pci_bus_id", None)
        if bus is None:
            return None
        for h in handles:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)        # "dddd:bb:dd.f"
            if int(bdf.split(":")[1], 16) == int(bus):
                return h
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                clk, pw = self._read()
                if clk:
                    self.samples.append(float(clk))
                if pw:
                    self.power.append(float(pw))
            except Exception as e:
                self.error = str(e)
            self._stop.wait(self.period)

    def start(self):
        import threading

        if self._read is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if not self.samples:
            return {"mhz_mean": None, "source": self.source, "error": self.error or "no clock source"}
        xs = sorted(self.samples)
        res = {"mhz_mean": round(sum(xs) / len(xs), 1), "mhz_median": xs[len(xs) // 2], "mhz_min": xs[0],
               "mhz_max": xs[-1], "samples": len(xs), "source": self.source}
        if self.power:
            res["socket_power_w_mean"] = round(sum(self.power) / len(self.power), 1)
        return res


def vs_active_pairs(w, vert, slash) -> float:
    """Causal (query, key) pairs inside active 64x64 tiles, summed over heads:
    the attention work of a vertical-slash workload (pairs x 4 d flops).

    Per query tile t the active key tiles are A = {kt in VT, kt <= t} united
    with B = {t - delta : delta in D, delta <= t}; |A u B| = |A| + |B| - |A n B|
    and |A n B| = sum_delta 1_D(delta) 1_VT(t - delta) is a convolution."""
    from scipy.signal import fftconvolve

    S = w.seq
    n = (S + 63) // 64
    t = np.arange(n)
    rows_in = np.minimum(S - 64 * t, 64).astype(np.float64)   # valid rows of query tile t
    total = 0.0
    for h in range(w.n_q_heads):
        ind_v = np.zeros(n)
        ind_v[np.unique(np.asarray(vert[h], dtype=np.int64) // 64)] = 1
        sl = np.asarray(slash[h], dtype=np.int64)
        a = sl // 64
        dset = np.unique(np.concatenate([a, (a + 1)[sl % 64 != 0]]))
        ind_d = np.zeros(n)
        ind_d[dset[dset < n]] = 1
        n_a = np.cumsum(ind_v)                                  # |A|
        n_b = np.cumsum(ind_d)                                  # |B|
        n_ab = np.rint(fftconvolve(ind_d, ind_v)[:n])           # |A n B|
        count = n_a + n_b - n_ab
        diag = np.maximum(ind_v, ind_d[0])                      # tile (t, t) active
        total += float((rows_in * 64 * (count - diag) + diag * rows_in * (rows_in + 1) / 2).sum())
    return total * w.batch


class Runner:
    """Holds device inputs and workspace for one workload; runs one step."""

    def __init__(self, w, device, seed=0):
        self.w = w
        log(f"[bench] generating inputs for {w.name}")
        self.q, self.k, self.v = synth.make_qkv(w, seed=seed, device=device)
        self.shape = api.shape_of(self.q, self.k)
        self.vert = self.slash = None
        self.mask = None
        if w.sparse:
            vn, sn = synth.vs_mask(w.n_q_heads, w.seq, w.n_vertical, w.n_slash, seed=seed)
            self.vert_host, self.slash_host = vn, sn
            self.vert = torch.from_numpy(vn).to(device)
            self.slash = torch.from_numpy(sn).to(device)
            self.mask = api.make_mask(self.vert, self.slash)
        self.nbytes = api.dca_workspace_size(w.seq, w.chunk, w.window, self.shape, self.mask)
        self.ws = api.alloc_workspace(self.nbytes, device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=device)
        self.ev = None

    def step(self, events=None):
        w = self.w
        if events is not None:
            events[0].record()
        api.dca_remap(self.q, self.k, self.v, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, self.shape,
                      self.ws, self.nbytes)
        if events is not None:
            events[1].record()
        if self.mask is not None:
            api.dca_vs_index(w.seq, w.chunk, w.window, self.mask, self.shape, self.ws, self.nbytes)
        if events is not None:
            events[2].record()
        api.dca_attention(self.out, self.lse, w.seq, w.chunk, w.window, self.mask, self.shape, self.ws,
                          self.nbytes)
        if events is not None:
            events[3].record()

    def time(self, steps, warmup):
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        clock = ClockSampler().start()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(evs[i])
            log(f"[bench] {self.w.name}: step {i + 1}/{steps} enqueued")
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        self.clock = clock.stop()
        remap_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
        index_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
        attn_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / steps
        self.step_event_ms = sorted(e[0].elapsed_time(e[3]) for e in evs)
        return wall * 1e3 / steps, remap_ms, index_ms, attn_ms

    def work_flops(self):
        w = self.w
        if not w.sparse:
            return w.dense_flops()
        return 4.0 * w.head_dim * vs_active_pairs(w, self.vert_host, self.slash_host)


def measure(name, steps, warmup, device):
    w = workloads.get(name)
    r = Runner(w, device)
    ms, remap_ms, index_ms, attn_ms = r.time(steps, warmup)
    flops = r.work_flops()
    res = {
        "workload": name, "ms_per_step": ms, "tflops": flops / (ms * 1e-3) / 1e12,
        "attention_ms": attn_ms, "attention_tflops": flops / (attn_ms * 1e-3) / 1e12,
        "remap_ms": remap_ms, "remap_gbs": remap_bytes(w) / (remap_ms * 1e-3) / 1e9,
        "flops": flops,
        # per-step times from the stream events (the mean above is the host clock over all steps)
        "step_ms_median": statistics.median(r.step_event_ms), "step_ms_min": r.step_event_ms[0],
    }
    # the attention kernel against the dense MFMA peak of its dtype (for a
    # vertical-slash workload: its actual work, the pairs of active tiles)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    res["attention_frac"] = res["attention_tflops"] / peak
    res["clock"] = clock_line(r.clock, res["attention_tflops"])
    if w.sparse:
        res["vs_index_ms"] = index_ms
        res["dense_equiv_tflops"] = w.dense_flops() / (ms * 1e-3) / 1e12
        res["active_fraction"] = flops / w.dense_flops()
    log(f"[bench] {name}: {json.dumps(res)}")
    del r
    torch.cuda.empty_cache()
    return w, res


def clock_line(clock, achieved_tflops):
    """The sampled clock beside the roofline: the bf16 dense MFMA rate at that
    clock (256 CUs x 4096 flop per clock) and the attention kernel's share of
    it, so that a gap between two runs reads as clock or as code."""
    res = dict(clock)
    mhz = clock.get("mhz_mean")
    if mhz:
        at_clock = 256 * 4096 * mhz * 1e6 / 1e12
        res["bf16_peak_at_clock_tflops"] = round(at_clock, 1)
        res["attention_frac_at_clock"] = round(achieved_tflops / at_clock, 4)
    return res


def measure_chunked(name, chunk, steps, warmup, device):
    """Chunked prefill [mizuki, Chunked Prefill]: the whole sequence of the
    workload as blocks of `chunk` rows, each one dca_prefill_chunk call on a
    workspace that holds every key but only one block's query variants. The
    blocks' q, k and v are resident in HBM before timing."""
    w = workloads.get(name)
    log(f"[bench] generating inputs for {name}, blocks of {chunk} rows")
    q, k, v = synth.make_qkv(w, seed=0, device=device)
    shape = api.shape_of(q, k)
    blocks = []
    for q0 in range(0, w.seq, chunk):
        n = min(chunk, w.seq - q0)
        blocks.append((q0, n, q[:, :, q0:q0 + n].contiguous(), k[:, :, q0:q0 + n].contiguous(),
                       v[:, :, q0:q0 + n].contiguous()))
    del q, k, v
    nbytes = api.dca_chunk_workspace_size(w.seq, min(chunk, w.seq), w.chunk, w.window, shape)
    ws = api.alloc_workspace(nbytes, device)
    outs = [torch.empty_like(b[2]) for b in blocks]

    def run():
        for (q0, n, qc, kc, vc), oc in zip(blocks, outs):
            api.dca_prefill_chunk(qc, kc, vc, oc, None, q0, n, w.seq, w.chunk, w.window, w.rope_base,
                                  w.yarn_scale, None, shape, ws, nbytes)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        run()
        log(f"[bench] {name} in blocks of {chunk}: pass {i + 1}/{steps} enqueued")
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    res = {"workload": f"{name}_chunked{chunk}", "block_rows": chunk, "calls_per_step": len(blocks),
           "ms_per_step": ms, "tflops": w.dense_flops() / (ms * 1e-3) / 1e12,
           "workspace_bytes": nbytes, "whole_sequence_workspace_bytes": api.dca_workspace_size(
               w.seq, w.chunk, w.window, shape)}
    log(f"[bench] {json.dumps(res)}")
    del blocks, outs, ws
    torch.cuda.empty_cache()
    return res


def measure_fused(name, device):
    """The whole path with the query rotation fused into the attention kernel
    (dca_prefill_fused): the pre-pass writes keys and values only."""
    w = workloads.get(name)
    log(f"[bench] generating inputs for {name}, fused query rotation")
    q, k, v = synth.make_qkv(w, seed=0, device=device)
    shape = api.shape_of(q, k)
    nbytes = api.dca_fused_workspace_size(w.seq, w.chunk, w.window, shape)
    ws = api.alloc_workspace(nbytes, device)
    out = torch.empty_like(q)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    api.dca_prefill_fused(q, k, v, out, None, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, None, shape,
                          ws, nbytes)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    res = {"workload": f"{name}_fused_rotation", "ms_per_step": ms, "tflops": w.dense_flops() / (ms * 1e-3) / 1e12,
           "workspace_bytes": nbytes,
           "materialized_workspace_bytes": api.dca_workspace_size(w.seq, w.chunk, w.window, shape)}
    log(f"[bench] {json.dumps(res)}")
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return res


def measure_estimate(name, device, n_vertical=1000, n_slash=2000, forced=64, n_last=64):
    """Online vertical-slash estimation (dca_vs_estimate) on the workload's
    shape: the last 64 query rows under continuous positions, per-head
    budgets of the 1M vertical-slash workload."""
    w = workloads.get(name)
    log(f"[bench] generating inputs for {name} vertical-slash estimate")
    q, k, v = synth.make_qkv(w, seed=0, device=device)
    del v
    shape = api.shape_of(q, k)
    nbytes = api.dca_vs_estimate_workspace_size(w.seq, shape)
    ws = api.alloc_workspace(nbytes, device)
    vert = torch.empty((w.n_q_heads, n_vertical), dtype=torch.int32, device=device)
    slash = torch.empty((w.n_q_heads, n_slash), dtype=torch.int32, device=device)

    def run():
        api.dca_vs_estimate(q, k, w.seq, n_last, w.rope_base, w.yarn_scale, n_vertical, n_slash, forced, shape,
                            vert, slash, None, None, ws, nbytes)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    # selection work: the scored rows' causal logits, twice (statistics, then sums)
    flops = 2 * 4.0 * w.head_dim * w.n_q_heads * n_last * w.seq
    res = {"workload": f"{name}_vs_estimate", "ms": ms, "n_last": n_last, "n_vertical": n_vertical,
           "n_slash": n_slash, "tflops": flops / (ms * 1e-3) / 1e12}
    log(f"[bench] {json.dumps(res)}")
    del q, k, ws
    torch.cuda.empty_cache()
    return res


def measure_online_vs(name, device, dense_step_ms=None, n_vertical=1000, n_slash=2000, forced=64, n_last=64):
    """The online vertical-slash flow on the workload's shape [mizuki,
    MInference sections]: each head's columns and offsets estimated from the
    last 64 rows under continuous positions (dca_vs_estimate), then the DCA
    prefill with that mask (dca_prefill: remap, tile index, sparse attention),
    timed as one step. The work is the active-tile pairs of the estimated
    mask; the dense prefill step of the same run is the comparison."""
    w = workloads.get(name)
    log(f"[bench] generating inputs for {name} online vertical-slash")
    q, k, v = synth.make_qkv(w, seed=0, device=device)
    shape = api.shape_of(q, k)
    eb = api.dca_vs_estimate_workspace_size(w.seq, shape)
    ews = api.alloc_workspace(eb, device)
    vert = torch.empty((w.n_q_heads, n_vertical), dtype=torch.int32, device=device)
    slash = torch.empty((w.n_q_heads, n_slash), dtype=torch.int32, device=device)
    mask = api.make_mask(vert, slash)
    pb = api.dca_workspace_size(w.seq, w.chunk, w.window, shape, mask)
    pws = api.alloc_workspace(pb, device)
    out = torch.empty_like(q)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        api.dca_vs_estimate(q, k, w.seq, n_last, w.rope_base, w.yarn_scale, n_vertical, n_slash, forced, shape,
                            vert, slash, None, None, ews, eb)
        if ev is not None:
            ev[1].record()
        api.dca_prefill(q, k, v, out, None, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, mask, shape,
                        pws, pb)
        if ev is not None:
            ev[2].record()

    step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    step(ev)
    torch.cuda.synchronize()
    est_ms, pre_ms = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
    ms = est_ms + pre_ms
    flops = 4.0 * w.head_dim * vs_active_pairs(w, vert.cpu().numpy(), slash.cpu().numpy())
    res = {"workload": f"{name}_online_vs", "n_vertical": n_vertical, "n_slash": n_slash, "ms_per_step": ms,
           "estimate_ms": est_ms, "prefill_ms": pre_ms, "active_fraction": flops / w.dense_flops(),
           "tflops": flops / (ms * 1e-3) / 1e12, "dense_equiv_tflops": w.dense_flops() / (ms * 1e-3) / 1e12}
    if dense_step_ms is not None:
        res["speedup_vs_dense_step"] = dense_step_ms / ms
    log(f"[bench] {json.dumps(res)}")
    del q, k, v, ews, pws, out
    torch.cuda.empty_cache()
    return res


def measure_decode(name, steps, device):
    """DCA decode of the last `steps` tokens of the workload's sequence, one
    dca_decode call each, against the key/value cache of everything before
    them (filled by the remap pre-pass). Bound by HBM: each call reads the
    cache once, (pos + 1) keys and values per KV head."""
    w = workloads.get(name)
    log(f"[bench] generating inputs for {name} decode")
    q, k, v = synth.make_qkv(w, seed=0, device=device)
    shape = api.shape_of(q, k)
    nbytes = api.dca_workspace_size(w.seq, w.chunk, w.window, shape)
    ws = api.alloc_workspace(nbytes, device)
    api.dca_remap(q, k, v, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale, shape, ws, nbytes)
    first = w.seq - steps
    toks = [(pos, q[:, :, pos].contiguous(), k[:, :, pos].contiguous(), v[:, :, pos].contiguous())
            for pos in range(first, w.seq)]
    del q, k, v
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=toks[0][1].dtype, device=device)

    def run():
        for pos, qt, kt, vt in toks:
            api.dca_decode(qt, kt, vt, out, None, pos, w.seq, w.chunk, w.window, w.rope_base, w.yarn_scale,
                           shape, ws, nbytes)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    esize = 2 if w.dtype == "bf16" else 4
    cache_bytes = np.mean([(pos + 1) * w.batch * w.n_kv_heads * w.head_dim * 2 * esize for pos, *_ in toks])
    res = {"workload": f"{name}_decode", "tokens": steps, "context": w.seq, "ms_per_token": ms,
           "cache_bytes_per_token": cache_bytes, "hbm_gbs": cache_bytes / (ms * 1e-3) / 1e9,
           "hbm_frac": cache_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    log(f"[bench] {json.dumps(res)}")
    del toks, ws
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(name, n_rows=64, seed=0):
    """The CPU oracle, as it stands, on a bounded sample of the workload:
    n_rows query rows spread evenly over the sequence, every head. Reported in
    the benchmark's unit (TFLOP/s of the sampled rows' causal work, 4 d flops
    per causal pair and head), with the time a full prefill would take at the
    same rate (time x total pairs / sampled pairs), labelled as such."""
    from oracle import dca_oracle as O

    w = workloads.get(name)
    q, k, v = synth.make_qkv(w, seed=seed, device="cuda:0")
    rows = torch.linspace(0, w.seq - 1, n_rows).round().long()
    q_rows = q[:, :, rows.to(q.device)].cpu()
    kc, vc = k.cpu(), v.cpu()
    del q, k, v
    torch.cuda.empty_cache()
    threads = torch.get_num_threads()
    t0 = time.perf_counter()
    O.dca_prefill_rows(q_rows, rows, kc, vc, w.chunk, w.window, w.rope_base, w.yarn_scale)
    dt = time.perf_counter() - t0
    pairs = float((rows + 1).sum()) * w.n_q_heads * w.batch
    total_pairs = w.n_q_heads * w.batch * w.seq * (w.seq + 1) / 2.0
    flops = 4.0 * w.head_dim * pairs
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_rows} query rows evenly spread over {w.name} (S={w.seq}), all {w.n_q_heads} "
                      f"heads, float64 torch-CPU oracle on {threads} threads, {dt:.1f} s",
            "seconds": round(dt, 2), "causal_pairs": pairs, "cpu_model": cpu_model(),
            "host_logical_cpus": os.cpu_count(), "affinity_cpus": affinity,
            "extrapolated_full_prefill_s": round(dt * total_pairs / pairs, 1),
            "extrapolation": "sample time x total causal pairs / sampled causal pairs (not measured)"}


# the files each kernel is compiled from: its source and every header it includes
KERNEL_SOURCES = {
    "attention": ["position_extrapolation_amd/csrc/attention.hip", "position_extrapolation_amd/csrc/tile_math.h",
                  "position_extrapolation_amd/csrc/frag.h", "position_extrapolation_amd/csrc/dca_internal.h",
                  "include/dca.h"],
    "remap": ["position_extrapolation_amd/csrc/remap.hip", "position_extrapolation_amd/csrc/frag.h",
              "position_extrapolation_amd/csrc/dca_internal.h", "include/dca.h"],
}


def code_text(src: str) -> str:
    """C/C++ source reduced to its code: comments dropped, whitespace runs
    collapsed to one space, string literals (inline asm) kept as written."""
    import re

    tok = re.compile(r'("(?:\\.|[^"\\\n])*")|/\*.*?\*/|//[^\n]*', re.S)
    code = tok.sub(lambda mt: mt.group(1) if mt.group(1) else " ", src)
    return " ".join(code.split())


def kernel_source_digest(kernel: str) -> str:
    """First 16 hex digits of the SHA-256 over the code of a kernel's source
    files, in order (comment-only edits leave it unchanged)."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(code_text(open(os.path.join(ROOT, f)).read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel_key: str = ""):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes (profiles/traffic.json, already scaled by the copy calibration), or
    None when the kernel's sources (its file or any header it includes) have
    changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("traffic", {}).get(workload + kernel_key)
    if rec is None:
        return None
    kernel = "remap" if kernel_key == ":remap" else "attention"
    if kernel_source_digest(kernel) != rec.get("sources_sha256_16"):
        return None
    return {"total": rec["read_bytes"] + rec["written_bytes"], "read": rec["read_bytes"],
            "written": rec["written_bytes"]}


def copy_calibration(mib: int, device):
    """A plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it
    converts those counters into bytes for the attention kernel."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="qwen14b_1m")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra workloads (128K, vertical-slash, chunked, decode, fused, estimate, "
                         "online vertical-slash)")
    ap.add_argument("--only", choices=["decode", "chunked", "fused", "estimate", "online"],
                    help="run just this 1M measurement and print its JSON (for profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=64)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path is single-GPU (multi-GPU sharding is a design "
              "note, not implemented); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, dev)
        return
    if args.only:
        run = {"decode": lambda: measure_decode("qwen14b_1m", 64, dev),
               "chunked": lambda: measure_chunked("qwen14b_1m", 32768, 1, 0, dev),
               "fused": lambda: measure_fused("qwen14b_1m", dev),
               "estimate": lambda: measure_estimate("qwen14b_1m", dev),
               "online": lambda: measure_online_vs("qwen14b_1m", dev)}[args.only]
        print(json.dumps(run()), flush=True)
        return
    api.lib()

    w, main_res = measure(args.workload, args.steps, args.warmup, dev)
    extra = []
    if not args.no_extra:
        for name in ("qwen7b_128k", "qwen14b_1m_vs"):
            if name != args.workload:
                # 128K: 30 steps (3 s), long enough for the 50 ms clock samples
                # to cover the load and not its edges
                steps = 30 if name == "qwen7b_128k" else min(5, max(1, args.steps))
                extra.append(measure(name, steps, 3 if name == "qwen7b_128k" else 1, dev)[1])
        extra.append(measure_chunked("qwen14b_1m", 32768, 1, 1, dev))
        extra.append(measure_decode("qwen14b_1m", 64, dev))
        extra.append(measure_fused("qwen14b_1m", dev))
        extra.append(measure_estimate("qwen14b_1m", dev))
        extra.append(measure_online_vs("qwen14b_1m", dev,
                                       main_res["ms_per_step"] if w.name == "qwen14b_1m" else None))

    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = main_res["attention_tflops"]
    traffic = measured_traffic(w.name)
    remap_traffic = measured_traffic(w.name, ":remap")
    result = {
        "metric": "DCA prefill attention TFLOP/s (1M tokens, Qwen2.5-14B layer shape, one MI355X)",
        "value": round(main_res["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1)*0.5 bf16 q/k/v)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "seq_len": w.seq,
                   "chunk": w.chunk, "window": w.window, "rope_base": w.rope_base,
                   "yarn_scale": round(w.yarn_scale, 10), "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100.0 * main_res["tflops"] / peak, 2),
        "roofline": {"kernel": "dca_attention_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": None if traffic is None else traffic["total"],
                     "traffic_detail": traffic},
        "remap": {"kernel": "remap_kernel", "bound": "hbm", "ms": round(main_res["remap_ms"], 3),
                  "achieved": round(main_res["remap_gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                  "frac": round(main_res["remap_gbs"] / PEAK_HBM_GBS, 4),
                  "algorithmic_bytes": remap_bytes(w),
                  # moved as well, by design, and not counted in `achieved`
                  "extra_bytes": remap_extra_bytes(w),
                  "traffic": None if remap_traffic is None else remap_traffic["total"]},
        "clock": main_res["clock"],
        "attention_ms": round(main_res["attention_ms"], 3),
        "step_ms_median": round(main_res["step_ms_median"], 3),
        "step_ms_min": round(main_res["step_ms_min"], 3),
        "extra": extra,
    }
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w.name, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
