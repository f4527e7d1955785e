"""The benchmark's host-side arithmetic, on the CPU: the pre-pass's
algorithmic bytes against the per-token figures of the RoPE/DCA pre-pass
(read q and k once, write three rotated query variants and the rotated
keys), the bytes it moves beyond them, the clock line's arithmetic, and a
clock sampler that has no source reporting why instead of a number."""

from __future__ import annotations

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from position_extrapolation_amd import workloads  # noqa: E402


@pytest.mark.parametrize("name,per_token", [("qwen7b_32k", 30720), ("qwen7b_128k", 30720), ("qwen14b_1m", 45056),
                                            ("qwen14b_1m_vs", 45056)])
def test_remap_algorithmic_bytes_per_token(name, per_token):
    w = workloads.get(name)
    # bf16: (Hq + Hkv) d 2 read + (3 Hq + Hkv) d 2 written, per token
    assert bench.remap_bytes(w) == per_token * w.seq * w.batch
    assert per_token == ((w.n_q_heads + w.n_kv_heads) + (3 * w.n_q_heads + w.n_kv_heads)) * w.head_dim * 2


def test_remap_extra_bytes():
    w = workloads.get("qwen14b_1m")
    extra = bench.remap_extra_bytes(w)
    assert extra["value_relayout"] == 2 * 8 * 128 * 2 * (1 << 20)          # read and write v once: 4 GiB
    assert extra["cos_sin_table"] == (262144 + 32768) * 64 * 8              # float2 per (position, pair)


def test_clock_line():
    line = bench.clock_line({"mhz_mean": 2000.0, "source": "test"}, 1048.576)
    assert line["bf16_peak_at_clock_tflops"] == pytest.approx(256 * 4096 * 2000e6 / 1e12, abs=0.05)
    assert line["attention_frac_at_clock"] == pytest.approx(0.5, abs=1e-4)
    assert bench.clock_line({"mhz_mean": None, "error": "x"}, 1000.0) == {"mhz_mean": None, "error": "x"}


def test_clock_sampler_without_a_source_reports_why():
    c = bench.ClockSampler(period=0.01)
    c._read = None          # as on a machine where neither amdsmi nor the DPM table can be read
    res = c.start().stop()
    assert res["mhz_mean"] is None and res.get("error")
