"""The DCA prefill workloads: the shapes the parity tests and the benchmark run.

Shapes follow the Qwen2.5 layer geometry the pages give (GQA at every size,
RoPE base 1e7) [yudong §3], with chunk C and local window W per workload and
the YaRN logit temperature 0.1 ln(S / C) + 1 [mizuki, DCA + YaRN].
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq: int
    chunk: int
    window: int
    dtype: str                 # "f32" or "bf16": the dtype of q, k, v and out
    input_scale: float         # inputs are N(0, 1) * input_scale, rounded to dtype
    yarn: bool                 # apply the YaRN logit temperature
    rope_base: float = 1.0e7
    n_vertical: int = 0        # vertical-slash mask sizes per head (0 = dense)
    n_slash: int = 0
    oracle_rows: int | None = None   # sampled query rows for parity (None = all)
    notes: str = field(default="", compare=False)

    @property
    def yarn_scale(self) -> float:
        if not self.yarn:
            return 1.0
        return max(1.0, 0.1 * math.log(self.seq / self.chunk) + 1.0)

    @property
    def sparse(self) -> bool:
        return self.n_vertical > 0 or self.n_slash > 0

    def dense_flops(self) -> float:
        """4 d flops per causal pair and query head (one QK^T and one PV
        multiply-add per head dimension)."""
        S = self.seq
        return 4.0 * self.head_dim * self.n_q_heads * self.batch * S * (S + 1) / 2.0


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_2k_f32", 1, 2, 1, 64, 2048, 512, 128, "f32", 1.0, False,
                 oracle_rows=None, notes="tiny DCA, fp32, every row checked"),
        Workload("qwen7b_32k", 1, 28, 4, 128, 32768, 8192, 1024, "bf16", 0.5, True,
                 oracle_rows=1024, notes="Qwen2.5-7B layer shape at 32K"),
        Workload("qwen7b_128k", 1, 28, 4, 128, 131072, 32768, 4096, "bf16", 0.5, True,
                 oracle_rows=256, notes="Qwen2.5-7B layer shape at 128K"),
        Workload("qwen14b_1m", 1, 40, 8, 128, 1048576, 262144, 32768, "bf16", 0.5, True,
                 oracle_rows=256, notes="Qwen2.5-14B layer shape at 1M"),
        Workload("qwen14b_1m_vs", 1, 40, 8, 128, 1048576, 262144, 32768, "bf16", 0.5, True,
                 n_vertical=1000, n_slash=2000, oracle_rows=256,
                 notes="1M + vertical-slash block-sparse mask, 64x64 tiles"),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
