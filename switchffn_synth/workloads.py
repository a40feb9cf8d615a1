"""The synthetic SwitchFFN workloads.

Shapes follow the pages' model families: a Switch-Base-like layer (T5-Base
width, d_model 768), a Switch-Large-like layer (T5-Large width, d_model 1024)
and a Switch-C-shaped layer (d_model 2080, d_ff 6144, 2048 experts), after
"Switch Transformers: Scaling to Trillion Parameter Models with Simple and
Efficient Sparsity", section 3.4 on expert/model/data parallelism (the Table 9
configurations) and section 5 "Experimental Analysis" (base models).  T = batch x sequence
tokens are flattened into one routing group ("Switch Transformer" paper note,
"Implementation Notes -- Batch and Sequence Shape").  Values: x ~ N(0, 1),
router and expert weights ~ N(0, 0.02^2), biases zero unless a test variant
asks for them.  The skewed workload adds a Zipf(s = 1.1) popularity bias to the
router through one constant input feature.
"""
from __future__ import annotations

import dataclasses
from typing import Optional


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens routed together (batch x sequence, flattened)
    d: int          # d_model
    F: int          # d_ff
    N: int          # experts
    CF: float       # capacity factor
    dtype: str      # "fp32" or "bf16": x, W1, b1, W2, b2 and y
    seed: int = 0
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    bias_sigma: float = 0.0       # 0 -> biases are absent (zero)
    zipf_s: Optional[float] = None  # expert popularity ~ (i+1)^-s via a router bias
    zipf_beta: float = 0.5          # strength of that bias, in units of the logit std
    glu: bool = False               # GEGLU experts: W1 [N, 2F, d] and b1 [N, 2F]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def has_bias(self) -> bool:
        return self.bias_sigma != 0.0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def describe(self) -> str:
        return (f"{self.name}: T={self.T} d={self.d} F={self.F} N={self.N} CF={self.CF} "
                f"dtype={self.dtype} seed={self.seed}" + (" geglu" if self.glu else ""))


WORKLOADS = {
    "tiny": Workload("tiny", T=64, d=32, F=64, N=4, CF=1.0, dtype="fp32"),
    "switch_base": Workload("switch_base", T=8192, d=768, F=3072, N=64, CF=1.25, dtype="bf16"),
    "skewed": Workload("skewed", T=16384, d=768, F=3072, N=128, CF=1.0, dtype="bf16",
                       zipf_s=1.1, zipf_beta=0.5),
    "switch_large": Workload("switch_large", T=32768, d=1024, F=4096, N=128, CF=1.25,
                             dtype="bf16"),
    "many_expert": Workload("many_expert", T=65536, d=2080, F=6144, N=2048, CF=1.0,
                            dtype="bf16"),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.replace(**overrides) if overrides else w
