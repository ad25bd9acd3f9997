"""The six synthetic workloads the path is tested and measured on.

Plain data, no arithmetic.  Shapes follow the pages' settings: head size
d_h = d_v = 64 and h = 8 heads (Kernel Zoo "The Running Example" model
parameters), r = 256 random features for d_h = 64 (Performer page sec. 2
"Parameter count and complexity"), DPFP with nu = 2 giving 2*d*nu = 256
features (Kernel Zoo sec. 6.3 / 6.7).  All inputs are i.i.d. N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    wid: int            # workload id, first word of every seed
    name: str
    mode: str           # "bidir" | "causal" | "decode" | "bidir+causal" | "causal_varlen"
    kind: str           # "elu1" | "favor" | "dpfp"
    dtype: str          # "f32" | "bf16"
    B: int
    H: int
    N: int              # tokens per sequence (1 for decode; all packed tokens for causal_varlen)
    d: int = 64
    dv: int = 64
    r: int = 64
    nu: int = 1
    sum_norm: bool = False
    norm: str = "attn"
    favor_scale: bool = False   # multiply q, k by d^-1/4 (softmax temperature)
    eps: float = 1e-6
    layers: int = 1     # decode: layers run back to back, each with its own state
    prefix: int = 0     # decode: tokens of causal prefill that build the state


ELU_SMALL = Workload(0, "elu1_small", "bidir+causal", "elu1", "f32", B=1, H=8, N=256, r=64)
FAVOR_BIDIR = Workload(1, "favor_bidir", "bidir", "favor", "bf16", B=4, H=8, N=4096, r=256,
                       favor_scale=True)
FAVOR_CAUSAL = Workload(2, "favor_causal_prefill", "causal", "favor", "bf16", B=1, H=8,
                        N=65536, r=256, favor_scale=True)
DPFP_CAUSAL = Workload(3, "dpfp_causal", "causal", "dpfp", "f32", B=8, H=8, N=2048, r=256, nu=2,
                       sum_norm=True, norm="none")
FAVOR_DECODE = Workload(4, "favor_decode", "decode", "favor", "bf16", B=256, H=8, N=1, r=256,
                        favor_scale=True, layers=12, prefix=64)

# the causal prefill's 65,536 tokens per head as 32 packed documents of mixed
# length (lengths from inputs.packed_lengths), each starting from zero state
FAVOR_VARLEN = Workload(5, "favor_causal_packed", "causal_varlen", "favor", "bf16", B=32, H=8,
                        N=65536, r=256, favor_scale=True)

ALL = (ELU_SMALL, FAVOR_BIDIR, FAVOR_CAUSAL, DPFP_CAUSAL, FAVOR_DECODE, FAVOR_VARLEN)


def scale_of(w: Workload) -> float:
    return float(w.d) ** -0.25 if w.favor_scale else 1.0
