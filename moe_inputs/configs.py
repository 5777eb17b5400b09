"""The synthetic workloads (Kimi-K2.x-shaped MoE layers and a tiny one).

Shapes: hidden H=7168, intermediate I=2048 (I=256 for the 8-way TP slice),
384 global experts with top-8 routing; a 48-expert local share stands for one
GPU of eight-way expert parallelism.  The tiny layer is the quick parity case.
"""

from __future__ import annotations

import dataclasses
from typing import Optional


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    T: int
    H: int
    I: int
    E_g: int
    E_l: int
    k: int
    seed: int
    layout: str = "indexed"          # indexed | contiguous | masked
    logits: str = "normal"           # router logits: normal | uniform
    expert_begin: int = 0
    scale_normalize: bool = True     # scales *= sqrt(256/K) to keep outputs unit-scale
    block_m: Optional[int] = None    # fixed block_m (None: planner's choice)
    max_m: int = 0                   # masked row budget per expert
    zipf_s: float = 1.2


TINY = WorkloadSpec("tiny_T16_H256_I128_E8_top2", T=16, H=256, I=128, E_g=8, E_l=8, k=2,
                    seed=0, scale_normalize=False, block_m=16)
DECODE = WorkloadSpec("kimi_decode_T64_ep48of384_top8", T=64, H=7168, I=2048, E_g=384,
                      E_l=48, k=8, seed=1)
PREFILL = WorkloadSpec("kimi_prefill_T8192_ep48of384_top8", T=8192, H=7168, I=2048,
                       E_g=384, E_l=48, k=8, seed=2, logits="uniform")
PREFILL_CONTIG = dataclasses.replace(PREFILL, name="kimi_prefill_T8192_ep48of384_top8_contiguous",
                                     layout="contiguous")


def tp_slice(T: int) -> WorkloadSpec:
    return WorkloadSpec(f"kimi_tp8slice_T{T}_all384_I256_top8", T=T, H=7168, I=256, E_g=384,
                        E_l=384, k=8, seed=3 + T)


def masked_zipf(E_l: int) -> WorkloadSpec:
    return WorkloadSpec(f"kimi_masked_zipf_E{E_l}_maxm256", T=0, H=7168, I=2048, E_g=384,
                        E_l=E_l, k=8, seed=40 + E_l, layout="masked", max_m=256)


WORKLOADS = [TINY, DECODE, PREFILL, PREFILL_CONTIG] + [tp_slice(t) for t in (1, 32, 512, 4096)] \
    + [masked_zipf(e) for e in (48, 96, 24)]


def workload_by_name(name: str) -> WorkloadSpec:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)
