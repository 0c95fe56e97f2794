"""The five workloads: shapes, stripe recipe, segment length S and tau.

Each workload is a single causal prefill attention layer with bfloat16
Q/K/V of shape [B, Hq, N, 128] / [B, Hkv, N, 128]. The layer shapes follow
the models named on the S2O summary page (Key points: Llama-3.1-8B at 128K,
ablations on Qwen3-8B at 128K): 32 query heads, 8 KV heads, head dim 128.
The seed of workload n is n.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Tuple

from .stripes import StripeSpec


@dataclass(frozen=True)
class WorkloadConfig:
    cid: int
    name: str
    spec: StripeSpec
    segments: Tuple[int, ...]      # S values (first is the default)
    taus: Tuple[float, ...]        # tau values (first is the default)
    block: int = 64
    variants: Tuple[str, ...] = ("s2o",)
    description: str = ""

    @property
    def segment(self) -> int:
        return self.segments[0]

    @property
    def tau(self) -> float:
        return self.taus[0]


def _mk() -> Dict[int, WorkloadConfig]:
    c = {}
    c[1] = WorkloadConfig(
        1, "tiny_n2048",
        StripeSpec(1, 1, 1, 2048, 128, n_vert=16, n_horiz=0, window=64, seed=1),
        segments=(512,), taus=(0.005,),
        description="tiny causal case: 1x1 head, N=2048, S=512, tau=0.005")
    c[2] = WorkloadConfig(
        2, "llama3_8b_layer_n32k",
        StripeSpec(1, 32, 8, 32768, 128, n_vert=64, n_horiz=32, window=128,
                   seed=2),
        segments=(2048,), taus=(0.005,),
        description="Llama-3.1-8B-shaped layer (32/8 heads, GQA 4:1), N=32768")
    c[3] = WorkloadConfig(
        3, "llama3_8b_layer_n128k",
        StripeSpec(1, 32, 8, 131072, 128, n_vert=256, n_horiz=128,
                   window=128, seed=3),
        segments=(2048,), taus=(0.005, 0.001, 0.020),
        description="Llama-3.1-8B-shaped layer at N=131072; tau sweep")
    c[4] = WorkloadConfig(
        4, "qwen3_8b_layer_n128k",
        StripeSpec(1, 32, 8, 131072, 128, n_vert_range=(16, 256),
                   n_horiz=128, window=128, seed=4),
        segments=(2048, 1024, 4096), taus=(0.010,),
        description="Qwen3-8B-shaped layer at N=131072, heterogeneous heads; "
                    "S sweep")
    c[5] = WorkloadConfig(
        5, "ablation_b4_n64k",
        StripeSpec(4, 32, 8, 65536, 128, n_vert=128, n_horiz=64, window=128,
                   seed=5),
        segments=(2048,), taus=(0.005,),
        variants=("s2o", "kv_perm_only", "tau0"),
        description="batch 4 at N=65536: full S2O, KV-permutation only, "
                    "tau=0 (dense)")
    return c


CONFIGS: Dict[int, WorkloadConfig] = _mk()


def get_config(cid: int) -> WorkloadConfig:
    return CONFIGS[int(cid)]
