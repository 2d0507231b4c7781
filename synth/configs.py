"""The LayerAdam workloads, as recipes for seeded synthetic inputs.

Each workload is one decoder layer (or one flat tensor) with the tensor sizes
of a public model family, random values of stated distributions, R gradient
replicas and the AdamW hyperparameters of one step. No weights or data are
read: the layers stand in for the real Qwen layers that SlideDP fine-tunes
("SlideDP: Scaling Host-Resident LLM Fine-Tuning Across Multiple GPUs",
"实验结果", results) and for the 101M-488M and 800M-parameter single layers of
its host micro-benchmarks (same page, "研究动机", motivation, and the figure
captions of "论文图表").

Distributions: N(0, s) has standard deviation s; U(a, b) is uniform.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

HYPER = dict(lr=1e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    tensors: Tuple[Tuple[str, int], ...]    # (name, numel)
    replicas: int
    grad_dtype: str                          # "bf16" | "fp16"
    step: int
    master_std: float = 0.02
    m_std: Optional[float] = 1e-4            # None: m = 0
    v_high: Optional[float] = 1e-6           # None: v = 0; else U(0, v_high)
    grad_std: float = 1e-3
    grad_prescale: float = 1.0               # multiplies the sample (loss scale)
    unscale: float = 1.0                     # passed to the update
    outlier_prob: float = 0.0                # per element, per replica
    outlier_mult: float = 1.0
    log_scale_range: Optional[Tuple[float, float]] = None  # per-tensor 10^U(a,b)
    with_flag: bool = False
    hyper: Dict[str, float] = field(default_factory=lambda: dict(HYPER))

    @property
    def numel(self) -> int:
        return sum(n for _, n in self.tensors)

    @property
    def bytes_per_param(self) -> int:
        # R gradient reads (2 B each) + master/m/v read and written (24 B)
        # + the BF16 weight written (2 B)
        return 2 * self.replicas + 26

    @property
    def traffic_bytes(self) -> int:
        return self.bytes_per_param * self.numel


def _decoder(h: int, ffn: int, q_dim: int, kv_dim: int):
    return (("q_proj", h * q_dim), ("k_proj", h * kv_dim), ("v_proj", h * kv_dim),
            ("o_proj", q_dim * h), ("gate_proj", h * ffn), ("up_proj", h * ffn),
            ("down_proj", ffn * h), ("input_layernorm", h),
            ("post_attention_layernorm", h))


WORKLOADS: Dict[str, Workload] = {
    # four FP32 tensors, one BF16 replica, zero moments, the first step
    "tiny": Workload(
        name="tiny", seed=1000,
        tensors=(("w0", 256 * 256), ("w1", 256 * 64), ("w2", 256 * 64),
                 ("w3", 688 * 256)),
        replicas=1, grad_dtype="bf16", step=1, m_std=None, v_high=None),
    # Qwen3-4B decoder layer: h=2560, FFN 9728, 32 q heads x 128, 8 kv heads
    "qwen3_4b_layer": Workload(
        name="qwen3_4b_layer", seed=1001, tensors=_decoder(2560, 9728, 4096, 1024),
        replicas=4, grad_dtype="bf16", step=10),
    # Qwen3-14B decoder layer: h=5120, FFN 17408, 40 q heads x 128, 8 kv heads;
    # 1 % of gradient entries x100
    "qwen3_14b_layer": Workload(
        name="qwen3_14b_layer", seed=1002, tensors=_decoder(5120, 17408, 5120, 1024),
        replicas=8, grad_dtype="bf16", step=100, outlier_prob=0.01,
        outlier_mult=100.0),
    # one flat FP32 tensor with an odd tail; FP16 gradients carry a x1024 loss
    # scale that the update removes; the overflow flag is on and must stay 0
    "flat_800m": Workload(
        name="flat_800m", seed=1003, tensors=(("flat", 800_000_003),),
        replicas=2, grad_dtype="fp16", step=1000, grad_prescale=1024.0,
        unscale=1.0 / 1024.0, with_flag=True),
    # Qwen2.5-72B decoder layer: h=8192, FFN 29568, 64 q heads x 128, 8 kv
    # heads; gradient scale per tensor 10^U(-5,-1)
    "qwen25_72b_layer": Workload(
        name="qwen25_72b_layer", seed=1004, tensors=_decoder(8192, 29568, 8192, 1024),
        replicas=8, grad_dtype="bf16", step=500, log_scale_range=(-5.0, -1.0)),
}

# The workload the benchmark times by default.
BENCH_WORKLOAD = "qwen3_14b_layer"


def shrink(w: Workload, divisor: int, min_numel: int = 1) -> Workload:
    """Same recipe with every tensor divided by ``divisor`` and given a ragged
    length (not a multiple of 8), so small runs still cross several tiles and
    end in partial groups."""
    tensors = []
    for i, (name, n) in enumerate(w.tensors):
        m = max(min_numel, n // divisor)
        m = (m - m % 8) + (3 + 2 * i) % 8 if m > 8 else m
        tensors.append((name, max(1, m)))
    return replace(w, name=f"{w.name}/{divisor}", tensors=tuple(tensors))
