"""The five synthetic workloads: sharding, draw recipe, loss scaling, step counts.

All hyper-parameters are those stated for the smallest workload (AdamW,
lr 1e-3, betas (0.9, 0.999), eps 1e-8, weight decay 0.01, clip at total norm
1.0); the larger workloads state none and reuse them.
"""
from __future__ import annotations

from typing import NamedTuple, Optional


class Workload(NamedTuple):
    name: str
    model: str            # key into PARAM_LISTS
    dp_size: int
    dp_rank: int
    bucket_size: int      # elements; <= 0 means a single bucket per buffer
    steps: int
    grad_sigma: float
    weight_sigma: float = 0.02
    zero_frac: float = 0.0
    # loss scaling
    dynamic_scale: bool = False
    initial_scale: float = 1.0
    inf_step: Optional[int] = None   # 1-based step at which one +inf is injected
    seed: int = 0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_grad_norm: float = 1.0
    pad_for_high_busbw: int = 0

    def scale_at(self, step: int) -> float:
        """Loss scale the gradients of 1-based ``step`` were produced with.

        Input recipe: the scale starts at ``initial_scale`` and halves after the
        step that carries the injected overflow.
        """
        if not self.dynamic_scale:
            return self.initial_scale
        s = self.initial_scale
        if self.inf_step is not None and step > self.inf_step:
            s *= 0.5
        return s


def default_bucket_size(dp_size: int) -> int:
    return max(40_000_000, 1_000_000 * dp_size)


WORKLOADS = {
    "tiny": Workload("tiny", "tiny", 4, 1, 0, 3, 1e-2),
    "gpt2-small": Workload("gpt2-small", "gpt2-small", 8, 3, 40_000_000, 10, 1e-3),
    "llama3-8b": Workload("llama3-8b", "llama3-8b", 8, 5, default_bucket_size(8), 5, 1e-3),
    "dense-7b": Workload("dense-7b", "dense-7b", 1, 0, default_bucket_size(1), 5, 1e-3,
                         dynamic_scale=True, initial_scale=65536.0, inf_step=3),
    "llama3-70b": Workload("llama3-70b", "llama3-70b", 64, 37, default_bucket_size(64), 5, 1e-3, zero_frac=0.01),
}
