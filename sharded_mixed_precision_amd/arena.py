"""Device memory for one rank's step, allocated with PyTorch.

Per flat buffer: the grad window arena (read by the step), the param window
arena (written back), and the fp32 master / Adam m / Adam v arenas, all of
``arena_numel`` elements; plus the workspace.  Allocation only; the step runs
in the library.
"""
from __future__ import annotations

from typing import Dict, List

import torch

from . import DTYPE_NAMES, Layout

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


class DeviceArenas:
    def __init__(self, layout: Layout, device: str = "cuda"):
        self.layout = layout
        self.device = device
        self.bufs: List[Dict[str, torch.Tensor]] = []
        self.info = []
        for k in range(layout.num_buffers):
            b = layout.buffer(k)
            pd, gd = DTYPE_NAMES[b["param_dtype"]], DTYPE_NAMES[b["grad_dtype"]]
            n = b["arena_numel"]
            t = {
                "grad": torch.zeros(n, dtype=TORCH_DTYPES[gd], device=device),
                "param": torch.zeros(n, dtype=TORCH_DTYPES[pd], device=device),
                "master": torch.empty(n, dtype=torch.float32, device=device) if pd != "f32" else None,
                "exp_avg": torch.empty(n, dtype=torch.float32, device=device),
                "exp_avg_sq": torch.empty(n, dtype=torch.float32, device=device),
            }
            self.bufs.append(t)
            self.info.append({"pd": pd, "gd": gd, "n": n, **b})
        self.workspace = torch.zeros(layout.workspace_bytes, dtype=torch.uint8, device=device)

    def state_bytes(self) -> int:
        tot = 0
        for t in self.bufs:
            for v in t.values():
                if v is not None:
                    tot += v.numel() * v.element_size()
        return tot + self.workspace.numel()
