"""Helpers shared by the GPU parity tests (inputs to device, tolerances)."""

import numpy as np
import torch

import fa_inputs

# Bars on the bf16 path (max-abs / rel-RMS on O, abs on LSE, rel-RMS on grads).
O_MAX_ABS = 2e-2
O_REL_RMS = 1e-2
LSE_ABS = 1e-3
GRAD_REL_RMS = 2e-2
FP8_O_REL_RMS = 6e-2


def to_dev(x: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def inputs_on_device(B, H, N, d, seed, with_do=False, outliers=False):
    host = fa_inputs.attention_inputs(B, H, N, d, seed, with_do=with_do, outliers=outliers)
    dev = {k: to_dev(v) for k, v in host.items()}
    return host, dev


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)
