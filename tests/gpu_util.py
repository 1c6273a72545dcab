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


# ------------------------------------------------ output coverage guards
# An output is carved out of a larger device buffer: the output region is
# filled with NaN (so any element a kernel leaves unwritten stays NaN) and the
# regions before and after it with a sentinel pattern (so any write past
# either end changes a sentinel bit).
GUARD_ELEMS = 4096
_SENTINEL = {torch.bfloat16: -7.25, torch.float32: -7.25}


class Guarded:
    """A NaN-poisoned contiguous tensor of `shape` between two sentinel regions."""

    def __init__(self, shape, dtype, device="cuda"):
        n = int(np.prod(shape))
        self.full = torch.full((n + 2 * GUARD_ELEMS,), _SENTINEL[dtype], dtype=dtype, device=device)
        self.full[GUARD_ELEMS:GUARD_ELEMS + n] = float("nan")
        self.t = self.full[GUARD_ELEMS:GUARD_ELEMS + n].view(shape)

    def check(self, tag=""):
        """Sentinels intact bit for bit; every output element written (finite)."""
        head = self.full[:GUARD_ELEMS]
        tail = self.full[-GUARD_ELEMS:]
        s = _SENTINEL[self.full.dtype]
        assert bool((head == s).all()) and bool((tail == s).all()), "write outside the output: %s" % tag
        assert bool(torch.isfinite(self.t).all()), "output element left unwritten (NaN): %s" % tag
