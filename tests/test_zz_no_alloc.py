"""fa_bwd_noalloc (the backward with its D vector in the library's static
per-GPU scratch) against fa_bwd (caller workspace), through the C ABI.

Two calls in a row, the second on a smaller problem, so that the second call
starts with the first call's D still in the scratch; each must give exactly
fa_bwd's gradients (same kernels), which the oracle checks too.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from gpu_util import GRAD_REL_RMS, inputs_on_device, to_host

pytestmark = pytest.mark.gpu


def _case(gpu, B, H, N, d, causal, seed):
    tag = "noalloc B%d H%d N%d d%d c%d" % (B, H, N, d, causal)
    print(tag, flush=True)
    host, dev = inputs_on_device(B, H, N, d, seed, with_do=True)
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    ref = gpu.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal)
    outs = tuple(torch.full_like(dev["q"], float("nan")) for _ in range(3))
    got = gpu.bwd_noalloc(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, out=outs)
    torch.cuda.synchronize()
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(g, r), "%s %s differs from fa_bwd" % (tag, name)
    return host, got


def test_bwd_noalloc_matches_fa_bwd_twice(gpu):
    _case(gpu, 2, 4, 1000, 128, True, 8100)
    host, got = _case(gpu, 1, 2, 300, 64, False, 8200)
    ref = A.backward(host["q"], host["k"], host["v"], host["do"], False, 1.0 / math.sqrt(64))
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        e = A.rel_rms(to_host(g), r)
        print("noalloc small %s rel_rms=%.3e" % (name, e), flush=True)
        assert e <= GRAD_REL_RMS


def test_bwd_noalloc_at_the_scratch_limit(gpu):
    """B * H * N = 2^21 rows: D fills the 8 MiB scratch exactly (the largest
    problem the entry point accepts), so the last rows of D sit at its very
    end. The gradients equal fa_bwd's bit for bit."""
    B, H, N, d = 64, 32, 1024, 64
    assert 4 * B * H * N == 8 << 20
    g = torch.Generator(device="cuda")
    g.manual_seed(8300)
    q, k, v, do = (torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(4))
    o, lse = gpu.fwd(q, k, v, causal=True)
    ref = gpu.bwd(q, k, v, o, do, lse, causal=True)
    outs = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    got = gpu.bwd_noalloc(q, k, v, o, do, lse, causal=True, out=outs)
    torch.cuda.synchronize()
    for name, a_, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a_, r), "noalloc at the limit: %s differs from fa_bwd" % name


def test_bwd_noalloc_rejects_too_large(gpu):
    """B * H * N rows of D beyond the 8 MiB scratch: FA_ERR_SCRATCH, nothing launched."""
    B, H, N, d = 1, 33, 65536, 64  # 2162688 rows > 2^21
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    with pytest.raises(gpu.FAError) as e:
        gpu.bwd_noalloc(q, q.clone(), q.clone(), q.clone(), q.clone(), lse)
    assert e.value.status == 10
