"""Parity along the sequence-length sweep (16384 tokens: N = 512 .. 16384,
B = 16384 / N, H = 16, d = 64 and 128, causal and not): the forward on two
heads per point against the fp64 oracle (all rows up to N = 2048, sampled
rows beyond)."""

import math

import numpy as np
import pytest

import fa_inputs
from oracle import attention as A
from gpu_util import LSE_ABS, O_MAX_ABS, O_REL_RMS, inputs_on_device, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [512, 1024, 2048, 4096, 8192, 16384])
def test_sweep_point(gpu, N, d, causal):
    B, H = 16384 // N, 16
    host, dev = inputs_on_device(B, H, N, d, fa_inputs.sweep_seed(N))
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    o, lse = to_host(o), lse.cpu().numpy()
    scale = 1.0 / math.sqrt(d)
    rows = None if N <= 2048 else np.unique(np.concatenate(
        [[0, 1, 255, 256, N // 2, N - 2, N - 1], np.random.default_rng(N + d).integers(0, N, 57)]))
    for b, h in ((0, 0), (B - 1, H - 1)):
        ro, rl = A.forward_head(host["q"][b, h], host["k"][b, h], host["v"][b, h], causal, scale, rows)
        go = o[b, h] if rows is None else o[b, h, rows]
        gl = lse[b, h] if rows is None else lse[b, h, rows]
        e, em, el = A.rel_rms(go, ro), A.max_abs(go, ro), np.abs(gl - rl).max()
        print("sweep N%d d%d c%d head (%d,%d): O max_abs=%.3e rel_rms=%.3e LSE abs=%.3e"
              % (N, d, causal, b, h, em, e, el), flush=True)
        assert em <= O_MAX_ABS and e <= O_REL_RMS and el <= LSE_ABS
