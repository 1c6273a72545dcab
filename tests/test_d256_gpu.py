"""Head dim 256 (forward, backward) against the fp64 oracle: plain, grouped,
strided, masked and cross-attention cases."""

import math

import numpy as np
import pytest
import torch

import fa_inputs
from oracle import attention as A
from gpu_util import GRAD_REL_RMS, LSE_ABS, O_REL_RMS, inputs_on_device, to_host
from test_mask_gpu import _run

pytestmark = pytest.mark.gpu

D = 256


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 100, 129, 300, 513])
def test_d256_lengths(gpu, N, causal):
    _run(gpu, 1, 2, 2, N, N, D, causal, None, False, 5000 + N)


@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
def test_d256_grouped_masked_cross(gpu, layout):
    _run(gpu, 1, 4, 2, 200, 333, D, True, (120, 0), True, 5100, layout)


@pytest.mark.parametrize("window", [(64, 64), (0, 0)])
def test_d256_window(gpu, window):
    _run(gpu, 2, 2, 1, 300, 300, D, False, window, False, 5200 + window[0])


def test_d256_n2048_causal(gpu):
    """B=1, H=4, N=2048, d=256, causal: full comparison."""
    B, H, N = 1, 4, 2048
    host, dev = inputs_on_device(B, H, N, D, 5300, with_do=True)
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    grads = gpu.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(D)
    ro, rl = A.forward(host["q"], host["k"], host["v"], True, scale)
    rg = A.backward(host["q"], host["k"], host["v"], host["do"], True, scale)
    e_o = A.rel_rms(to_host(o), ro)
    e_l = np.abs(lse.cpu().numpy() - rl).max()
    print("d256 n2048 O rel_rms=%.3e LSE abs=%.3e" % (e_o, e_l), flush=True)
    assert e_o <= O_REL_RMS and e_l <= LSE_ABS
    for name, g, r in zip(("dQ", "dK", "dV"), grads, rg):
        e = A.rel_rms(to_host(g), r)
        print("d256 n2048 %s rel_rms=%.3e" % (name, e), flush=True)
        assert e <= GRAD_REL_RMS


@pytest.mark.parametrize("causal,window", [(False, (60, 30)), (True, None)])
def test_d256_alibi(gpu, causal, window):
    _run(gpu, 1, 4, 2, 333, 333, D, causal, window, True, 5400)
