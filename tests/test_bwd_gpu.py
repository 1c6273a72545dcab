"""fa_bwd (bf16, recomputation from the saved LSE) against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from gpu_util import GRAD_REL_RMS, inputs_on_device, to_host

pytestmark = pytest.mark.gpu


def _run(gpu, B, H, N, d, causal, seed):
    host, dev = inputs_on_device(B, H, N, d, seed, with_do=True)
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    dq, dk, dv = gpu.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal)
    torch.cuda.synchronize()
    return host, dev, (o, lse), (dq, dk, dv)


def _check_grads(got, ref, tag):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = np.asarray(g, np.float64)
        assert np.isfinite(g).all(), (tag, name)
        if np.linalg.norm(np.ravel(r)) == 0.0:
            # exactly zero by definition (a single visible key: dS = P (dP - D) = 0);
            # the kernel's D and dP differ only by summation order
            print("%s %s max_abs=%.3e (zero reference)" % (tag, name, np.abs(g).max()), flush=True)
            assert np.abs(g).max() <= 1e-4, (tag, name)
            continue
        e = A.rel_rms(g, r)
        print("%s %s rel_rms=%.3e" % (tag, name, e), flush=True)
        assert e <= GRAD_REL_RMS, (tag, name, e)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 100, 129, 255, 300, 640])
def test_bwd_edge_lengths(gpu, N, d, causal):
    host, dev, _, got = _run(gpu, 1, 2, N, d, causal, 2000 + N)
    ref = A.backward(host["q"], host["k"], host["v"], host["do"], causal, 1.0 / math.sqrt(d))
    _check_grads([to_host(t) for t in got], ref, "N%d d%d c%d" % (N, d, causal))


@pytest.mark.parametrize("N,causal", [(1024, False), (1025, False), (4097, True)])
def test_bwd_workgroup_shape_boundaries(gpu, N, causal):
    """The dQ pass on both sides of its switch between four- and eight-wave
    workgroups (1024 keys without a mask, 4096 causal; 4096 itself is the
    backward workload below), the longer ones ragged."""
    host, dev, _, got = _run(gpu, 1, 1, N, 128, causal, 3100 + N)
    ref = A.backward(host["q"], host["k"], host["v"], host["do"], causal, 1.0 / math.sqrt(128))
    _check_grads([to_host(t) for t in got], ref, "N%d c%d" % (N, causal))


def test_bwd_n4096_d128_causal(gpu):
    """The backward workload: B=2, H=16, N=4096, d=128, causal; O, LSE from fa_fwd."""
    B, H, N, d = 2, 16, 4096, 128
    host, dev, _, got = _run(gpu, B, H, N, d, True, 4)
    got = [to_host(t) for t in got]
    ref = A.backward(host["q"], host["k"], host["v"], host["do"], True, 1.0 / math.sqrt(d))
    _check_grads(got, ref, "bwd n4096")


def test_bwd_n8192_d128_causal_whole(gpu):
    """N = 8192 (the headline backward shape: the forward workload's Q, K, V
    plus dO from the same seed): every element of dQ, dK, dV of all 32 heads
    against the fp64 oracle (whole-tensor rel-RMS), the worst head reported."""
    B, H, N, d = 2, 16, 8192, 128
    host, dev, _, got = _run(gpu, B, H, N, d, True, 3)
    got = [to_host(t) for t in got]
    del dev
    ref = A.backward(host["q"], host["k"], host["v"], host["do"], True, 1.0 / math.sqrt(d))
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        worst = max(((A.rel_rms(g[b, h], r[b, h]), b, h) for b in range(B) for h in range(H)))
        print("n8192 %s worst head (%d,%d) rel_rms=%.3e" % (name, worst[1], worst[2], worst[0]), flush=True)
    _check_grads(got, ref, "bwd n8192 whole tensor")


def test_bwd_deterministic(gpu):
    # no atomics: every gradient element is summed by one wave in a fixed order
    host, dev, (o, lse), (dq, dk, dv) = _run(gpu, 1, 4, 700, 128, True, 6)
    dq2, dk2, dv2 = gpu.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2) and torch.equal(dq, dq2)


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 2, 300, 64, False),
    (1, 2, 300, 128, True),
    (1, 2, 257, 256, True),
    (2, 16, 1024, 128, True),  # the persistent four-wave dQ instance
    (2, 16, 8192, 128, True),  # the headline shape: the persistent eight-wave instance
])
def test_bwd_row_delta_in_workspace(gpu, B, H, N, d, causal):
    """Row term D = rowsum(dO o O) of every query row, formed by the dQ kernel
    from the kernel's own bf16 O and left in the caller's workspace (filled
    with NaN bytes beforehand), against the oracle's row_delta. The products
    of two bf16 values are exact in fp32, so the only error is the fp32 sum."""
    host, dev = inputs_on_device(B, H, N, d, 40 + N, with_do=True)
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    ws = torch.full((gpu.bwd_workspace_bytes(B, H, N, d),), 0xFF, dtype=torch.uint8, device="cuda")
    gpu.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, workspace=ws)
    torch.cuda.synchronize()
    got = ws[: B * H * N * 4].view(torch.float32).reshape(B, H, N).cpu().numpy().astype(np.float64)
    o_host = to_host(o)
    ref = A.row_delta(o_host, host["do"])
    bound = np.abs(o_host * host["do"]).sum(axis=-1)
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    print("D max_abs=%.3e max_rel_to_sum_abs=%.3e" % (err.max(), (err / np.maximum(bound, 1e-30)).max()), flush=True)
    assert (err <= 1e-5 * bound + 1e-30).all()
