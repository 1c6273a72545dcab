"""fa_fwd (bf16) against the fp64 oracle, through the C ABI, on the GPU."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from gpu_util import LSE_ABS, O_MAX_ABS, O_REL_RMS, inputs_on_device, to_host

pytestmark = pytest.mark.gpu


def _check(o, lse, o_ref, lse_ref, tag=""):
    o = np.asarray(o, np.float64)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), tag
    mx = A.max_abs(o, o_ref)
    rr = A.rel_rms(o, o_ref)
    le = A.max_abs(lse, lse_ref)
    print("%s max_abs=%.3e rel_rms=%.3e lse_abs=%.3e" % (tag, mx, rr, le), flush=True)
    assert mx <= O_MAX_ABS and rr <= O_REL_RMS and le <= LSE_ABS, tag


def _full(gpu, B, H, N, d, causal, seed):
    host, dev = inputs_on_device(B, H, N, d, seed)
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.forward(host["q"], host["k"], host["v"], causal, 1.0 / math.sqrt(d))
    _check(to_host(o), to_host(lse), o_ref, lse_ref, "B%d H%d N%d d%d c%d" % (B, H, N, d, causal))
    return host, dev, o, lse


def test_fwd_small_noncausal(gpu):
    _full(gpu, 1, 2, 256, 64, False, 1)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_n2048_d64(gpu, causal):
    _full(gpu, 4, 16, 2048, 64, causal, 2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 100, 129, 255, 300, 513])
def test_fwd_edge_lengths(gpu, N, d, causal):
    _full(gpu, 1, 3, N, d, causal, 1000 + N)


@pytest.mark.parametrize("N,causal", [(1024, False), (1025, False), (4096, True), (4097, True)])
def test_fwd_workgroup_shape_boundaries(gpu, N, causal):
    """Key lengths on both sides of the switch between four- and eight-wave
    workgroups (1024 keys without a mask, 4096 under the causal mask), the
    longer ones ragged."""
    _full(gpu, 1, 2, N, 128, causal, 3000 + N)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_several_tiles_d(gpu, d):
    _full(gpu, 2, 3, 1000, d, True, 77)


def test_fwd_n8192_d128_causal_whole(gpu):
    """Full-size workload (2 x 16 x 8192 x 128, causal): every element of O and
    LSE of all 32 heads against the fp64 oracle (whole-tensor max-abs and
    rel-RMS), the worst head reported."""
    B, H, N, d = 2, 16, 8192, 128
    host, dev = inputs_on_device(B, H, N, d, 3)
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    torch.cuda.synchronize()
    # causal row 0 sees only key 0: O_0 = V_0 exactly
    assert torch.equal(o[:, :, 0], dev["v"][:, :, 0])
    o_h, lse_h = to_host(o), to_host(lse)
    del o, lse, dev
    o_ref, lse_ref = A.forward(host["q"], host["k"], host["v"], True, 1.0 / math.sqrt(d))
    worst = max(((A.rel_rms(o_h[b, h], o_ref[b, h]), b, h) for b in range(B) for h in range(H)))
    print("n8192 worst head (%d,%d) rel_rms=%.3e" % (worst[1], worst[2], worst[0]), flush=True)
    _check(o_h, lse_h, o_ref, lse_ref, "n8192 whole tensor")


def test_fwd_deterministic_and_covers_outputs(gpu):
    B, H, N, d = 2, 4, 777, 128
    host, dev = inputs_on_device(B, H, N, d, 5)
    o1 = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l1 = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    gpu.fwd(dev["q"], dev["k"], dev["v"], causal=True, out=o1, lse=l1)
    o2, l2 = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_scale_argument(gpu):
    host, dev = inputs_on_device(1, 2, 300, 64, 9)
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=False, scale=0.37)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.forward(host["q"], host["k"], host["v"], False, 0.37)
    _check(to_host(o), to_host(lse), o_ref, lse_ref, "scale 0.37")


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_late_max_jump(gpu, causal):
    """Keys far past the first tiles (rows 600..615) scaled by 8 (exact in bf16) raise
    the rows' score maxima by far more than the kernel's rescale slack after several
    tiles, so the delayed rescale of O and l runs mid-sequence."""
    from gpu_util import to_dev
    import fa_inputs
    B, H, N, d = 1, 2, 1000, 128
    host = fa_inputs.attention_inputs(B, H, N, d, 31)
    host["k"][:, :, 600:616, :] *= 8.0
    dev = {k: to_dev(v) for k, v in host.items()}
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = A.forward(host["q"], host["k"], host["v"], causal, 1.0 / math.sqrt(d))
    _check(to_host(o), to_host(lse), o_ref, lse_ref, "late max jump c%d" % causal)
