"""Grouped / multi-query heads and strided views ([B, N, H, d] storage, padded
rows) through fa_fwd_strided and fa_bwd_strided, against the fp64 oracle's
forward_gqa / backward_gqa (K and V repeated over each group of query heads)."""

import math

import numpy as np
import pytest
import torch

import fa_inputs
from oracle import attention as A
from gpu_util import GRAD_REL_RMS, LSE_ABS, O_MAX_ABS, O_REL_RMS, to_dev, to_host

pytestmark = pytest.mark.gpu


def _layout(x: np.ndarray, layout: str) -> torch.Tensor:
    """A bf16 [B, H, N, d] GPU view of x stored as `layout`."""
    if layout == "bhnd":
        return to_dev(x)
    if layout == "bnhd":
        return to_dev(x.transpose(0, 2, 1, 3)).transpose(1, 2)
    if layout == "padded":  # rows 64 elements longer than d
        B, H, N, d = x.shape
        big = torch.full((B, H, N, d + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        big[..., :d] = to_dev(x)
        return big[..., :d]
    raise ValueError(layout)


def _check_fwd(o, lse, ro, rl, tag):
    o = to_host(o)
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all(), tag
    e_max, e_rms, e_lse = np.abs(o - ro).max(), A.rel_rms(o, ro), np.abs(lse - rl).max()
    print("%s O max_abs=%.3e rel_rms=%.3e LSE abs=%.3e" % (tag, e_max, e_rms, e_lse), flush=True)
    assert e_max <= O_MAX_ABS and e_rms <= O_REL_RMS and e_lse <= LSE_ABS, tag


def _check_grads(got, ref, tag):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = to_host(g)
        assert g.shape == r.shape and np.isfinite(g).all(), (tag, name)
        e = A.rel_rms(g, r)
        print("%s %s rel_rms=%.3e" % (tag, name, e), flush=True)
        assert e <= GRAD_REL_RMS, (tag, name, e)


CASES = [  # (B, H, H_kv, N, d)
    (2, 8, 2, 300, 64),
    (1, 8, 2, 129, 128),
    (1, 4, 1, 200, 128),   # multi-query
    (2, 6, 3, 97, 64),
    (1, 4, 4, 255, 128),   # ordinary multi-head through the strided entry points
]


@pytest.mark.parametrize("layout", ["bhnd", "bnhd", "padded"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,d", CASES)
def test_grouped_fwd_bwd(gpu, B, H, Hkv, N, d, causal, layout):
    tag = "B%d H%d Hkv%d N%d d%d c%d %s" % (B, H, Hkv, N, d, causal, layout)
    print(tag, flush=True)
    x = fa_inputs.grouped_inputs(B, H, Hkv, N, d, seed=3000 + N + H + Hkv, with_do=True)
    q, k, v, do = (_layout(x[n], layout) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = gpu.fwd(q, k, v, causal=causal)
    dq, dk, dv = gpu.bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    if layout == "bnhd":  # outputs follow the inputs' layout
        assert o.stride() == q.stride() and dq.stride() == q.stride() and dk.stride() == k.stride()
    ro, rl = A.forward_gqa(x["q"], x["k"], x["v"], causal, scale)
    _check_fwd(o, lse, ro, rl, tag)
    _check_grads((dq, dk, dv), A.backward_gqa(x["q"], x["k"], x["v"], x["do"], causal, scale), tag)


@pytest.mark.parametrize("causal", [False, True])
def test_layouts_give_identical_bits(gpu, causal):
    """Strides change only addressing: [B, N, H, d] storage gives the same bits
    as contiguous [B, H, N, d] through the plain entry points."""
    x = fa_inputs.attention_inputs(2, 4, 333, 128, seed=77, with_do=True)
    c = {n: to_dev(x[n]) for n in x}
    t = {n: _layout(x[n], "bnhd") for n in x}
    o1, l1 = gpu.fwd(c["q"], c["k"], c["v"], causal=causal)
    g1 = gpu.bwd(c["q"], c["k"], c["v"], o1, c["do"], l1, causal=causal)
    o2, l2 = gpu.fwd(t["q"], t["k"], t["v"], causal=causal)
    g2 = gpu.bwd(t["q"], t["k"], t["v"], o2, t["do"], l2, causal=causal)
    torch.cuda.synchronize()
    assert not o2.is_contiguous()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_gqa_n2048_d128_causal(gpu):
    """A larger grouped case: B=1, H=16 query heads on H_kv=2, N=2048, d=128, causal."""
    B, H, Hkv, N, d = 1, 16, 2, 2048, 128
    x = fa_inputs.grouped_inputs(B, H, Hkv, N, d, seed=3100, with_do=True)
    q, k, v, do = (_layout(x[n], "bnhd") for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = gpu.fwd(q, k, v, causal=True)
    dq, dk, dv = gpu.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    ro, rl = A.forward_gqa(x["q"], x["k"], x["v"], True, scale)
    _check_fwd(o, lse, ro, rl, "gqa n2048")
    _check_grads((dq, dk, dv), A.backward_gqa(x["q"], x["k"], x["v"], x["do"], True, scale), "gqa n2048")


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_n8192_d128_sampled(gpu, causal):
    """H=16 query heads on H_kv=2 at N=8192 (the work of one K/V head's key
    block is then shared by several workgroups, whose fp32 partials a
    reduction adds): sampled dQ rows of two query heads and dK / dV rows of
    both K/V heads, each summed over its 8 query heads."""
    B, H, Hkv, N, d = 1, 16, 2, 8192, 128
    x = fa_inputs.grouped_inputs(B, H, Hkv, N, d, seed=3200 + causal, with_do=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = gpu.fwd(q, k, v, causal=causal)
    dq, dk, dv = (to_host(t) for t in gpu.bwd(q, k, v, o, do, lse, causal=causal))
    idx = np.unique(np.concatenate([[0, 1, 127, 128, 4095, 8190, 8191],
                                    np.random.default_rng(7).integers(0, N, 12)]))
    g = H // Hkv
    for h in (0, 13):
        hk = h // g
        rq = A.backward_head_rows(x["q"][0, h], x["k"][0, hk], x["v"][0, hk], x["do"][0, h], idx, causal, scale)
        e = A.rel_rms(dq[0, h, idx], rq)
        print("c%d dQ head %d rel_rms=%.3e" % (causal, h, e), flush=True)
        assert e <= GRAD_REL_RMS
    for hk in range(Hkv):
        rk = np.zeros((len(idx), d))
        rv = np.zeros((len(idx), d))
        for h in range(hk * g, (hk + 1) * g):
            a, c = A.backward_head_cols(x["q"][0, h], x["k"][0, hk], x["v"][0, hk], x["do"][0, h], idx, causal, scale)
            rk += a
            rv += c
        ek, ev = A.rel_rms(dk[0, hk, idx], rk), A.rel_rms(dv[0, hk, idx], rv)
        print("c%d dK/dV kv head %d rel_rms=%.3e %.3e" % (causal, hk, ek, ev), flush=True)
        assert ek <= GRAD_REL_RMS and ev <= GRAD_REL_RMS


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_row_stride_at_the_32_bit_offset_limit(gpu, d, causal):
    """The forward loads full K / V tiles from the tile's first row plus a
    32-bit per-lane byte offset while 64 row strides fit in 2^32 bytes (row
    stride below 2^25 elements), and forms 64-bit addresses otherwise (and for
    the ragged last tile). Q, K and V share rows of one buffer, with row
    strides just below and at 2^25 elements (O, an output, may not overlap
    them and has its own); N = 66 gives one full tile and a ragged one. Both
    strides give the same bits, and both match the oracle."""
    N, B, H = 66, 1, 1
    x = fa_inputs.attention_inputs(B, H, N, d, seed=4400 + d + causal)
    scale = 1.0 / math.sqrt(d)
    ro, rl = A.forward(x["q"], x["k"], x["v"], causal, scale)
    got = []
    for rs in ((1 << 25) - 64, 1 << 25):
        tag = "d%d c%d rs=%d" % (d, causal, rs)
        print(tag, flush=True)
        buf = torch.empty(N * rs, dtype=torch.bfloat16, device="cuda")  # N rows of rs elements
        q, k, v = (buf.as_strided((B, H, N, d), (N * rs, N * rs, rs, 1), j * d) for j in range(3))
        for t, n in zip((q, k, v), ("q", "k", "v")):
            t.copy_(to_dev(x[n]))
        o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        o2, lse = gpu.fwd(q, k, v, causal=causal, out=o)
        torch.cuda.synchronize()
        assert o2.data_ptr() == o.data_ptr()
        got.append((o.clone(), lse.clone()))
        _check_fwd(o, lse, ro, rl, tag)
        del buf, q, k, v, o, o2
        torch.cuda.empty_cache()
    assert torch.equal(got[0][0], got[1][0]) and torch.equal(got[0][1], got[1][1])
