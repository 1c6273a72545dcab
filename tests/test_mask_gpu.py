"""Sliding windows, ALiBi and cross-attention (N_q != N_k) through fa_fwd_ext and
fa_bwd_ext, against the fp64 oracle's forward_general / backward_general."""

import math

import numpy as np
import pytest
import torch

import fa_inputs
from oracle import attention as A
from gpu_util import GRAD_REL_RMS, LSE_ABS, O_MAX_ABS, O_REL_RMS, to_dev, to_host

pytestmark = pytest.mark.gpu


def _inputs(B, H, Hkv, Nq, Nk, d, seed):
    """Q, dO [B, H, Nq, d] and K, V [B, Hkv, Nk, d] (exact bf16 values)."""
    a = fa_inputs.grouped_inputs(B, H, Hkv, Nq, d, seed, with_do=True)
    b = fa_inputs.grouped_inputs(B, H, Hkv, Nk, d, seed + 1)
    return {"q": a["q"], "do": a["do"], "k": b["k"], "v": b["v"]}


def _check(o, lse, grads, ref_o, ref_lse, ref_grads, tag):
    o = to_host(o)
    lse = lse.cpu().numpy().astype(np.float64)
    hidden = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), hidden), tag
    assert np.all(o[hidden] == 0.0), tag
    live = ~hidden
    e_max, e_rms = np.abs(o - ref_o).max(), A.rel_rms(o, ref_o)
    e_lse = np.abs(lse[live] - ref_lse[live]).max() if live.any() else 0.0
    print("%s O max_abs=%.3e rel_rms=%.3e LSE abs=%.3e hidden=%d" % (tag, e_max, e_rms, e_lse, hidden.sum()),
          flush=True)
    assert np.isfinite(o).all() and e_max <= O_MAX_ABS and e_rms <= O_REL_RMS and e_lse <= LSE_ABS, tag
    for name, g, r in zip(("dQ", "dK", "dV"), grads, ref_grads):
        g = to_host(g)
        assert g.shape == r.shape and np.isfinite(g).all(), (tag, name)
        if np.linalg.norm(r) == 0.0:
            assert np.abs(g).max() <= 1e-4, (tag, name)
            continue
        e = A.rel_rms(g, r)
        print("%s %s rel_rms=%.3e" % (tag, name, e), flush=True)
        assert e <= GRAD_REL_RMS, (tag, name, e)


def _run(gpu, B, H, Hkv, Nq, Nk, d, causal, window, alibi, seed, layout="bhnd"):
    tag = "B%d H%d Hkv%d Nq%d Nk%d d%d c%d w%s alibi%d %s" % (B, H, Hkv, Nq, Nk, d, causal, window, alibi, layout)
    print(tag, flush=True)
    x = _inputs(B, H, Hkv, Nq, Nk, d, seed)
    if layout == "bnhd":
        dev = {n: to_dev(x[n].transpose(0, 2, 1, 3)).transpose(1, 2) for n in x}
    else:
        dev = {n: to_dev(x[n]) for n in x}
    slopes = fa_inputs.alibi_slopes(H) if alibi else None
    sl = torch.from_numpy(slopes).cuda() if alibi else None
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=causal, window=window, alibi_slopes=sl)
    grads = gpu.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, window=window,
                    alibi_slopes=sl)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    w = window if window is not None else (-1, -1)
    ro, rl = A.forward_general(x["q"], x["k"], x["v"], causal, scale, w, slopes)
    rg = A.backward_general(x["q"], x["k"], x["v"], x["do"], causal, scale, w, slopes)
    _check(o, lse, grads, ro, rl, rg, tag)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,window,causal", [
    (300, (64, 0), True), (700, (100, 0), True), (333, (50, 70), False), (257, (0, 0), False),
    (513, (0, 200), False), (450, (255, -1), False), (200, (-1, 31), False), (130, (1, 1), True),
])
def test_sliding_window(gpu, N, window, causal, d):
    _run(gpu, 1, 2, 2, N, N, d, causal, window, False, 4000 + N)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,causal,window", [(257, True, None), (200, False, None), (380, True, (128, 0)),
                                             (301, False, (40, 90))])
def test_alibi(gpu, N, causal, window, d):
    _run(gpu, 1, 4, 4, N, N, d, causal, window, True, 4100 + N)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk,causal,window", [
    (100, 300, True, None), (100, 300, False, None), (300, 100, True, None), (300, 100, False, None),
    (1, 1000, True, None), (513, 77, True, None), (64, 640, True, (100, 0)), (200, 90, False, (10, 5)),
    (150, 20, False, (0, 3)),
])
def test_cross_attention(gpu, Nq, Nk, causal, window, d):
    _run(gpu, 2, 2, 1, Nq, Nk, d, causal, window, False, 4200 + Nq + Nk)


@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
def test_everything_together(gpu, layout):
    """GQA, cross-attention, a causal window and ALiBi in one call."""
    _run(gpu, 2, 8, 2, 190, 420, 128, True, (150, 0), True, 4300, layout)


def test_window_wider_than_sequence_is_bitwise_causal(gpu):
    x = fa_inputs.attention_inputs(1, 4, 777, 128, seed=4400, with_do=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o1, l1 = gpu.fwd(q, k, v, causal=True)
    g1 = gpu.bwd(q, k, v, o1, do, l1, causal=True)
    o2, l2 = gpu.fwd(q, k, v, causal=True, window=(5000, 7))
    g2 = gpu.bwd(q, k, v, o2, do, l2, causal=True, window=(5000, 7))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_window_n8192_d128_sampled(gpu):
    """A 1024-key causal sliding window at N = 8192, d = 128: sampled rows of O,
    LSE, dQ and sampled dK / dV rows against the oracle."""
    B, H, N, d, window = 1, 2, 8192, 128, (1024, 0)
    x = fa_inputs.attention_inputs(B, H, N, d, seed=4500, with_do=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = gpu.fwd(q, k, v, causal=True, window=window)
    dq, dk, dv = gpu.bwd(q, k, v, o, do, lse, causal=True, window=window)
    torch.cuda.synchronize()
    o, dq, dk, dv = (to_host(t) for t in (o, dq, dk, dv))
    lse = lse.cpu().numpy()
    idx = np.unique(np.concatenate([[0, 1, 1023, 1024, 1025, 4095, 8190, 8191],
                                    np.random.default_rng(9).integers(0, N, 10)]))
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        args = (x["q"][0, h], x["k"][0, h], x["v"][0, h], x["do"][0, h])
        ro, rl, rq = A.general_head_rows(*args, idx, True, scale, window)
        rk, rv = A.general_head_cols(*args, idx, True, scale, window)
        e = (A.rel_rms(o[0, h, idx], ro), np.abs(lse[0, h, idx] - rl).max(), A.rel_rms(dq[0, h, idx], rq),
             A.rel_rms(dk[0, h, idx], rk), A.rel_rms(dv[0, h, idx], rv))
        print("head %d O %.3e LSE %.3e dQ %.3e dK %.3e dV %.3e" % ((h,) + e), flush=True)
        assert e[0] <= O_REL_RMS and e[1] <= LSE_ABS and max(e[2:]) <= GRAD_REL_RMS
