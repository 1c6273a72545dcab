"""Output coverage: every output element written exactly inside its tensor.

Each output is carved out of a larger device buffer (tests/gpu_util.Guarded):
the output itself is NaN-filled before the call, and sentinel regions sit
directly before and after it. After the call every output element must be
finite (a tile, row or column a kernel skipped would stay NaN, whatever the
caching allocator held before) and every sentinel bit unchanged (no write past
either end). The values are also compared with the fp64 oracle.

Backward cases cover each write path of the gradients: the plain key-stationary
epilogue, grouped heads whose key blocks are split over workgroups (fp32
partials summed by a reduction kernel), d = 256 (two workgroups per key block,
one per half of the dK / dV columns), and key blocks that no query sees (dK,
dV written as zeros). The fp8 forward's O and LSE are guarded the same way.
"""

import math

import numpy as np
import pytest
import torch

import fa_inputs
from oracle import attention as A
from oracle import fp8 as F
from gpu_util import FP8_O_REL_RMS, GRAD_REL_RMS, LSE_ABS, O_MAX_ABS, Guarded, to_dev, to_host

pytestmark = pytest.mark.gpu


def _grads_guarded(gpu, B, H, Hkv, Nq, Nk, d, causal, window, seed):
    tag = "B%d H%d Hkv%d Nq%d Nk%d d%d c%d w%s" % (B, H, Hkv, Nq, Nk, d, causal, window)
    print(tag, flush=True)
    a = fa_inputs.grouped_inputs(B, H, Hkv, Nq, d, seed, with_do=True)
    b = fa_inputs.grouped_inputs(B, H, Hkv, Nk, d, seed + 1)
    x = {"q": a["q"], "do": a["do"], "k": b["k"], "v": b["v"]}
    dev = {n: to_dev(x[n]) for n in x}
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=causal, window=window)
    gq = Guarded((B, H, Nq, d), torch.bfloat16)
    gk = Guarded((B, Hkv, Nk, d), torch.bfloat16)
    gv = Guarded((B, Hkv, Nk, d), torch.bfloat16)
    gpu.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal, window=window,
            out=(gq.t, gk.t, gv.t))
    torch.cuda.synchronize()
    for name, g in (("dQ", gq), ("dK", gk), ("dV", gv)):
        g.check("%s %s" % (tag, name))
    ref = A.backward_general(x["q"], x["k"], x["v"], x["do"], causal, 1.0 / math.sqrt(d),
                             window if window is not None else (-1, -1))
    for name, g, r in zip(("dQ", "dK", "dV"), (gq.t, gk.t, gv.t), ref):
        got = to_host(g)
        if np.linalg.norm(r) == 0.0:
            assert np.abs(got).max() <= 1e-4, (tag, name)
            continue
        e = A.rel_rms(got, r)
        print("%s %s rel_rms=%.3e" % (tag, name, e), flush=True)
        assert e <= GRAD_REL_RMS, (tag, name, e)
    return ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_outputs_covered_plain(gpu, d, causal):
    """Contiguous multi-head backward (fa_bwd), ragged N over several key blocks."""
    _grads_guarded(gpu, 2, 3, 3, 777, 777, d, causal, None, 7100 + d)


def test_bwd_outputs_covered_persistent_dkdv(gpu):
    """Causal d = 128 with at most 1024 keys runs the dK / dV kernel on a
    persistent grid (each XCD taking whole heads' key blocks per round, the
    order reversed on odd rounds): 64 K/V heads, ragged N = 1000 (8 key
    blocks), two rounds per workgroup."""
    _grads_guarded(gpu, 4, 16, 16, 1000, 1000, 128, True, None, 7150)


def test_bwd_outputs_covered_grouped_split(gpu):
    """H = 8 on H_kv = 2, short N: each key block's four query heads are split
    over workgroups that leave fp32 partials for the reduction kernel."""
    B, H, Hkv, N, d = 1, 8, 2, 300, 64
    ws = gpu.bwd_workspace_bytes(B, H, N, d, H_kv=Hkv, causal=True)
    assert ws > gpu.bwd_workspace_bytes(B, H, N, d), "expected the split (partials) path"
    _grads_guarded(gpu, B, H, Hkv, N, N, d, True, None, 7200)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_outputs_covered_d256(gpu, causal):
    """d = 256: two workgroups per key block, each writing one half of the dK / dV columns."""
    _grads_guarded(gpu, 1, 2, 2, 300, 300, 256, causal, None, 7300)


def test_bwd_outputs_covered_unseen_key_blocks(gpu):
    """64 queries on 1024 keys, causal, 32-key window: query i sees keys
    928 + i .. 960 + i only, so key blocks 0 .. 6 are seen by no query and the
    dK / dV rows there must be written as zeros."""
    ref = _grads_guarded(gpu, 1, 2, 2, 64, 1024, 128, True, (32, 0), 7400)
    assert np.all(ref[1][:, :, :896] == 0.0) and np.all(ref[2][:, :, :896] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,exp_mode", [(64, 0), (128, 0), (128, 1), (128, 2)])
def test_fwd_fp8_outputs_covered(gpu, d, exp_mode, causal):
    """exp_mode 1 and 2 (the software 2^x) are separate kernel instances."""
    B, H, N = 2, 3, 777
    host = fa_inputs.attention_inputs(B, H, N, d, 7500 + d, outliers=True)
    dev = {n: to_dev(host[n]) for n in host}
    qz = {n: gpu.quant_fp8(dev[n]) for n in ("q", "k", "v")}
    go = Guarded((B, H, N, d), torch.bfloat16)
    gl = Guarded((B, H, N), torch.float32)
    gpu.fwd_fp8(qz["q"][0], qz["k"][0], qz["v"][0], qz["q"][1], qz["k"][1], qz["v"][1], causal=causal,
                out=go.t, lse=gl.t, exp_mode=exp_mode)
    torch.cuda.synchronize()
    go.check("fp8 O d%d c%d mode %d" % (d, causal, exp_mode))
    gl.check("fp8 LSE d%d c%d mode %d" % (d, causal, exp_mode))
    deq = {n: F.dequantize(qz[n][0].cpu().numpy(), qz[n][1].cpu().numpy()) for n in ("q", "k", "v")}
    r_o, _ = A.forward(deq["q"], deq["k"], deq["v"], causal, 1.0 / math.sqrt(d))
    e = A.rel_rms(to_host(go.t), r_o)
    print("fp8 guarded d%d c%d rel_rms=%.3e" % (d, causal, e), flush=True)
    assert e <= FP8_O_REL_RMS


@pytest.mark.parametrize("B,H,N,d,causal", [
    (4, 16, 2048, 64, True),     # persistent, head-major per XCD, two rounds (Q-block order flipped)
    (16, 16, 1024, 128, True),   # persistent, head-major per XCD, four rounds
    (16, 16, 1024, 128, False),  # the same without a mask
    (5, 13, 2048, 64, True),     # B H not a multiple of 8: falling-cost dealing, two rounds
    (7, 9, 2048, 128, True),     # the same at d = 128
    (2, 16, 8192, 64, True),     # 64 Q-blocks per head do not divide the slots of an XCD: falling cost
])
def test_fwd_persistent_dealings_cover_outputs(gpu, B, H, N, d, causal):
    """Each persistent dealing of the short-key forward writes every O and LSE
    element once and nothing outside them, with results equal to a plain call
    and, on sampled rows of the first and last heads, to the fp64 oracle."""
    tag = "B%d H%d N%d d%d c%d" % (B, H, N, d, causal)
    print(tag, flush=True)
    x = fa_inputs.attention_inputs(B, H, N, d, seed=5100 + N + d + H)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    go = Guarded((B, H, N, d), torch.bfloat16)
    gl = Guarded((B, H, N), torch.float32)
    gpu.fwd(q, k, v, causal=causal, out=go.t, lse=gl.t)
    o2, l2 = gpu.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    go.check(tag + " O")
    gl.check(tag + " LSE")
    assert torch.equal(go.t, o2) and torch.equal(gl.t, l2), tag
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N - 2, N - 1],
                                     np.random.default_rng(N).integers(0, N, 10)]))
    o_h, l_h = to_host(go.t), to_host(gl.t)
    for b, h in ((0, 0), (B - 1, H - 1)):
        ro, rl = A.forward_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], causal, 1.0 / math.sqrt(d), rows=rows)
        e = np.abs(o_h[b, h, rows] - ro).max()
        el = np.abs(l_h[b, h, rows] - rl).max()
        print("%s head (%d,%d) O max_abs=%.3e LSE abs=%.3e" % (tag, b, h, e, el), flush=True)
        assert e <= O_MAX_ABS and el <= LSE_ABS, (tag, b, h)


def test_bwd_dq_persistent_dealing_covers_outputs(gpu):
    """The causal d = 128 dQ kernel at N = 8192 runs a persistent grid, each
    XCD taking all Q-blocks of a head per round (two rounds here, the second
    in reversed Q-block order): every dQ element written once and nothing
    outside it, equal to the unguarded call, and sampled rows of the first
    and last heads against the fp64 oracle."""
    B, H, N, d = 1, 16, 8192, 128
    x = fa_inputs.attention_inputs(B, H, N, d, seed=5300, with_do=True)
    dev = {n: to_dev(x[n]) for n in x}
    o, lse = gpu.fwd(dev["q"], dev["k"], dev["v"], causal=True)
    gq = Guarded((B, H, N, d), torch.bfloat16)
    gk = Guarded((B, H, N, d), torch.bfloat16)
    gv = Guarded((B, H, N, d), torch.bfloat16)
    gpu.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True, out=(gq.t, gk.t, gv.t))
    dq2, dk2, dv2 = gpu.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True)
    torch.cuda.synchronize()
    for name, g, ref in (("dQ", gq, dq2), ("dK", gk, dk2), ("dV", gv, dv2)):
        g.check("n8192 " + name)
        assert torch.equal(g.t, ref), name
    rows = np.unique(np.concatenate([[0, 255, 256, 4095, 8191], np.random.default_rng(11).integers(0, N, 8)]))
    got = to_host(gq.t)
    for h in (0, H - 1):
        ref = A.backward_head_rows(x["q"][0, h], x["k"][0, h], x["v"][0, h], x["do"][0, h], rows, True,
                                   1.0 / math.sqrt(d))
        e = A.rel_rms(got[0, h, rows], ref)
        print("dQ head %d sampled rel_rms=%.3e" % (h, e), flush=True)
        assert e <= GRAD_REL_RMS, h


@pytest.mark.parametrize("exp_mode", [0, 2])
def test_fwd_fp8_persistent_dealing_covers_outputs(gpu, exp_mode):
    """Causal d = 128 fp8 forward on its persistent grid (each XCD taking all
    Q-blocks of a head per round, four rounds, the order reversed on odd
    rounds), with the hardware and the software exponential: O and LSE
    written once and nothing outside them; two heads against the fp64 oracle
    on the dequantised inputs."""
    B, H, N, d = 16, 16, 1024, 128
    host = fa_inputs.attention_inputs(B, H, N, d, 7600, outliers=True)
    dev = {n: to_dev(host[n]) for n in host}
    qz = {n: gpu.quant_fp8(dev[n]) for n in ("q", "k", "v")}
    go = Guarded((B, H, N, d), torch.bfloat16)
    gl = Guarded((B, H, N), torch.float32)
    gpu.fwd_fp8(qz["q"][0], qz["k"][0], qz["v"][0], qz["q"][1], qz["k"][1], qz["v"][1], causal=True,
                out=go.t, lse=gl.t, exp_mode=exp_mode)
    torch.cuda.synchronize()
    go.check("fp8 persistent O mode %d" % exp_mode)
    gl.check("fp8 persistent LSE mode %d" % exp_mode)
    o_h = to_host(go.t)
    for b, h in ((0, 0), (B - 1, H - 1)):
        deq = {n: F.dequantize(qz[n][0][b:b + 1, h:h + 1].cpu().numpy(), qz[n][1][b:b + 1, h:h + 1].cpu().numpy())
               for n in ("q", "k", "v")}
        r_o, _ = A.forward(deq["q"], deq["k"], deq["v"], True, 1.0 / math.sqrt(d))
        e = A.rel_rms(o_h[b:b + 1, h:h + 1], r_o)
        print("fp8 persistent head (%d,%d) rel_rms=%.3e" % (b, h, e), flush=True)
        assert e <= FP8_O_REL_RMS, (b, h)
