"""Pins for the oracle's general masks: sliding windows, ALiBi, cross-attention
(N_q != N_k, bottom-right alignment) and fully hidden rows. None of them
re-types the mask or bias formula of ``oracle/attention.py``.

Pin list:
  W-1 window sets by hand (tests/golden/window_visible_sets.json): with Q = 0,
      O is the mean of the listed V rows and LSE = log(count)
  W-2 window (0, 0) gives O_i = V of the diagonal key, LSE_i = its score
  W-3 a window row equals the plain (pinned) forward of that query on the
      slice of keys the window keeps
  X-1 causal cross-attention, N_q < N_k: the plain causal forward on Q padded
      at the front to N_k rows, last N_q rows taken
  X-2 causal cross-attention, N_q > N_k: the first N_q - N_k rows see nothing
      (O = 0, LSE = -inf); the rest are the plain causal forward
  A-1 ALiBi, Q = 0: P and LSE in closed form (geometric sums), causal and not
  A-2 ALiBi, causal: the plain causal forward with one extra dimension
      carrying slope * j in K and 1 in Q (the row constant -slope * i moves
      LSE only)
  D-1 finite differences of sum(O * dO) match backward_general (window,
      ALiBi, cross-attention, grouped heads together)
  D-2 torch SDPA with the same float mask, and its autograd, on rows that see
      at least one key
  Planted mistakes: each plausible bug fails at least one of these pins.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _bh(x):
    return x[None, None]


# ------------------------------------------------------------------ pins
def pin_window_sets():
    g = json.load(open(os.path.join(GOLDEN, "window_visible_sets.json")))
    for case in g["cases"]:
        n_q, n_k, d = case["n_q"], case["n_k"], 4
        v = _rand((n_k, d), 11)
        q, k = np.zeros((n_q, d)), _rand((n_k, d), 12)
        o, lse = A.forward_general(_bh(q), _bh(k), _bh(v), case["causal"], 0.5, tuple(case["window"]))
        for i, keys in enumerate(case["visible"]):
            if not keys:
                assert np.all(o[0, 0, i] == 0.0) and np.isneginf(lse[0, 0, i]), (case, i)
                continue
            assert np.allclose(o[0, 0, i], v[keys].mean(axis=0), rtol=1e-13, atol=1e-14), (case, i)
            assert abs(lse[0, 0, i] - math.log(len(keys))) < 1e-13, (case, i)


def pin_window_zero():
    for n_q, n_k in ((9, 9), (5, 9)):
        q, k, v = _rand((n_q, 8), 13), _rand((n_k, 8), 14), _rand((n_k, 8), 15)
        o, lse = A.forward_general(_bh(q), _bh(k), _bh(v), False, 0.4, (0, 0))
        for i in range(n_q):
            j = i + n_k - n_q
            assert np.allclose(o[0, 0, i], v[j], rtol=1e-14, atol=1e-14)
            assert abs(lse[0, 0, i] - A.scale_as_f32(0.4) * (q[i] @ k[j])) < 1e-12


def pin_window_slices(n_q=13, n_k=13, window=(3, 2), causal=False):
    q, k, v = _rand((n_q, 8), 16), _rand((n_k, 8), 17), _rand((n_k, 8), 18)
    o, lse = A.forward_general(_bh(q), _bh(k), _bh(v), causal, 0.3, window)
    left, right = window
    for i in range(n_q):
        # the keys the window keeps, written as a contiguous slice
        c = i + n_k - n_q
        lo = 0 if left < 0 else max(0, c - left)
        hi = n_k if right < 0 else min(n_k, c + right + 1)
        if causal:
            hi = min(hi, c + 1)
        if hi <= lo:  # the window misses every key
            assert np.all(o[0, 0, i] == 0.0) and np.isneginf(lse[0, 0, i]), i
            continue
        ro, rl = A.forward_head(q[i:i + 1], k[lo:hi], v[lo:hi], False, 0.3)
        assert np.allclose(o[0, 0, i], ro[0], rtol=1e-12, atol=1e-13), i
        assert abs(lse[0, 0, i] - rl[0]) < 1e-12, i


def pin_cross_short_queries(n_q=5, n_k=12):
    q, k, v = _rand((n_q, 8), 19), _rand((n_k, 8), 20), _rand((n_k, 8), 21)
    o, lse = A.forward_general(_bh(q), _bh(k), _bh(v), True, 0.35)
    padded = np.concatenate([_rand((n_k - n_q, 8), 22), q])
    ro, rl = A.forward(_bh(padded), _bh(k), _bh(v), True, 0.35)
    assert np.allclose(o[0, 0], ro[0, 0, n_k - n_q:], rtol=1e-12, atol=1e-13)
    assert np.allclose(lse[0, 0], rl[0, 0, n_k - n_q:], rtol=1e-12, atol=1e-13)


def pin_cross_long_queries(n_q=12, n_k=5):
    q, k, v = _rand((n_q, 8), 23), _rand((n_k, 8), 24), _rand((n_k, 8), 25)
    o, lse = A.forward_general(_bh(q), _bh(k), _bh(v), True, 0.35)
    e = n_q - n_k
    assert np.all(o[0, 0, :e] == 0.0) and np.all(np.isneginf(lse[0, 0, :e]))
    ro, rl = A.forward(_bh(q[e:]), _bh(k), _bh(v), True, 0.35)
    assert np.allclose(o[0, 0, e:], ro[0, 0], rtol=1e-12, atol=1e-13)
    assert np.allclose(lse[0, 0, e:], rl[0, 0], rtol=1e-12, atol=1e-13)


def pin_alibi_closed_form(causal):
    n, slope = 11, 0.375
    q, k = np.zeros((n, 4)), _rand((n, 4), 26)
    v = np.eye(n)  # O_i is row i of P
    o, lse = A.forward_general(_bh(q), _bh(k), _bh(v), causal, 0.5, slopes=[slope])
    r = math.exp(-slope)
    for i in range(n):
        # sum over distances t = 0..i (keys at or before i), and t = 1..n-1-i after
        z = (1 - r ** (i + 1)) / (1 - r)
        if not causal:
            z += r * (1 - r ** (n - 1 - i)) / (1 - r)
        assert abs(lse[0, 0, i] - math.log(z)) < 1e-13, i
        for j in range(n):
            want = 0.0 if (causal and j > i) else r ** abs(i - j) / z
            assert abs(o[0, 0, i, j] - want) < 1e-14, (i, j)


def pin_alibi_extra_dimension(n=14, d=6, slope=0.7):
    q, k, v = _rand((n, d), 27), _rand((n, d), 28), _rand((n, d), 29)
    scale = 0.4
    s32 = A.scale_as_f32(scale)
    o, lse = A.forward_general(_bh(q), _bh(k), _bh(v), True, scale, slopes=[slope])
    q1 = np.concatenate([q, np.ones((n, 1))], axis=1)
    k1 = np.concatenate([k, (float(np.float32(slope)) * np.arange(n) / s32)[:, None]], axis=1)
    ro, rl = A.forward(_bh(q1), _bh(k1), _bh(v), True, scale)
    assert np.allclose(o[0, 0], ro[0, 0], rtol=1e-11, atol=1e-12)
    assert np.allclose(lse[0, 0], rl[0, 0] - float(np.float32(slope)) * np.arange(n), rtol=1e-11, atol=1e-11)


GENERAL_CASES = [  # (n_q, n_k, causal, window, alibi, H, Hkv)
    (6, 6, False, (2, 1), False, 2, 1),
    (4, 7, True, (3, -1), True, 2, 2),
    (7, 4, True, (-1, -1), True, 4, 2),
    (5, 5, False, (-1, 0), True, 1, 1),
    (6, 9, False, (1, 2), False, 2, 1),
]


def _general_inputs(n_q, n_k, H, Hkv, d, seed):
    q, do = _rand((1, H, n_q, d), seed), _rand((1, H, n_q, d), seed + 1)
    k, v = _rand((1, Hkv, n_k, d), seed + 2), _rand((1, Hkv, n_k, d), seed + 3)
    return q, k, v, do


def pin_finite_differences_general(case, d=3):
    n_q, n_k, causal, window, alibi, H, Hkv = case
    q, k, v, do = _general_inputs(n_q, n_k, H, Hkv, d, 30)
    slopes = [0.25 * (h + 1) for h in range(H)] if alibi else None
    scale = 0.6

    def loss(q_, k_, v_):
        o, _ = A.forward_general(q_, k_, v_, causal, scale, window, slopes)
        return float((o * do).sum())

    dq, dk, dv = A.backward_general(q, k, v, do, causal, scale, window, slopes)
    eps = 1e-6
    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-7), (case, which, np.abs(g - num).max())


def pin_torch_masked_sdpa(case, d=5):
    n_q, n_k, causal, window, alibi, H, Hkv = case
    q, k, v, do = _general_inputs(n_q, n_k, H, Hkv, d, 40)
    slopes = [0.3 * (h + 1) for h in range(H)] if alibi else None
    scale = 0.45
    o, lse = A.forward_general(q, k, v, causal, scale, window, slopes)
    dq, dk, dv = A.backward_general(q, k, v, do, causal, scale, window, slopes)
    vis = A.visible(n_q, n_k, causal, window)
    live = vis.any(axis=1)
    g = H // Hkv
    # torch: explicit float mask (0 or -inf, plus the bias), rows that see nothing dropped
    mask = np.where(vis, 0.0, -np.inf)[None].repeat(H, 0)
    if alibi:
        for h in range(H):
            mask[h] += A.alibi_bias(n_q, n_k, slopes[h])
    tq = torch.tensor(q[:, :, live], requires_grad=True)
    tk = torch.tensor(np.repeat(k, g, axis=1), requires_grad=True)
    tv = torch.tensor(np.repeat(v, g, axis=1), requires_grad=True)
    tm = torch.tensor(mask[:, live][None])
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=A.scale_as_f32(scale))
    to.backward(torch.tensor(do[:, :, live]))
    assert np.allclose(o[:, :, live], to.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(o[:, :, ~live] == 0.0) and np.all(np.isneginf(lse[:, :, ~live]))
    tl = torch.logsumexp(A.scale_as_f32(scale) * (tq.detach() @ tk.detach().transpose(-1, -2)) + tm, -1)
    assert np.allclose(lse[:, :, live], tl.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dq[:, :, live], tq.grad.numpy(), rtol=1e-10, atol=1e-10)
    assert np.all(dq[:, :, ~live] == 0.0)
    tdk = tk.grad.numpy().reshape(1, Hkv, g, n_k, d).sum(axis=2)
    tdv = tv.grad.numpy().reshape(1, Hkv, g, n_k, d).sum(axis=2)
    assert np.allclose(dk, tdk, rtol=1e-10, atol=1e-10)
    assert np.allclose(dv, tdv, rtol=1e-10, atol=1e-10)


# ------------------------------------------------------------------ tests
def test_w1_window_sets_by_hand():
    pin_window_sets()


def test_w2_window_zero():
    pin_window_zero()


@pytest.mark.parametrize("n_q,n_k,window,causal", [
    (13, 13, (3, 2), False), (13, 13, (4, -1), True), (7, 15, (2, 3), False), (15, 7, (-1, 1), False),
    (10, 10, (0, 5), True), (8, 8, (-1, 0), False)])
def test_w3_window_rows_are_slices(n_q, n_k, window, causal):
    pin_window_slices(n_q, n_k, window, causal)


def test_x1_cross_attention_short_queries():
    pin_cross_short_queries()


def test_x2_cross_attention_long_queries():
    pin_cross_long_queries()


@pytest.mark.parametrize("causal", [False, True])
def test_a1_alibi_closed_form(causal):
    pin_alibi_closed_form(causal)


def test_a2_alibi_extra_dimension():
    pin_alibi_extra_dimension()


@pytest.mark.parametrize("case", GENERAL_CASES)
def test_d1_finite_differences(case):
    pin_finite_differences_general(case)


@pytest.mark.parametrize("case", GENERAL_CASES)
def test_d2_torch_masked_sdpa(case):
    pin_torch_masked_sdpa(case)


def test_general_reduces_to_plain():
    q, k, v, do = (_rand((2, 3, 10, 4), s) for s in (50, 51, 52, 53))
    for causal in (False, True):
        o1, l1 = A.forward_general(q, k, v, causal, 0.3)
        o2, l2 = A.forward(q, k, v, causal, 0.3)
        assert np.allclose(o1, o2, rtol=1e-14, atol=1e-15) and np.allclose(l1, l2, rtol=1e-14, atol=1e-15)
        g1 = A.backward_general(q, k, v, do, causal, 0.3)
        g2 = A.backward(q, k, v, do, causal, 0.3)
        for a, b in zip(g1, g2):
            assert np.allclose(a, b, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("case", GENERAL_CASES)
def test_sampled_general_matches_full(case):
    n_q, n_k, causal, window, alibi, H, Hkv = case
    q, k, v, do = _general_inputs(n_q, n_k, H, Hkv, 4, 60)
    slopes = [0.2 * (h + 1) for h in range(H)] if alibi else None
    o, lse = A.forward_general(q, k, v, causal, 0.5, window, slopes)
    dq, dk, dv = A.backward_general(q, k, v, do, causal, 0.5, window, slopes)
    g = H // Hkv
    rows, cols = np.arange(n_q), np.arange(n_k)
    for h in range(H):
        hk = h // g
        sl = None if slopes is None else slopes[h]
        ro, rl, rq = A.general_head_rows(q[0, h], k[0, hk], v[0, hk], do[0, h], rows, causal, 0.5, window, sl)
        assert np.allclose(ro, o[0, h], rtol=1e-13, atol=1e-14) and np.allclose(rq, dq[0, h], rtol=1e-12, atol=1e-13)
        assert np.array_equal(np.isneginf(rl), np.isneginf(lse[0, h]))
    for hk in range(Hkv):
        sk, sv = np.zeros((n_k, 4)), np.zeros((n_k, 4))
        for h in range(hk * g, (hk + 1) * g):
            sl = None if slopes is None else slopes[h]
            a, b = A.general_head_cols(q[0, h], k[0, hk], v[0, hk], do[0, h], cols, causal, 0.5, window, sl, chunk=3)
            sk += a
            sv += b
        assert np.allclose(sk, dk[0, hk], rtol=1e-12, atol=1e-13) and np.allclose(sv, dv[0, hk], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ planted mistakes
_visible = A.visible
_alibi = A.alibi_bias
_softmax = A.softmax_rows_or_empty


def _window_exclusive(n_q, n_k, causal, window=(-1, -1)):
    """Off by one: the window's left edge excluded."""
    left, right = window
    w = (left - 1 if left > 0 else left, right)
    return _visible(n_q, n_k, causal, w)


def _top_left(n_q, n_k, causal, window=(-1, -1)):
    """Wrong alignment: query i aligned with key i."""
    vis = np.ones((n_q, n_k), dtype=bool)
    i, j = np.arange(n_q)[:, None], np.arange(n_k)[None, :]
    if causal:
        vis &= j <= i
    left, right = window
    if left >= 0:
        vis &= j >= i - left
    if right >= 0:
        vis &= j <= i + right
    return vis


def _alibi_wrong_sign(n_q, n_k, slope):
    return -_alibi(n_q, n_k, slope)


def _alibi_signed(n_q, n_k, slope):
    """No absolute value: a reward for keys after the diagonal."""
    diag = np.arange(n_q)[:, None] + (n_k - n_q)
    return -float(np.float32(slope)) * (diag - np.arange(n_k)[None, :])


def _empty_rows_uniform(s):
    """Hidden rows averaged over every key instead of giving zero."""
    empty = np.isneginf(s).all(axis=1)
    s = np.where(empty[:, None], 0.0, s)
    return _softmax(s)


@pytest.mark.parametrize("target,replacement,pins", [
    ("visible", _window_exclusive, ["sets", "slices"]),
    ("visible", _top_left, ["cross_short", "cross_long", "window_zero"]),
    ("alibi_bias", _alibi_wrong_sign, ["alibi", "alibi_dim"]),
    ("alibi_bias", _alibi_signed, ["alibi_noncausal"]),
    ("softmax_rows_or_empty", _empty_rows_uniform, ["cross_long", "sets"]),
])
def test_planted_mistakes_are_caught(monkeypatch, target, replacement, pins):
    monkeypatch.setattr(A, target, replacement)
    runners = {
        "sets": pin_window_sets,
        "slices": lambda: pin_window_slices(13, 13, (3, 2), False),
        "cross_short": pin_cross_short_queries,
        "cross_long": pin_cross_long_queries,
        "window_zero": pin_window_zero,
        "alibi": lambda: pin_alibi_closed_form(True),
        "alibi_noncausal": lambda: pin_alibi_closed_form(False),
        "alibi_dim": pin_alibi_extra_dimension,
    }
    for name in pins:
        with pytest.raises((AssertionError, ValueError, FloatingPointError)):
            runners[name]()
