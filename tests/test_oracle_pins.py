"""Pins for the fp64 oracle: checks against facts the pages and the mathematics
fix, none of which re-types the oracle's own formula.

Pin list (each test names what it pins):
  P-1 two-pass softmax == online recurrence for any key partition
  P-2 rows of P sum to 1
  P-3 Q = 0 gives the mean of the visible V rows, LSE = log(#visible)
  P-4 LSE == scipy.special.logsumexp of the score row
  P-5 finite differences of L = sum(O * dO) match the analytic gradients
  P-6 torch SDPA (CPU, float64) and torch.autograd agree with O, dQ, dK, dV
  P-7 special cases (N = 1, causal row 0, V shift / scale, key permutation)
  P-8 D = rowsum(dO o O) equals rowsum(P o dP) when O = P V (and a closed form)
  G-1 hand-derived closed-form example (tests/golden/tiny_closed_form.json)
  Planted mistakes: each plausible bug in the oracle fails at least one pin.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ------------------------------------------------------------------ pins as functions
def pin_online_equals_two_pass(causal):
    q, k, v = (_rand((37, 16), s) for s in (1, 2, 3))
    o_ref, lse_ref = A.forward_head(q, k, v, causal, 0.25)
    for edges in ([0, 37], list(range(38)), [0, 5, 6, 20, 37], [0, 16, 32, 37], [0, 32, 37]):
        o, lse = A.online_forward_head(q, k, v, causal, 0.25, edges)
        assert np.allclose(o, o_ref, rtol=1e-12, atol=1e-13), edges
        assert np.allclose(lse, lse_ref, rtol=1e-12, atol=1e-13), edges


def pin_rows_sum_to_one(causal):
    q, k = _rand((50, 8), 4), _rand((50, 8), 5)
    p = A.probabilities(q, k, causal, 0.5)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert (p >= 0).all()
    if causal:
        assert np.all(p[np.triu_indices(50, 1)] == 0.0)


def pin_zero_query(causal):
    n, d = 23, 8
    q = np.zeros((1, 1, n, d))
    k = _rand((1, 1, n, d), 6)
    v = _rand((1, 1, n, d), 7)
    o, lse = A.forward(q, k, v, causal, 0.3)
    for i in range(n):
        visible = i + 1 if causal else n
        assert np.allclose(o[0, 0, i], v[0, 0, :visible].mean(axis=0), rtol=1e-12, atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(visible)) < 1e-13


def pin_lse_logsumexp(causal):
    q, k, v = _rand((40, 16), 8), _rand((40, 16), 9), _rand((40, 16), 10)
    scale = 1.0 / math.sqrt(16)
    _, lse = A.forward_head(q, k, v, causal, scale)
    s = float(np.float32(scale)) * (q @ k.T)
    for i in range(40):
        row = s[i, : i + 1] if causal else s[i]
        assert abs(lse[i] - scipy.special.logsumexp(row)) < 1e-12


def pin_finite_differences(n, d, causal):
    rng = np.random.default_rng(100 * n + d)
    q, k, v, do = (rng.standard_normal((1, 1, n, d)) for _ in range(4))
    scale = 0.7
    dq, dk, dv = A.backward(q, k, v, do, causal, scale)

    def loss(q_, k_, v_):
        o, _ = A.forward(q_, k_, v_, causal, scale)
        return float((o * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name] = xp
            args_m[name] = xm
            num[idx] = (loss(**{kk + "_": vv for kk, vv in args_p.items()})
                        - loss(**{kk + "_": vv for kk, vv in args_m.items()})) / (2 * h)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(g), 1e-30)
        assert err < 1e-7 or np.linalg.norm(num - g) < 1e-9, (name, err)


def pin_torch_sdpa(causal, n=33, d=16):
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (_rand((2, 3, n, d), 20 + i) for i in range(4))
    o, _ = A.forward(q, k, v, causal, scale)
    dq, dk, dv = A.backward(q, k, v, do, causal, scale)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=float(np.float32(scale)))
    to.backward(torch.tensor(do, dtype=torch.float64))
    assert np.allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-10)
    assert np.allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-10)
    assert np.allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-10)


def pin_torch_sdpa_gqa(causal, n=17, d=8):
    """Grouped heads: torch's fp64 SDPA with enable_gqa (and its autograd) as the
    independent reference for forward_gqa / backward_gqa; GQA (4 query heads on 2
    key/value heads) and MQA (4 on 1)."""
    scale = 1.0 / math.sqrt(d)
    for hkv in (2, 1):
        q, do = _rand((2, 4, n, d), 40), _rand((2, 4, n, d), 41)
        k, v = _rand((2, hkv, n, d), 42), _rand((2, hkv, n, d), 43)
        o, lse = A.forward_gqa(q, k, v, causal, scale)
        dq, dk, dv = A.backward_gqa(q, k, v, do, causal, scale)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=float(np.float32(scale)), enable_gqa=True)
        to.backward(torch.tensor(do, dtype=torch.float64))
        assert dk.shape == k.shape and dv.shape == v.shape
        assert np.allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-10)
        assert np.allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-10)
        assert np.allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-10)


def pin_special_cases():
    # N = 1: O = V, LSE = s q.k
    q, k, v = _rand((1, 1, 1, 8), 30), _rand((1, 1, 1, 8), 31), _rand((1, 1, 1, 8), 32)
    for causal in (False, True):
        o, lse = A.forward(q, k, v, causal, 0.125)
        assert np.array_equal(o, v)
        assert abs(lse[0, 0, 0] - 0.125 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-13
    # causal row 0: O_0 = V_0 exactly, LSE_0 = s q0.k0
    q, k, v = _rand((1, 1, 9, 4), 33), _rand((1, 1, 9, 4), 34), _rand((1, 1, 9, 4), 35)
    o, lse = A.forward(q, k, v, True, 0.5)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    assert abs(lse[0, 0, 0] - 0.5 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-14
    # V + 1 c^T -> O + 1 c^T ; alpha V -> alpha O ; joint K/V row permutation (non-causal)
    c = _rand((4,), 36)
    for causal in (False, True):
        o0, _ = A.forward(q, k, v, causal, 0.5)
        o1, _ = A.forward(q, k, v + c, causal, 0.5)
        assert np.allclose(o1, o0 + c, atol=1e-13)
        o2, _ = A.forward(q, k, 3.0 * v, causal, 0.5)
        assert np.allclose(o2, 3.0 * o0, atol=1e-13)
    perm = np.random.default_rng(37).permutation(9)
    o0, l0 = A.forward(q, k, v, False, 0.5)
    o3, l3 = A.forward(q, k[:, :, perm], v[:, :, perm], False, 0.5)
    assert np.allclose(o3, o0, atol=1e-13) and np.allclose(l3, l0, atol=1e-13)


def _parse(s):
    s = str(s)
    if s.startswith("ln"):
        return math.log(float(s[2:]))
    if "/" in s:
        a, b = s.split("/")
        return float(a) / float(b)
    return float(s)


def pin_golden_closed_form():
    g = json.load(open(os.path.join(GOLDEN, "tiny_closed_form.json")))
    q = np.array([[_parse(x) for x in r] for r in g["q"]])[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    for key, causal in (("noncausal", False), ("causal", True)):
        o, lse = A.forward(q, k, v, causal, g["scale"])
        o_exp = np.array([[_parse(x) for x in r] for r in g[key]["o"]])
        lse_exp = np.array([_parse(x) for x in g[key]["lse"]])
        assert np.allclose(o[0, 0], o_exp, rtol=0, atol=1e-14), key
        assert np.allclose(lse[0, 0], lse_exp, rtol=0, atol=1e-14), key


def pin_sampled_rows_and_cols(causal):
    n, d = 70, 8
    q, k, v, do = (_rand((n, d), 40 + i) for i in range(4))
    o, lse = A.forward_head(q, k, v, causal, 0.3)
    rows = np.array([0, 5, 69, 33])
    o_r, lse_r = A.forward_head(q, k, v, causal, 0.3, rows)
    assert np.allclose(o_r, o[rows], atol=1e-14) and np.allclose(lse_r, lse[rows], atol=1e-14)
    dq, dk, dv = A.backward_head(q, k, v, do, causal, 0.3)
    assert np.allclose(A.backward_head_rows(q, k, v, do, rows, causal, 0.3), dq[rows], atol=1e-13)
    dk_c, dv_c = A.backward_head_cols(q, k, v, do, rows, causal, 0.3, chunk=16)
    assert np.allclose(dk_c, dk[rows], atol=1e-13) and np.allclose(dv_c, dv[rows], atol=1e-13)


# ------------------------------------------------------------------ tests
@pytest.mark.parametrize("causal", [False, True])
def test_p1_online_recurrence(causal):
    pin_online_equals_two_pass(causal)


@pytest.mark.parametrize("causal", [False, True])
def test_p2_rows_sum_to_one(causal):
    pin_rows_sum_to_one(causal)


@pytest.mark.parametrize("causal", [False, True])
def test_p3_zero_query_mean_of_visible_values(causal):
    pin_zero_query(causal)


@pytest.mark.parametrize("causal", [False, True])
def test_p4_lse_is_logsumexp(causal):
    pin_lse_logsumexp(causal)


@pytest.mark.parametrize("n,d", [(1, 2), (2, 4), (5, 2), (8, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_p5_finite_differences(n, d, causal):
    pin_finite_differences(n, d, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_p6_torch_sdpa_and_autograd(causal):
    pin_torch_sdpa(causal)


@pytest.mark.parametrize("causal", [False, True])
def test_p10_torch_sdpa_gqa(causal):
    pin_torch_sdpa_gqa(causal)


def test_gqa_with_all_heads_is_multi_head():
    q, k, v = _rand((1, 3, 11, 8), 50), _rand((1, 3, 11, 8), 51), _rand((1, 3, 11, 8), 52)
    o1, l1 = A.forward_gqa(q, k, v, True, 0.25)
    o2, l2 = A.forward(q, k, v, True, 0.25)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_p7_special_cases():
    pin_special_cases()


def test_g1_hand_derived_example():
    pin_golden_closed_form()


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_evaluation_matches_full(causal):
    pin_sampled_rows_and_cols(causal)


def test_metrics():
    ref = np.array([3.0, 4.0])
    assert A.rel_rms(ref + np.array([0.3, 0.4]), ref) == pytest.approx(0.1)
    assert A.max_abs(ref + np.array([0.3, -0.5]), ref) == pytest.approx(0.5)


def pin_row_delta(causal):
    """D from O and dO equals sum_j P_ij dP_ij computed from P and dP = dO V^T,
    which is how the chain rule reaches it; plus a hand-computed case."""
    q, k, v, do = (_rand((29, 8), s) for s in (21, 22, 23, 24))
    o, _ = A.forward_head(q, k, v, causal, 0.3)
    p = A.probabilities(q, k, causal, 0.3)
    ref = (p * (do @ v.T)).sum(axis=1)
    assert np.allclose(A.row_delta(o, do), ref, rtol=1e-12, atol=1e-12)
    assert A.row_delta(np.array([[1.0, 2.0], [0.5, -1.0]]), np.array([[3.0, 4.0], [2.0, 2.0]])).tolist() == [11.0, -1.0]


@pytest.mark.parametrize("causal", [False, True])
def test_p8_row_delta(causal):
    pin_row_delta(causal)


# ------------------------------------------------------------------ planted mistakes
def _mask_off_by_one(q, k, scale, causal, rows=None):
    """Causal mask that lets each query see one key too many."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = float(np.float32(scale)) * (q[idx] @ k.T)
    if causal:
        s[np.arange(k.shape[0])[None, :] > idx[:, None] + 1] = -np.inf
    return s


def _scores_unscaled(q, k, scale, causal, rows=None):
    return A.__dict__["_orig_head_scores"](q, k, 1.0, causal, rows)


def _backward_wrong_sign(q, k, v, do, causal, scale):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = float(np.float32(scale))
    p, _, _ = A.safe_softmax_rows(A.head_scores(q, k, scale, causal))
    dp = do @ v.T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp + dd[:, None])
    return s * (ds @ k), s * (ds.T @ q), p.T @ do


def _backward_transposed(q, k, v, do, causal, scale):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = float(np.float32(scale))
    p, _, _ = A.safe_softmax_rows(A.head_scores(q, k, scale, causal))
    dp = do @ v.T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    return s * (ds @ k), s * (ds @ q), p.T @ do


def _backward_no_scale(q, k, v, do, causal, scale):
    dq, dk, dv = A.__dict__["_orig_backward_head"](q, k, v, do, causal, scale)
    return dq / float(np.float32(scale)), dk, dv


def _softmax_no_log(s):
    p, m, l = A.__dict__["_orig_safe_softmax_rows"](s)
    return p, m, np.exp(l)  # LSE would become m + l


def _expand_kv_modulo(x, H):
    """Wrong head mapping: query head h reads key/value head h % H_kv."""
    x = np.asarray(x, dtype=np.float64)
    return np.tile(x, (1, H // x.shape[1], 1, 1))


def _row_delta_over_rows(o, do):
    """Wrong axis: sums dO o O over the rows instead of along d."""
    return (np.asarray(do, np.float64) * np.asarray(o, np.float64)).sum(axis=0)


def _row_delta_o_squared(o, do):
    """Wrong operand: sums O o O along d."""
    return (np.asarray(o, np.float64) ** 2).sum(axis=-1)


def _backward_gqa_first_head(q, k, v, do, causal=False, scale=None):
    """Forgets the group sum: keeps only the first query head's dK, dV."""
    B, H, N, d = q.shape
    g = H // k.shape[1]
    dq, dk, dv = A.backward(q, A.expand_kv(k, H), A.expand_kv(v, H), do, causal, scale)
    return dq, dk[:, ::g], dv[:, ::g]


@pytest.mark.parametrize("target,replacement,pins", [
    ("expand_kv", _expand_kv_modulo, ["sdpa_gqa"]),
    ("backward_gqa", _backward_gqa_first_head, ["sdpa_gqa"]),
    ("head_scores", _mask_off_by_one, ["zero_query", "sdpa", "special"]),
    ("head_scores", _scores_unscaled, ["sdpa", "lse", "golden_scale"]),
    ("backward_head", _backward_wrong_sign, ["fd", "sdpa"]),
    ("backward_head", _backward_transposed, ["fd", "sdpa"]),
    ("backward_head", _backward_no_scale, ["fd", "sdpa"]),
    ("safe_softmax_rows", _softmax_no_log, ["lse", "zero_query", "golden"]),
    ("row_delta", _row_delta_over_rows, ["row_delta"]),
    ("row_delta", _row_delta_o_squared, ["row_delta"]),
])
def test_planted_mistakes_are_caught(monkeypatch, target, replacement, pins):
    """Each planted bug (in the oracle, on the CPU) must fail every listed pin."""
    monkeypatch.setitem(A.__dict__, "_orig_head_scores", A.head_scores)
    monkeypatch.setitem(A.__dict__, "_orig_backward_head", A.backward_head)
    monkeypatch.setitem(A.__dict__, "_orig_safe_softmax_rows", A.safe_softmax_rows)
    monkeypatch.setattr(A, target, replacement)
    runners = {
        "zero_query": lambda: pin_zero_query(True),
        "sdpa": lambda: pin_torch_sdpa(True, n=9, d=4),
        "special": pin_special_cases,
        "lse": lambda: pin_lse_logsumexp(True),
        "fd": lambda: pin_finite_differences(5, 2, True),
        "golden": pin_golden_closed_form,
        "golden_scale": lambda: pin_torch_sdpa(False, n=9, d=4),
        "sdpa_gqa": lambda: pin_torch_sdpa_gqa(True, n=9, d=4),
        "row_delta": lambda: pin_row_delta(True),
    }
    for name in pins:
        with pytest.raises((AssertionError, ValueError, FloatingPointError)):
            runners[name]()


def test_default_scale_is_inverse_sqrt_d():
    """[HUB] "How it works": scores are divided by sqrt(d). Exact values at
    d = 4, 64 and 256, and a forward without a scale equals one with 1/sqrt(d)
    for a hand-checkable case (d = 4, two keys, causal row 1)."""
    assert A.default_scale(4) == 0.5 and A.default_scale(64) == 0.125 and A.default_scale(256) == 0.0625
    q = np.array([[[[2.0, 0.0, 0.0, 0.0], [2.0, 0.0, 0.0, 0.0]]]])
    k = np.array([[[[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]]]])
    v = np.array([[[[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]]]])
    o, lse = A.forward(q, k, v, True)
    # row 1: scores s * (2, 0) = (1, 0) with s = 1/2, so P = (e, 1) / (e + 1)
    e = math.e
    assert np.allclose(o[0, 0, 1], [e / (e + 1), 1 / (e + 1), 0, 0], rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 1] - math.log(e + 1)) < 1e-15
