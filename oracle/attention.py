"""Attention by definition, in float64, materialising S and P.

Test infrastructure only (see the package docstring for who may import it).

Definitions followed
--------------------
* [HUB] section "How it works": S = Q K^T / sqrt(d), P = softmax(S), O = P V,
  computed as three separate steps; the per-row logsumexp L_i = m_i + log l_i
  is what the fused kernel saves, and the backward pass recomputes
  P_ij = exp(S_ij - L_i) from it.
* [LIB] section "The trick that made it all possible: online softmax": the
  safe softmax (row maximum m subtracted before exponentiating) and the online
  recurrence m' = max(m, m_new), l' = exp(m - m') l + sum exp(x - m'), with
  the partial output rescaled by the same factor; dividing by the final l is
  exact.
* [LIB] section "Cases where FlashAttention does not help": the causal mask
  is one of the masks the kernels ship; grouped-query and multi-query
  attention (GQA/MQA) are supported natively.

Readings where the pages are silent
-----------------------------------
* The scale is an argument; the oracle uses float64(float32(scale)) so that it
  is bit-identical to the float32 scale the kernels receive.
* Causal: query i sees key j iff j <= i (lower triangle, diagonal included,
  N_q == N_k), so no row is ever fully masked.
* LSE uses the natural logarithm of the sum over the *scaled* scores.
* GQA/MQA (the pages name them only): H query heads share H_kv key/value
  heads, query head h reading key/value head h // (H // H_kv) (consecutive
  query heads form a group). The forward is the multi-head definition with
  each shared head repeated; the key/value gradients of a shared head are the
  sums over its group (chain rule through the repetition).
* Backward: the pages only say that P is recomputed from L. The gradients
  below are the derivative of the forward definition (chain rule through the
  softmax): dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij,
  dS = P * (dP - D), dQ = s dS K, dK = s dS^T Q.

Arrays are ``[B, H, N, d]`` (row-major, d fastest); LSE and D are ``[B, H, N]``.
"""

from __future__ import annotations

import math

import numpy as np


def scale_as_f32(scale: float) -> float:
    """The float32 value of ``scale``, widened exactly to float64."""
    return float(np.float32(scale))


def default_scale(d: int) -> float:
    """1/sqrt(d) ([HUB] "How it works")."""
    return 1.0 / math.sqrt(d)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def head_scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool,
                rows: np.ndarray | None = None) -> np.ndarray:
    """S = s Q K^T for one head, with masked entries set to -inf.

    ``rows`` selects query rows (absolute indices) so that large heads can be
    evaluated a few rows at a time; each row of S depends only on its own query.
    """
    q = _f64(q)
    k = _f64(k)
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = scale_as_f32(scale) * (q[idx] @ k.T)
    if causal:
        keys = np.arange(k.shape[0])
        s[keys[None, :] > idx[:, None]] = -np.inf
    return s


def safe_softmax_rows(s: np.ndarray):
    """Row-wise safe softmax: returns (P, m, l) with m the row max and l the
    row sum of exp(S - m) ([LIB] "online softmax", the standard softmax)."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def forward_head(q, k, v, causal: bool, scale: float, rows=None):
    """O and LSE for one head (or for the query rows in ``rows``)."""
    s = head_scores(q, k, scale, causal, rows)
    p, m, l = safe_softmax_rows(s)
    o = p @ _f64(v)
    lse = m + np.log(l)
    return o, lse


def forward(q, k, v, causal: bool = False, scale: float | None = None):
    """Forward for ``[B, H, N, d]`` inputs: returns (O, LSE) in float64."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    o = np.empty((B, H, N, v.shape[-1]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], causal, scale)
    return o, lse


def probabilities(q, k, causal: bool = False, scale: float | None = None):
    """P = softmax(S) for one head (exposed for the row-sum invariant)."""
    if scale is None:
        scale = default_scale(np.shape(q)[-1])
    p, _, _ = safe_softmax_rows(head_scores(q, k, scale, causal))
    return p


def backward_head(q, k, v, do, causal: bool, scale: float):
    """(dQ, dK, dV) for one head by the chain rule through the definition."""
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    s = scale_as_f32(scale)
    p, _, _ = safe_softmax_rows(head_scores(q, k, scale, causal))
    dv = p.T @ do
    dp = do @ v.T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    dq = s * (ds @ k)
    dk = s * (ds.T @ q)
    return dq, dk, dv


def row_delta(o, do) -> np.ndarray:
    """D_i = sum_d dO_id O_id in float64, over the last axis. It is the row term
    of dS = P * (dP - D): with O = P V, sum_d dO_id O_id = sum_j P_ij dP_ij
    (the chain rule through the softmax; the pages only say that the backward
    recomputes P). The kernels form D from their own bf16 O."""
    return (_f64(do) * _f64(o)).sum(axis=-1)


def backward(q, k, v, do, causal: bool = False, scale: float | None = None):
    """Backward for ``[B, H, N, d]`` inputs: returns (dQ, dK, dV) in float64."""
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = backward_head(q[b, h], k[b, h], v[b, h], do[b, h],
                                                         causal, scale)
    return dq, dk, dv


def expand_kv(x, H: int) -> np.ndarray:
    """[B, H_kv, N, d] -> [B, H, N, d]: query head h sees key/value head h // (H // H_kv)."""
    x = _f64(x)
    Hkv = x.shape[1]
    if Hkv < 1 or H % Hkv:
        raise ValueError("H_kv must divide H")
    return np.repeat(x, H // Hkv, axis=1)


def forward_gqa(q, k, v, causal: bool = False, scale: float | None = None):
    """Forward with grouped key/value heads: k, v are [B, H_kv, N, d]."""
    H = q.shape[1]
    return forward(q, expand_kv(k, H), expand_kv(v, H), causal, scale)


def backward_gqa(q, k, v, do, causal: bool = False, scale: float | None = None):
    """Backward with grouped key/value heads: dK, dV summed over each group."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = backward(q, expand_kv(k, H), expand_kv(v, H), do, causal, scale)
    g = H // Hkv
    return dq, dk.reshape(B, Hkv, g, N, d).sum(axis=2), dv.reshape(B, Hkv, g, N, d).sum(axis=2)


# ------------------------------------------- masks, ALiBi, cross-attention
# [LIB] "Cases where FlashAttention does not help" lists the masks and shapes
# the kernels ship beyond causal: sliding windows, ALiBi, cross-attention
# (query and key lengths differ). The pages name them without formulas; the
# readings used here are:
# * diagonal: query i (of N_q) is aligned with key i + N_k - N_q (bottom-right
#   alignment: the last query sits on the last key; N_q = N_k gives i);
# * causal: keys after the diagonal are hidden;
# * window (left, right): only keys within [diagonal - left, diagonal + right]
#   are visible; -1 leaves that side unbounded;
# * ALiBi: the scaled score gets the bias -slope_h * |diagonal - j|, one slope
#   per query head;
# * a query that sees no key at all (possible only with N_q > N_k or a window
#   clear of the keys) has O = 0 and LSE = -inf (log of an empty sum).

def visible(n_q: int, n_k: int, causal: bool, window=(-1, -1)) -> np.ndarray:
    """Boolean [n_q, n_k]: True where query i may attend to key j."""
    diag = np.arange(n_q)[:, None] + (n_k - n_q)
    j = np.arange(n_k)[None, :]
    vis = np.ones((n_q, n_k), dtype=bool)
    left, right = window
    if causal:
        vis &= j <= diag
    if left >= 0:
        vis &= j >= diag - left
    if right >= 0:
        vis &= j <= diag + right
    return vis


def alibi_bias(n_q: int, n_k: int, slope: float) -> np.ndarray:
    """[n_q, n_k] bias -slope |i + n_k - n_q - j| (slope as its float32 value)."""
    diag = np.arange(n_q)[:, None] + (n_k - n_q)
    return -float(np.float32(slope)) * np.abs(diag - np.arange(n_k)[None, :]).astype(np.float64)


def general_scores(q, k, scale: float, causal: bool, window=(-1, -1), slope=None, rows=None):
    """S = s Q K^T (+ ALiBi bias) for one head, hidden entries -inf."""
    q = _f64(q)
    k = _f64(k)
    n_q, n_k = q.shape[0], k.shape[0]
    idx = np.arange(n_q) if rows is None else np.asarray(rows)
    s = scale_as_f32(scale) * (q[idx] @ k.T)
    if slope is not None:
        s = s + alibi_bias(n_q, n_k, slope)[idx]
    s[~visible(n_q, n_k, causal, window)[idx]] = -np.inf
    return s


def softmax_rows_or_empty(s: np.ndarray):
    """Safe softmax per row; a row with no finite score gives P = 0, LSE = -inf."""
    empty = np.isneginf(s).all(axis=1)
    m = np.where(empty, 0.0, s.max(axis=1))
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / np.where(empty, 1.0, l)[:, None]
    lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    return p, lse


def _kv_head(h: int, H: int, Hkv: int) -> int:
    return h // (H // Hkv)


def forward_general(q, k, v, causal: bool = False, scale: float | None = None, window=(-1, -1),
                    slopes=None):
    """(O, LSE) for q [B, H, N_q, d], k, v [B, H_kv, N_k, d] with the masks above;
    ``slopes`` is None or H ALiBi slopes."""
    q, k, v = (_f64(x) for x in (q, k, v))
    B, H, n_q, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = default_scale(d)
    o = np.empty((B, H, n_q, v.shape[-1]))
    lse = np.empty((B, H, n_q))
    for b in range(B):
        for h in range(H):
            hk = _kv_head(h, H, Hkv)
            sl = None if slopes is None else slopes[h]
            p, lse[b, h] = softmax_rows_or_empty(general_scores(q[b, h], k[b, hk], scale, causal, window, sl))
            o[b, h] = p @ v[b, hk]
    return o, lse


def backward_general(q, k, v, do, causal: bool = False, scale: float | None = None, window=(-1, -1),
                     slopes=None):
    """(dQ, dK, dV) for forward_general (slopes are constants, not differentiated);
    dK, dV of a shared key/value head summed over its query heads."""
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    B, H, n_q, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = default_scale(d)
    s = scale_as_f32(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            hk = _kv_head(h, H, Hkv)
            sl = None if slopes is None else slopes[h]
            p, _ = softmax_rows_or_empty(general_scores(q[b, h], k[b, hk], scale, causal, window, sl))
            dv[b, hk] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, hk].T
            dd = (p * dp).sum(axis=1)
            ds = p * (dp - dd[:, None])
            dq[b, h] = s * (ds @ k[b, hk])
            dk[b, hk] += s * (ds.T @ q[b, h])
    return dq, dk, dv


def general_head_rows(q, k, v, do, rows, causal: bool, scale: float, window=(-1, -1), slope=None):
    """O, LSE and dQ of the selected query rows of one head (general masks)."""
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    rows = np.asarray(rows)
    p, lse = softmax_rows_or_empty(general_scores(q, k, scale, causal, window, slope, rows))
    dp = do[rows] @ v.T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    return p @ v, lse, scale_as_f32(scale) * (ds @ k)


def general_head_cols(q, k, v, do, cols, causal: bool, scale: float, window=(-1, -1), slope=None,
                      chunk: int = 1024):
    """(dK, dV) of the selected key rows of one (query head, key/value head) pair."""
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    cols = np.asarray(cols)
    n = q.shape[0]
    dk = np.zeros((cols.size, q.shape[1]))
    dv = np.zeros((cols.size, v.shape[1]))
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        p, _ = softmax_rows_or_empty(general_scores(q, k, scale, causal, window, slope, rows))
        dp = do[rows] @ v.T
        dd = (p * dp).sum(axis=1)
        ds_cols = p[:, cols] * (dp[:, cols] - dd[:, None])
        dv += p[:, cols].T @ do[rows]
        dk += scale_as_f32(scale) * (ds_cols.T @ q[rows])
    return dk, dv


def backward_head_rows(q, k, v, do, rows, causal: bool, scale: float):
    """dQ for the selected query rows of one head.

    Row i of dQ needs only row i of P and dP, so this evaluates large heads a
    few rows at a time. Same formulas as ``backward_head``.
    """
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    rows = np.asarray(rows)
    s = scale_as_f32(scale)
    p, _, _ = safe_softmax_rows(head_scores(q, k, scale, causal, rows))
    dp = do[rows] @ v.T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    return s * (ds @ k)


def backward_head_cols(q, k, v, do, cols, causal: bool, scale: float, chunk: int = 1024):
    """(dK, dV) for the selected key rows of one head.

    Column j of P needs every row's normaliser, so all rows are visited in
    chunks of ``chunk`` queries (row-local softmax, so chunking changes no
    value); only the selected columns of dS and P are kept.
    """
    q, k, v, do = (_f64(x) for x in (q, k, v, do))
    cols = np.asarray(cols)
    s = scale_as_f32(scale)
    n = q.shape[0]
    dk = np.zeros((cols.size, q.shape[1]))
    dv = np.zeros((cols.size, v.shape[1]))
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        p, _, _ = safe_softmax_rows(head_scores(q, k, scale, causal, rows))
        dp = do[rows] @ v.T
        dd = (p * dp).sum(axis=1)
        ds_cols = p[:, cols] * (dp[:, cols] - dd[:, None])
        dv += p[:, cols].T @ do[rows]
        dk += s * (ds_cols.T @ q[rows])
    return dk, dv


def online_forward_head(q, k, v, causal: bool, scale: float, block_edges):
    """Diagnostic: the online recurrence over key blocks ([LIB] "online softmax").

    ``block_edges`` is an increasing list of key offsets starting at 0 and
    ending at N (any partition, ragged allowed). Per block: new running max,
    rescale factor exp(m_old - m_new) applied to l and to the partial output,
    add this block's exp(x - m_new) terms; divide by l at the end. Used only to
    check that the two-pass definition and the recurrence agree.
    """
    q, k, v = (_f64(x) for x in (q, k, v))
    n = q.shape[0]
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, v.shape[1]))
    for j0, j1 in zip(block_edges[:-1], block_edges[1:]):
        s = scale_as_f32(scale) * (q @ k[j0:j1].T)
        if causal:
            keys = np.arange(j0, j1)
            s[keys[None, :] > np.arange(n)[:, None]] = -np.inf
        m_new = np.maximum(m, s.max(axis=1))
        # rows whose running max is still -inf have seen no visible key yet
        alpha = np.where(np.isneginf(m_new), 0.0, np.exp(m - np.where(np.isneginf(m_new), 0.0, m_new)))
        p = np.where(np.isneginf(m_new)[:, None], 0.0,
                     np.exp(s - np.where(np.isneginf(m_new), 0.0, m_new)[:, None]))
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[j0:j1]
        m = m_new
    return acc / l[:, None], m + np.log(l)


# ---------------------------------------------------------------- metrics
def rel_rms(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole tensor."""
    x = _f64(x)
    ref = _f64(ref)
    return float(np.linalg.norm((x - ref).ravel()) / np.linalg.norm(ref.ravel()))


def max_abs(x, ref) -> float:
    return float(np.max(np.abs(_f64(x) - _f64(ref)))) if np.size(ref) else 0.0
