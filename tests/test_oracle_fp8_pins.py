"""Pins for the fp8 side of the oracle (rotation, codec, block quantiser).

  P-8 the rotation is H_128 diag(s) / sqrt(128) (scipy's Sylvester Hadamard
      matrix), orthogonal, and leaves Q K^T (hence attention) unchanged
  P-9 the e4m3 codec: hand-derived points (tests/golden/e4m3_points.json),
      code -> value -> code round trip for all 256 codes, agreement with
      torch.float8_e4m3fn on in-range values
  Q-1 block quantiser: amax maps to the largest code, the error bound of
      round-to-nearest holds element by element, zero blocks, ragged blocks
  Planted mistakes in the codec and the butterflies fail these pins.
"""

import json
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import attention as A
from oracle import fp8 as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _signs(seed=3):
    return (np.random.default_rng(seed).integers(0, 2, 128) * 2 - 1).astype(np.int8)


# ------------------------------------------------------------------ pins as functions
def pin_rotation_matrix():
    s = _signs()
    rot = F.hadamard_rotate(np.eye(128, dtype=np.float32), s).astype(np.float64)  # rows: e_i -> M e_i
    expect = (scipy.linalg.hadamard(128) * s[None, :]).T / np.sqrt(128.0)
    # each entry is +-fl32(1/sqrt(128)) exactly
    assert np.array_equal(np.abs(rot), np.full((128, 128), float(np.float32(1 / np.sqrt(128.0)))))
    assert np.allclose(rot, expect, rtol=1e-7, atol=0)
    assert np.allclose(rot @ rot.T, np.eye(128), atol=1e-6)
    x = np.random.default_rng(4).standard_normal((7, 128)).astype(np.float32)
    y = F.hadamard_rotate(x, s).astype(np.float64)
    ref = (x.astype(np.float64) * s) @ scipy.linalg.hadamard(128).T / np.sqrt(128.0)
    assert np.allclose(y, ref, rtol=0, atol=1e-5 * np.abs(ref).max())


def pin_rotation_preserves_attention():
    s = _signs(5)
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, 1, 64, 128)).astype(np.float32) for _ in range(3))
    o0, l0 = A.forward(q, k, v, True, 128 ** -0.5)
    o1, l1 = A.forward(F.hadamard_rotate(q, s), F.hadamard_rotate(k, s), v, True, 128 ** -0.5)
    assert A.rel_rms(o1, o0) < 1e-5 and np.max(np.abs(l1 - l0)) < 1e-4


def pin_codec_golden():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_points.json")))
    vals = np.array([float(p[0]) for p in g["points"]], dtype=np.float32)
    codes = F.e4m3_encode(vals)
    for p, c in zip(g["points"], codes):
        assert int(c) == int(p[1], 16), (p, hex(int(c)))


def pin_codec_roundtrip_and_torch():
    all_codes = np.arange(256, dtype=np.uint8)
    vals = F.e4m3_decode(all_codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254
    back = F.e4m3_encode(vals[finite].astype(np.float32))
    assert np.array_equal(back, all_codes[finite])
    assert np.nanmax(vals) == 448.0 and np.nanmin(vals) == -448.0
    # torch's decoder agrees on every finite code
    tv = torch.from_numpy(all_codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(tv[finite], vals[finite])
    # torch's RNE cast agrees on in-range float32 inputs spanning all binades
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000) * np.exp2(rng.uniform(-12, 9, 200000))).astype(np.float32)
    x = np.clip(x, -448, 448).astype(np.float32)
    # plus every exact midpoint between neighbouring codes (the ties)
    pos = np.unique(vals[finite & (vals >= 0)])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    tc = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(x), tc)


def pin_block_quantiser():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 3, 300, 64)).astype(np.float32)
    x[0, 1, 128:256] = 0.0          # an all-zero block
    x[1, 2, 5, 7] = 40.0            # an outlier
    codes, scales = F.block_quantize(x)
    assert codes.shape == x.shape and scales.shape == (2, 3, 3)
    assert scales[0, 1, 1] == 1.0 and not codes[0, 1, 128:256].any()
    deq = F.dequantize(codes, scales)
    for b in range(2):
        for h in range(3):
            for j in range(3):
                blk = x[b, h, 128 * j:128 * (j + 1)].astype(np.float64)
                amax = np.abs(blk).max()
                if amax == 0:
                    continue
                assert abs(scales[b, h, j] - amax / 448.0) <= 2 ** -23 * amax / 448.0
                c = codes[b, h, 128 * j:128 * (j + 1)]
                at = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
                assert (int(c[at]) & 0x7F) == 0x7E
                err = np.abs(deq[b, h, 128 * j:128 * (j + 1)] - blk)
                bound = np.maximum(2.0 ** -4 * np.abs(blk), 2.0 ** -10 * scales[b, h, j]) * (1 + 1e-6)
                assert np.all(err <= bound)


# ------------------------------------------------------------------ tests
def test_p8_rotation_matrix():
    pin_rotation_matrix()


def test_p8_rotation_preserves_attention():
    pin_rotation_preserves_attention()


def test_p9_codec_golden_points():
    pin_codec_golden()


def test_p9_codec_roundtrip_and_torch():
    pin_codec_roundtrip_and_torch()


def test_q1_block_quantiser():
    pin_block_quantiser()


def test_quantize_with_rotation_requires_d128():
    with pytest.raises(ValueError):
        F.quantize(np.zeros((1, 1, 4, 64), np.float32), _signs())


# ------------------------------------------------------------------ planted mistakes
class _RoundHalfAwayNumpy:
    """numpy with rint replaced by round-half-away-from-zero."""

    def __getattr__(self, name):
        return getattr(np, name)

    @staticmethod
    def rint(x):
        return np.sign(x) * np.floor(np.abs(x) + 0.5)


def _encode_ties_away(x):
    return F.__dict__["_orig_encode"](x)


def _encode_no_saturation(x):
    x = np.asarray(x, dtype=np.float32)
    c = F.__dict__["_orig_encode"](x)
    big = np.abs(x.astype(np.float64)) >= 464.0
    return np.where(big, c | 0x7F, c).astype(np.uint8)


def _rotate_swapped_butterfly(x, signs):
    y = np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    n = y.shape[-1]
    y = y.copy()
    h = 1
    while h < n:
        z = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a - b
        z[..., 1, :] = a + b
        y = z.reshape(y.shape)
        h *= 2
    return (y * np.float32(1.0 / np.sqrt(128.0))).astype(np.float32)


@pytest.mark.parametrize("target,replacement,pins", [
    ("e4m3_encode", _encode_ties_away, ["golden", "torch"]),
    ("e4m3_encode", _encode_no_saturation, ["golden"]),
    ("hadamard_rotate", _rotate_swapped_butterfly, ["matrix"]),
])
def test_planted_mistakes_are_caught(monkeypatch, target, replacement, pins):
    monkeypatch.setitem(F.__dict__, "_orig_encode", F.e4m3_encode)
    monkeypatch.setattr(F, target, replacement)
    if replacement is _encode_ties_away:
        monkeypatch.setattr(F, "np", _RoundHalfAwayNumpy())
    runners = {"golden": pin_codec_golden, "torch": pin_codec_roundtrip_and_torch,
               "matrix": pin_rotation_matrix}
    for name in pins:
        with pytest.raises(AssertionError):
            runners[name]()
