"""The fp8 forward's software 2^x (exp_mode 1 and 2), checked on the CPU:
its polynomial's coefficients are read from the kernel source and the
function is emulated in fp32, step for step (range reduction by adding
1.5 * 2^23, a degree-4 polynomial for 2^f on [-1/2, 1/2] in Horner form with
fused multiply-adds, 2^n added into the exponent field, 0 below -126). The
relative error bound that the kernel's documentation states (2.7e-6 over
[-125.5, 8]) is what the GPU tests' LSE tolerance between exponential modes
rests on."""

import math
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "exact_attention_104_amd", "csrc", "fa_fp8.hip")
f32 = np.float32


def _coefficients():
    text = open(SRC).read()
    body = text[text.index("float soft_exp2(float x)"):]
    body = body[:body.index("\n}")]
    return [float(c) for c in re.findall(r"(\d\.\d+)f", body)]


def _fma32(a, b, c):
    # a * b is exact in fp64 for fp32 operands; one rounding of the sum to fp32
    return (a.astype(np.float64) * b + c).astype(f32)


def _soft_exp2(x):
    c4, c3, c2, c1, c0 = (f32(v) for v in _coefficients())
    x = x.astype(f32)
    xc = np.maximum(x, f32(-126.0))
    t = (xc + f32(12582912.0)).astype(f32)
    f = (xc - (t - f32(12582912.0)).astype(f32)).astype(f32)
    p = _fma32(np.full_like(f, c4), f, c3)
    p = _fma32(p, f, c2)
    p = _fma32(p, f, c1)
    p = _fma32(p, f, c0)
    r = (p.view(np.uint32) + (t.view(np.uint32) << np.uint32(23))).view(f32)
    return np.where(x < f32(-126.0), f32(0.0), r)


def test_coefficients_are_the_documented_five():
    c = _coefficients()
    assert len(c) == 5
    # 2^f = exp(f ln 2): the fit stays close to the Taylor coefficients
    taylor = [math.log(2) ** k / math.factorial(k) for k in (4, 3, 2, 1, 0)]
    assert all(abs(a - b) <= 0.02 * max(abs(b), 1e-3) + 2e-3 for a, b in zip(c, taylor))


def test_relative_error_within_the_stated_bound():
    x = np.linspace(-126.0, 8.0, 4_000_001, dtype=np.float64).astype(f32)
    y = _soft_exp2(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    ok = x > -125.5  # below, 2^n with n = -126 leaves the normal range
    rel = np.abs(y[ok] - ref[ok]) / ref[ok]
    assert rel.max() <= 2.75e-6, rel.max()
    # near-unbiased: the least-squares fit
    assert abs(np.mean((y[ok] - ref[ok]) / ref[ok])) < 1e-7


def test_integers_and_masked_scores():
    n = np.arange(-120, 9, dtype=np.float32)
    y = _soft_exp2(n).astype(np.float64)
    assert np.all(np.abs(y / np.exp2(n.astype(np.float64)) - 1) <= 1e-6)
    assert np.all(_soft_exp2(np.array([-np.inf, -1e30, -127.0, -126.5], dtype=np.float32)) == 0)
