"""The seeded input generator: deterministic, exact bf16 values, outlier recipe."""

import numpy as np

import fa_inputs


def test_deterministic_and_bf16_exact():
    a = fa_inputs.attention_inputs(1, 2, 100, 64, seed=11, with_do=True)
    b = fa_inputs.attention_inputs(1, 2, 100, 64, seed=11, with_do=True)
    for n in ("q", "k", "v", "do"):
        assert np.array_equal(a[n], b[n])
        bits = a[n].view(np.uint32)
        assert not (bits & 0xFFFF).any()  # low half of every float32 is zero: a bf16 value
    c = fa_inputs.attention_inputs(1, 2, 100, 64, seed=12)
    assert not np.array_equal(a["q"], c["q"])


def test_outliers():
    x = fa_inputs.attention_inputs(1, 2, 500, 64, seed=5, outliers=False)
    y = fa_inputs.attention_inputs(1, 2, 500, 64, seed=5, outliers=True)
    for n in ("q", "k", "v"):
        changed = x[n] != y[n]
        assert changed.sum() == round(0.001 * x[n].size)
        ratio = y[n][changed] / x[n][changed]
        assert np.all(np.abs(ratio - 20.0) < 0.2)  # x20, then bf16 rounding of both sides


def test_signs_and_bits():
    s = fa_inputs.hadamard_signs()
    assert s.dtype == np.int8 and s.shape == (128,) and set(np.unique(s)) == {-1, 1}
    assert np.array_equal(s, fa_inputs.hadamard_signs())
    v = np.array([1.0, -2.5, 0.0], dtype=np.float32)
    assert list(fa_inputs.bf16_bits(v)) == [0x3F80, 0xC020, 0x0000]


def test_grouped_inputs():
    a = fa_inputs.grouped_inputs(2, 8, 2, 33, 64, seed=9, with_do=True)
    assert a["q"].shape == a["do"].shape == (2, 8, 33, 64)
    assert a["k"].shape == a["v"].shape == (2, 2, 33, 64)
    b = fa_inputs.grouped_inputs(2, 8, 2, 33, 64, seed=9, with_do=True)
    for n in a:
        assert np.array_equal(a[n], b[n]) and not (a[n].view(np.uint32) & 0xFFFF).any()
    # with H_kv = H the draws are those of attention_inputs
    c = fa_inputs.grouped_inputs(1, 2, 2, 10, 64, seed=3)
    e = fa_inputs.attention_inputs(1, 2, 10, 64, seed=3)
    assert all(np.array_equal(c[n], e[n]) for n in ("q", "k", "v"))
