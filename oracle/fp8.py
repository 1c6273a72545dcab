"""fp32 emulation of the fp8 (e4m3) input path: Hadamard rotation and block
quantisation, bit-for-bit in the order the kernels use.

Test infrastructure only (see the package docstring for who may import it).

What the pages fix
------------------
[LIB] section "FA3 — the Hopper moment", pillar 3, and [LIN] section "FA3
(2024) — the Hopper masterclass", idea 3: FP8 (E4M3) attention inputs, one
scale per tile of rows instead of one per tensor ("block quantisation"), and
"incoherent processing": multiplying by a random orthogonal Hadamard-based
matrix that spreads outliers before quantising.

Readings where the pages are silent or disagree
-----------------------------------------------
* Format: OCP E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
  largest finite 448, no infinities, 0x7F/0xFF are NaN). Encoding rounds to
  nearest, ties to even, and saturates: a finite input never becomes NaN.
* Block: 128 consecutive token rows x the full head dim of one (batch, head);
  the last block of a head is partial when N % 128 != 0. (One page says 64 x d
  tiles; the 128-row block is the reading used here.)
* Scale: scale = fl32(amax / 448); codes = e4m3(fl32(x * fl32(448 / amax)));
  both divisions correctly rounded fp32, the product one fp32 multiply. A block
  whose amax is 0 gets scale 1 and all-zero codes. Dequantised value =
  decode(code) * scale.
* Rotation: x' = H_128 (s o x) / sqrt(128) along the head dim (d must be 128),
  with H_128 the Sylvester Hadamard matrix and s a vector of 128 random signs;
  the same s for Q and K, V is not rotated. Since H^T H = 128 I and s o s = 1,
  Q' K'^T = Q K^T exactly in real arithmetic. Fixed fp32 order: multiply by s,
  then radix-2 butterflies (a, b) -> (a + b, a - b) at strides 1, 2, 4, ..., 64,
  then one fp32 multiply by fl32(1 / sqrt(128)). No bf16 rounding before the
  quantiser.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK_ROWS = 128


def e4m3_encode(x) -> np.ndarray:
    """Round-to-nearest-even, saturating float32 -> E4M3FN codes (uint8).

    Written from the format definition: subnormals are multiples of 2^-9 below
    2^-6, normals are 2^e (1 + m/8) for e in [-6, 8]. Every step below is exact
    in float64 for float32 inputs, and ``np.rint`` rounds half to even.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.int64)
    sat = a >= E4M3_MAX
    sub = a < 2.0 ** -6
    nor = ~sat & ~sub
    # subnormal range (a carry to 8 lands exactly on the smallest normal code)
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    # normal range
    an = a[nor]
    e = np.floor(np.log2(an)).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    e = np.where(an < np.ldexp(1.0, e), e - 1, e)
    e = np.where(an >= np.ldexp(1.0, e + 1), e + 1, e)
    m = np.rint((an / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code[nor] = ((e + 7) << 3) | m
    code[sat] = 0x7E
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN codes -> exact float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def hadamard_rotate(x, signs) -> np.ndarray:
    """x' = H_128 (s o x) / sqrt(128) along the last axis, in float32, in the
    fixed butterfly order stated in the module docstring."""
    y = np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    n = y.shape[-1]
    if n != 128:
        raise ValueError("rotation is defined for a head dim of 128")
    y = y.copy()
    h = 1
    while h < n:
        z = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        h *= 2
    return (y * np.float32(1.0 / np.sqrt(128.0))).astype(np.float32)


def block_quantize(x):
    """Per (batch, head, 128-row block) quantisation of float32 ``[B,H,N,d]``.

    Returns (codes uint8 ``[B,H,N,d]``, scales float32 ``[B,H,ceil(N/128)]``).
    """
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nb = (N + BLOCK_ROWS - 1) // BLOCK_ROWS
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    for j in range(nb):
        blk = x[:, :, j * BLOCK_ROWS:(j + 1) * BLOCK_ROWS, :]
        amax = np.abs(blk).max(axis=(2, 3)).astype(np.float32)
        zero = amax == 0
        safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
        scale = np.where(zero, np.float32(1.0), (safe / np.float32(E4M3_MAX)).astype(np.float32))
        factor = np.where(zero, np.float32(1.0), (np.float32(E4M3_MAX) / safe).astype(np.float32))
        scales[:, :, j] = scale
        prod = (blk * factor[:, :, None, None].astype(np.float32)).astype(np.float32)
        codes[:, :, j * BLOCK_ROWS:(j + 1) * BLOCK_ROWS, :] = e4m3_encode(prod)
    return codes, scales


def quantize(x, signs=None):
    """The whole input path for one tensor: optional rotation, then block
    quantisation. ``x`` holds bf16 values (as float32 or float64)."""
    x = np.asarray(x, dtype=np.float32)
    if signs is not None:
        x = hadamard_rotate(x, signs)
    return block_quantize(x)


def dequantize(codes, scales) -> np.ndarray:
    """decode(code) * scale in float64 (exact)."""
    codes = np.asarray(codes)
    N = codes.shape[2]
    s = np.repeat(np.asarray(scales, dtype=np.float64), BLOCK_ROWS, axis=2)[:, :, :N]
    return e4m3_decode(codes) * s[..., None]
