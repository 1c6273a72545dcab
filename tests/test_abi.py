"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments before touching the GPU."""

import ctypes
import os
import re

import pytest
import torch

import exact_attention_104_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

P = 0x10000  # a 16-byte aligned, non-null fake address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def declared_status_codes():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(FA_[A-Z_]+)\s*=\s*(\d+)", text)}


def test_every_declared_symbol_is_exported_and_bound():
    lib = fa.load_library()
    names = declared_functions()
    assert names == sorted(fa.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert fa.abi_version() == 4
    codes = declared_status_codes()
    assert codes["FA_OK"] == 0 and len(codes) == 11
    for name, val in codes.items():
        assert fa.FA_STATUS[val] == name
        assert fa.status_string(val).startswith(name)
    assert fa.status_string(1234) == "FA_ERR_UNKNOWN"


def test_workspace_bytes():
    lib = fa.load_library()
    n = lib.fa_bwd_workspace_bytes(2, 16, 4096, 128)
    assert n == 2 * 16 * 4096 * 4  # fp32 D per row
    assert lib.fa_bwd_workspace_bytes(1, 1, 3, 64) == 256  # rounded to 256 B
    assert lib.fa_bwd_workspace_bytes(1, 1, 3, 96) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 3, 256) == 256
    assert lib.fa_bwd_workspace_bytes(0, 1, 3, 64) == 0


def test_strided_workspace_bytes():
    lib = fa.load_library()
    for causal in (0, 1):  # H_kv = H: D only, as fa_bwd
        assert lib.fa_bwd_strided_workspace_bytes(2, 16, 16, 4096, 128, causal) == 2 * 16 * 4096 * 4
    # B=1, H=8, H_kv=2, N=256: 4 (batch, K/V head, key block) units, so the whole
    # group of 4 is split: D + fp32 dK, dV partials of 2 x 1 x 2 x 4 x 256 x 64
    assert lib.fa_bwd_strided_workspace_bytes(1, 8, 2, 256, 64, 1) == 8 * 256 * 4 + 2 * 2 * 4 * 256 * 64 * 4
    # B=2, H=16, H_kv=2, N=8192: 256 units; causal splits the group of 8 in 4
    assert lib.fa_bwd_strided_workspace_bytes(2, 16, 2, 8192, 128, 1) == \
        2 * 16 * 8192 * 4 + 2 * 2 * 2 * 4 * 8192 * 128 * 4
    assert lib.fa_bwd_strided_workspace_bytes(2, 16, 2, 8192, 128, 0) == 2 * 16 * 8192 * 4
    assert lib.fa_bwd_strided_workspace_bytes(1, 8, 3, 256, 64, 1) == 0   # H_kv does not divide H
    assert lib.fa_bwd_strided_workspace_bytes(1, 8, 2, 256, 64, 2) == 0   # causal not 0 / 1
    assert lib.fa_bwd_strided_workspace_bytes(1, 8, 2, 256, 96, 0) == 0


def _fwd(**kw):
    a = dict(q=P, k=P + 0x100000, v=P + 0x200000, o=P + 0x300000, lse=P + 0x400000,
             B=1, H=1, N=64, d=64, causal=0, scale=0.125, stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                                    a["d"], a["causal"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(causal=2), 9), (dict(scale=float("nan")), 9), (dict(scale=0.0), 9), (dict(scale=-1.0), 9),
    (dict(q=None), 1), (dict(lse=None), 1),
    (dict(d=96), 3), (dict(d=192), 3), (dict(d=512), 3),
    (dict(B=0), 2), (dict(N=0), 2), (dict(H=-1), 2), (dict(N=(1 << 24) + 1), 2),
    (dict(k=P + 8), 4), (dict(lse=P + 0x400004), 4),
    (dict(o=P), 7), (dict(lse=P + 0x100000 + 64), 7), (dict(o=P + 0x200000 + 0x10), 7),
])
def test_fwd_rejects_bad_arguments(kw, status):
    assert _fwd(**kw) == status


def test_bwd_quant_fp8_reject_bad_arguments():
    lib = fa.load_library()
    ws = 0x40000000
    good = [P + i * 0x100000 for i in range(9)]
    args = good + [1, 1, 64, 64, 1, 0.125, ws, lib.fa_bwd_workspace_bytes(1, 1, 64, 64), None]
    bad = list(args)
    bad[15] = ws + 16                   # misaligned workspace
    assert lib.fa_bwd(*bad) == 5
    bad = list(args)
    bad[16] = 100                       # too small
    assert lib.fa_bwd(*bad) == 5
    bad = list(args)
    bad[6] = good[0]                    # dq aliases q
    assert lib.fa_bwd(*bad) == 7
    bad = list(args)
    bad[5] = None
    assert lib.fa_bwd(*bad) == 1
    # quantiser: rotation needs d = 128; NULL output; misalignment
    assert lib.fa_quant_fp8(P, P + 0x100000, P + 0x200000, P + 0x300000, 1, 1, 64, 64, None) == 3
    assert lib.fa_quant_fp8(P, None, P + 0x200000, None, 1, 1, 64, 64, None) == 1
    assert lib.fa_quant_fp8(P, P + 0x100000 + 4, P + 0x200000, None, 1, 1, 64, 64, None) == 4
    assert lib.fa_quant_fp8(P, P + 0x40, P + 0x200000, None, 1, 1, 64, 64, None) == 7
    # the rotation's signs are 16-byte aligned like every tensor
    assert lib.fa_quant_fp8(P, P + 0x100000, P + 0x200000, P + 0x300000 + 8, 1, 1, 64, 128, None) == 4
    f8 = [P + i * 0x100000 for i in range(8)]
    assert lib.fa_fwd_fp8(*f8[:7], None, 1, 1, 64, 64, 0, 0.125, None) == 1
    assert lib.fa_fwd_fp8(*f8, 1, 1, 64, 80, 0, 0.125, None) == 3
    # software-exponential mode: 0, 1 or 2, and 1 or 2 only at d = 128
    for mode in (-1, 3):
        assert lib.fa_fwd_fp8_ext(*f8, 1, 1, 64, 128, 0, 0.125, mode, None) == 9
    assert lib.fa_fwd_fp8_ext(*f8, 1, 1, 64, 64, 0, 0.125, 1, None) == 3
    assert lib.fa_fwd_fp8_ext(*f8, 1, 1, 64, 64, 0, 0.125, 2, None) == 3
    assert lib.fa_fwd_fp8_ext(*f8[:7], None, 1, 1, 64, 128, 0, 0.125, 1, None) == 1


def _st(*triples):
    arr = (fa.Strides * len(triples))()
    for i, t in enumerate(triples):
        arr[i] = fa.Strides(*t)
    return arr


def test_strided_entry_points_reject_bad_arguments():
    """Every call below fails host validation before any HIP call."""
    lib = fa.load_library()
    B, H, N, d = 1, 4, 64, 64
    c = (H * N * d, N * d, d)               # contiguous [B, H, N, d]
    ckv = (2 * N * d, N * d, d)             # contiguous [B, 2, N, d]
    q, k, v, o, lse = (P + i * 0x100000 for i in range(5))

    def fwd(st, Hkv=2, **kw):
        a = dict(q=q, k=k, v=v, o=o, lse=lse, B=B, H=H, Hkv=Hkv, N=N, d=d, st=st, causal=1, scale=0.125)
        a.update(kw)
        return lib.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["N"],
                                  a["d"], a["st"], a["causal"], a["scale"], None)
    good = _st(c, ckv, ckv, c)
    assert fwd(None) == 1                                   # no strides
    assert fwd(good, Hkv=3) == 2                            # H_kv does not divide H
    assert fwd(good, Hkv=0) == 2
    assert fwd(_st(c, ckv, ckv, (c[0], c[1], 0))) == 9      # row stride 0
    assert fwd(_st(c, (ckv[0], ckv[1], 1 << 31), ckv, c)) == 9  # row stride 2^31
    assert fwd(_st(c, ckv, (ckv[0], ckv[1], d + 4), c)) == 4  # rows not on 16-byte boundaries
    assert fwd(_st(c, ckv, ckv, (c[0], 8, d))) == 7         # o overlaps itself (heads 8 elements apart)
    assert fwd(good, o=q) == 7                              # o aliases q
    assert fwd(good, d=96) == 3
    # [B, N, H, d] strides for q and o, grouped K/V: accepted up to the device check,
    # which only a machine without a GPU reaches (see below)
    bwd_st = _st(c, ckv, ckv, c, c, c, ckv, ckv)
    ws = 0x40000000
    ptrs = [P + i * 0x100000 for i in range(9)]
    args = ptrs + [B, H, 2, N, d, bwd_st, 1, 0.125, ws, lib.fa_bwd_strided_workspace_bytes(B, H, 2, N, d, 1), None]
    bad = list(args)
    bad[14] = None
    assert lib.fa_bwd_strided(*bad) == 1
    bad = list(args)
    bad[11] = 3                                             # H_kv = 3 does not divide 4
    assert lib.fa_bwd_strided(*bad) == 2
    bad = list(args)
    bad[14] = _st(c, ckv, ckv, c, c, c, (ckv[0], 8, d), ckv)  # dk overlaps itself
    assert lib.fa_bwd_strided(*bad) == 7
    bad = list(args)
    bad[8] = ptrs[7]                                        # dv aliases dk
    assert lib.fa_bwd_strided(*bad) == 7
    bad = list(args)
    bad[17] = ws + 8                                        # misaligned workspace
    assert lib.fa_bwd_strided(*bad) == 5
    bad = list(args)
    bad[18] = lib.fa_bwd_workspace_bytes(B, H, N, d)        # no room for the partials
    assert lib.fa_bwd_strided(*bad) == 5


@pytest.mark.skipif(torch.cuda.is_available(), reason="valid-looking fake pointers must never reach a GPU")
def test_strided_no_device_is_reported_after_validation():
    lib = fa.load_library()
    B, H, N, d = 2, 4, 64, 64
    bnhd = (N * H * d, d, H * d)                            # [B, N, H, d] viewed as [B, H, N, d]
    kv = (N * 2 * d, d, 2 * d)
    st = _st(bnhd, kv, kv, bnhd)
    ptrs = [P + i * 0x100000 for i in range(5)]
    assert lib.fa_fwd_strided(*ptrs, B, H, 2, N, d, st, 1, 0.125, None) == 6


@pytest.mark.skipif(torch.cuda.is_available(), reason="valid-looking fake pointers must never reach a GPU")
def test_no_device_is_reported_after_validation():
    assert _fwd() == 6


def _mask(causal=0, left=-1, right=-1, slopes=None):
    return ctypes.byref(fa.Mask(causal, left, right, slopes))


def test_ext_entry_points_reject_bad_arguments():
    """fa_fwd_ext / fa_bwd_ext: every call below fails host validation first."""
    lib = fa.load_library()
    B, H, Hkv, Nq, Nk, d = 1, 4, 2, 48, 80, 64
    cq, ck = (H * Nq * d, Nq * d, d), (Hkv * Nk * d, Nk * d, d)
    q, k, v, o, lse = (P + i * 0x100000 for i in range(5))
    sl = P + 0x600000

    def fwd(mask, **kw):
        a = dict(q=q, k=k, v=v, o=o, lse=lse, Nq=Nq, Nk=Nk, st=_st(cq, ck, ck, cq))
        a.update(kw)
        return lib.fa_fwd_ext(a["q"], a["k"], a["v"], a["o"], a["lse"], B, H, Hkv, a["Nq"], a["Nk"], d, a["st"],
                              mask, 0.125, None)
    assert fwd(_mask(2)) == 9                               # causal not 0 / 1
    assert fwd(_mask(0, -2)) == 9                           # window side below -1
    assert fwd(_mask(0, 3, (1 << 24) + 1)) == 9             # window side above 2^24
    assert fwd(_mask(0, 3, 3, sl + 2)) == 4                 # slopes not 4-byte aligned
    assert fwd(_mask(0, 3, 3, o + 64)) == 7                 # slopes inside the output
    assert fwd(_mask(1), Nk=0) == 2
    assert fwd(_mask(1), st=_st(cq, ck, ck, cq[:2] + (8,))) == 7  # o rows overlap
    ws = 0x40000000
    need = lib.fa_bwd_ext_workspace_bytes(B, H, Hkv, Nq, Nk, d, _mask(1, 16, 0))
    assert need >= B * H * Nq * 4
    assert lib.fa_bwd_ext_workspace_bytes(B, H, Hkv, Nq, Nk, d, _mask(0, -5)) == 0
    assert lib.fa_bwd_ext_workspace_bytes(B, H, 3, Nq, Nk, d, None) == 0
    ptrs = [P + i * 0x100000 for i in range(9)]
    st8 = _st(cq, ck, ck, cq, cq, cq, ck, ck)
    args = ptrs + [B, H, Hkv, Nq, Nk, d, st8, _mask(1, 16, 0), 0.125, ws, need, None]
    bad = list(args)
    bad[19] = need - 256                                    # workspace too small
    assert lib.fa_bwd_ext(*bad) == 5
    bad = list(args)
    bad[16] = _mask(1, 16, 0, ptrs[6] + 4)                  # slopes inside dq
    assert lib.fa_bwd_ext(*bad) == 7
    bad = list(args)
    bad[16] = _mask(3)
    assert lib.fa_bwd_ext(*bad) == 9


@pytest.mark.skipif(torch.cuda.is_available(), reason="valid-looking fake pointers must never reach a GPU")
def test_ext_no_device_is_reported_after_validation():
    lib = fa.load_library()
    B, H, Hkv, Nq, Nk, d = 2, 4, 1, 33, 300, 128
    cq, ck = (H * Nq * d, Nq * d, d), (Hkv * Nk * d, Nk * d, d)
    ptrs = [P + i * 0x1000000 for i in range(9)]
    sl = P + 0x20000000
    assert lib.fa_fwd_ext(*ptrs[:5], B, H, Hkv, Nq, Nk, d, _st(cq, ck, ck, cq), _mask(1, 100, 0, sl), 0.1,
                          None) == 6
    assert lib.fa_fwd_ext(*ptrs[:5], B, H, Hkv, Nq, Nk, d, _st(cq, ck, ck, cq), None, 0.1, None) == 6
    st8 = _st(cq, ck, ck, cq, cq, cq, ck, ck)
    need = lib.fa_bwd_ext_workspace_bytes(B, H, Hkv, Nq, Nk, d, None)
    assert lib.fa_bwd_ext(*ptrs, B, H, Hkv, Nq, Nk, d, st8, None, 0.1, 0x40000000, need, None) == 6


def test_bwd_noalloc_rejects_bad_arguments():
    """fa_bwd_noalloc: host validation as fa_bwd (no workspace argument), and
    FA_ERR_SCRATCH, before any HIP call, when D would not fit the static
    scratch (4 bytes per row, FA_BWD_NOALLOC_SCRATCH_BYTES = 8 MiB)."""
    lib = fa.load_library()
    good = [P + i * 0x100000 for i in range(9)]
    args = good + [1, 1, 64, 64, 1, 0.125, None]
    bad = list(args)
    bad[6] = good[0]                    # dq aliases q
    assert lib.fa_bwd_noalloc(*bad) == 7
    bad = list(args)
    bad[5] = None                       # NULL lse
    assert lib.fa_bwd_noalloc(*bad) == 1
    bad = list(args)
    bad[12] = 96                        # head dim
    assert lib.fa_bwd_noalloc(*bad) == 3
    bad = list(args)
    bad[13] = 2                         # causal flag
    assert lib.fa_bwd_noalloc(*bad) == 9
    # 2^21 + 64 rows of D (each tensor 1 GiB + 16 KiB apart): one row block too many
    rows_max = (8 << 20) // 4
    B, H, N, d = 1, 1, rows_max + 64, 64
    span = 2 * N * d
    big = [P + i * (span + 0x100000) for i in range(9)]
    assert lib.fa_bwd_noalloc(*big, B, H, N, d, 0, 0.125, None) == 10
    assert fa.status_string(10).startswith("FA_ERR_SCRATCH")


@pytest.mark.skipif(torch.cuda.is_available(), reason="valid-looking fake pointers must never reach a GPU")
def test_bwd_noalloc_no_device_is_reported_after_validation():
    lib = fa.load_library()
    rows_max = (8 << 20) // 4
    N, d = rows_max, 64               # exactly fills the scratch
    span = 2 * N * d
    ptrs = [P + i * (span + 0x100000) for i in range(9)]
    assert lib.fa_bwd_noalloc(*ptrs, 1, 1, N, d, 1, 0.125, None) == 6
