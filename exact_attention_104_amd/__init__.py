"""Python binding of the gfx950 attention library (``libfa_mi355x.so``).

Argument marshalling only: every step of attention runs in the HIP kernels
behind the C ABI of ``include/fa.h``. PyTorch supplies device memory and the
current stream. There is no fallback: if the library is missing, every call
raises.

    o, lse = fwd(q, k, v, causal=True)                  # bf16 [B, H, N, d] CUDA tensors
    dq, dk, dv = bwd(q, k, v, o, do, lse, causal=True)
    # any [B, H, N, d] views with contiguous d (e.g. [B, N, H, d].transpose(1, 2)),
    # and grouped K/V heads: k, v of shape [B, H_kv, N, d] with H_kv dividing H;
    # k, v may have another length N_k (cross-attention), and
    o, lse = fwd(q, k, v, causal=True, window=(256, 0), alibi_slopes=slopes)  # slopes: fp32 [H]
    q8, qs = quant_fp8(q, signs)                        # signs: int8 [128] or None
    o8, lse8 = fwd_fp8(q8, k8, v8, qs, ks, vs, causal=True)
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA_MI355X_LIB names another build of the same library (e.g. the
# host-sanitized one, for CPU tests of the C ABI).
LIB_PATH = os.environ.get("FA_MI355X_LIB") or os.path.join(_HERE, "libfa_mi355x.so")

FA_STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEADDIM", 4: "FA_ERR_ALIGN",
    5: "FA_ERR_WORKSPACE", 6: "FA_ERR_DEVICE", 7: "FA_ERR_ALIAS", 8: "FA_ERR_LAUNCH", 9: "FA_ERR_ARG",
    10: "FA_ERR_SCRATCH",
}

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float

class Strides(ctypes.Structure):
    """fa_strides: element strides (batch, head, row) of a [B, H, N, d] view."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("row", ctypes.c_int64)]


class Mask(ctypes.Structure):
    """fa_mask: causal flag, sliding window (left, right; -1 unbounded), ALiBi slopes."""
    _fields_ = [("causal", ctypes.c_int), ("window_left", ctypes.c_int), ("window_right", ctypes.c_int),
                ("alibi_slopes", ctypes.c_void_p)]


# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_abi_version": (_I, []),
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "fa_fwd_strided": (_I, [_P] * 5 + [_I, _I, _I, _I, _I, _P, _I, _F, _P]),
    "fa_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "fa_bwd": (_I, [_P] * 9 + [_I, _I, _I, _I, _I, _F, _P, ctypes.c_size_t, _P]),
    "fa_bwd_noalloc": (_I, [_P] * 9 + [_I, _I, _I, _I, _I, _F, _P]),
    "fa_bwd_strided": (_I, [_P] * 9 + [_I, _I, _I, _I, _I, _P, _I, _F, _P, ctypes.c_size_t, _P]),
    "fa_bwd_strided_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I]),
    "fa_fwd_ext": (_I, [_P] * 5 + [_I] * 6 + [_P, _P, _F, _P]),
    "fa_bwd_ext_workspace_bytes": (ctypes.c_size_t, [_I] * 6 + [_P]),
    "fa_bwd_ext": (_I, [_P] * 9 + [_I] * 6 + [_P, _P, _F, _P, ctypes.c_size_t, _P]),
    "fa_quant_fp8": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "fa_fwd_fp8": (_I, [_P] * 8 + [_I, _I, _I, _I, _I, _F, _P]),
    "fa_fwd_fp8_ext": (_I, [_P] * 8 + [_I, _I, _I, _I, _I, _F, _I, _P]),
}


class FAError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__("%s returned %d (%s)" % (call, status, status_string(status)))


def load_library(path: str | None = None):
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError("HIP attention library not built: %s is missing "
                           "(run python -m exact_attention_104_amd.build)" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fa_status_string(status).decode()


def abi_version() -> int:
    return load_library().fa_abi_version()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check_tensor(name, t, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _bhnd(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d], got %s" % (tuple(q.shape),))
    return tuple(int(x) for x in q.shape)


def _check_view(name, t, shape):
    """A bf16 [B, H, N, d] view on the GPU whose last dimension is contiguous."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be torch.bfloat16, got %s" % (name, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.stride(3) != 1:
        raise ValueError("%s must have a contiguous last dimension" % name)


def _strides(*ts):
    arr = (Strides * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = Strides(t.stride(0), t.stride(1), t.stride(2))
    return arr


def _kv_heads(q, k, v):
    B, H, N, d = _bhnd(q)
    Hkv = int(k.shape[1]) if k.dim() == 4 else -1
    if Hkv < 1 or H % Hkv:
        raise ValueError("k, v need H_kv heads with H_kv dividing H = %d, got %s" % (H, tuple(k.shape)))
    return B, H, Hkv, N, d


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _raise(st, call):
    if st != 0:
        raise FAError(st, call)


def _mask(causal, window, alibi_slopes, H, device):
    """fa_mask for the arguments, or None when the plain calls suffice."""
    left, right = (int(window[0]), int(window[1])) if window is not None else (-1, -1)
    if alibi_slopes is not None:
        _check_tensor("alibi_slopes", alibi_slopes, torch.float32, (H,))
        if alibi_slopes.device != device:
            raise ValueError("alibi_slopes must be on the device of q")
    if (left, right) == (-1, -1) and alibi_slopes is None:
        return None
    return Mask(int(bool(causal)), left, right, alibi_slopes.data_ptr() if alibi_slopes is not None else None)


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, window=None,
        alibi_slopes=None):
    """bf16 forward: returns (O bf16 [B,H,N_q,d], LSE fp32 [B,H,N_q]).

    q: [B, H, N_q, d]; k, v: [B, H_kv, N_k, d] (H_kv divides H: grouped / multi-query
    heads; N_k != N_q: cross-attention, the last query aligned with the last key);
    any views with a contiguous last dimension. window = (left, right) keys around
    each query's diagonal key (-1: unbounded); alibi_slopes: fp32 [H] on the GPU.
    O takes q's layout."""
    lib = load_library()
    B, H, Hkv, Nq, d = _kv_heads(q, k, v)
    Nk = int(k.shape[2])
    _check_view("q", q, (B, H, Nq, d))
    _check_view("k", k, (B, Hkv, Nk, d))
    _check_view("v", v, (B, Hkv, Nk, d))
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_view("out", o, (B, H, Nq, d))
    _check_tensor("lse", lse_t, torch.float32, (B, H, Nq))
    sc, c = _scale(scale, d), int(bool(causal))
    m = _mask(causal, window, alibi_slopes, H, q.device)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr())
    if m is not None or Nk != Nq:
        m = m if m is not None else Mask(c, -1, -1, None)
        st = lib.fa_fwd_ext(*ptrs, B, H, Hkv, Nq, Nk, d, _strides(q, k, v, o), ctypes.byref(m), sc, _stream())
        _raise(st, "fa_fwd_ext")
    elif Hkv == H and all(t.is_contiguous() for t in (q, k, v, o)):
        st = lib.fa_fwd(*ptrs, B, H, Nq, d, c, sc, _stream())
        _raise(st, "fa_fwd")
    else:
        st = lib.fa_fwd_strided(*ptrs, B, H, Hkv, Nq, d, _strides(q, k, v, o), c, sc, _stream())
        _raise(st, "fa_fwd_strided")
    return o, lse_t


def bwd_workspace_bytes(B, H, N, d, H_kv=None, causal=False, N_k=None, window=None, alibi=False) -> int:
    """Workspace bytes of bwd: fa_bwd's, or (H_kv, N_k or a window given) fa_bwd_ext's."""
    lib = load_library()
    if H_kv is None and N_k is None and window is None:
        return int(lib.fa_bwd_workspace_bytes(B, H, N, d))
    left, right = window if window is not None else (-1, -1)
    m = Mask(int(bool(causal)), int(left), int(right), None)
    return int(lib.fa_bwd_ext_workspace_bytes(B, H, H if H_kv is None else H_kv, N, N if N_k is None else N_k,
                                              d, ctypes.byref(m)))


def bwd(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None, workspace=None, window=None,
        alibi_slopes=None, out=None):
    """bf16 backward by recomputation: returns (dQ, dK, dV) bf16.

    Shapes, layouts and masks as in fwd; dK, dV have k's and v's shapes (for
    grouped heads, the sums over each group's query heads). out = (dq, dk, dv)
    writes into caller-owned views (any layout with a contiguous last
    dimension); otherwise new tensors take q's, k's and v's layouts."""
    lib = load_library()
    B, H, Hkv, Nq, d = _kv_heads(q, k, v)
    Nk = int(k.shape[2])
    for n, t in (("q", q), ("o", o), ("do", do)):
        _check_view(n, t, (B, H, Nq, d))
    for n, t in (("k", k), ("v", v)):
        _check_view(n, t, (B, Hkv, Nk, d))
    _check_tensor("lse", lse, torch.float32, (B, H, Nq))
    sc, c = _scale(scale, d), int(bool(causal))
    m = _mask(causal, window, alibi_slopes, H, q.device)
    mm = m if m is not None else Mask(c, -1, -1, None)
    need = int(lib.fa_bwd_ext_workspace_bytes(B, H, Hkv, Nq, Nk, d, ctypes.byref(mm)))
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    _check_tensor("workspace", ws, torch.uint8)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _check_view("dq", dq, (B, H, Nq, d))
        _check_view("dk", dk, (B, Hkv, Nk, d))
        _check_view("dv", dv, (B, Hkv, Nk, d))
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    if m is not None or Nk != Nq:
        st = lib.fa_bwd_ext(*ptrs, B, H, Hkv, Nq, Nk, d, _strides(q, k, v, o, do, dq, dk, dv), ctypes.byref(mm),
                            sc, ws.data_ptr(), ws.numel(), _stream())
        _raise(st, "fa_bwd_ext")
    elif Hkv == H and all(t.is_contiguous() for t in (q, k, v, o, do, dq, dk, dv)):
        st = lib.fa_bwd(*ptrs, B, H, Nq, d, c, sc, ws.data_ptr(), ws.numel(), _stream())
        _raise(st, "fa_bwd")
    else:
        st = lib.fa_bwd_strided(*ptrs, B, H, Hkv, Nq, d, _strides(q, k, v, o, do, dq, dk, dv), c, sc,
                                ws.data_ptr(), ws.numel(), _stream())
        _raise(st, "fa_bwd_strided")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None, out=None):
    """fa_bwd_noalloc: the contiguous multi-head backward with no workspace
    argument (the library's static per-GPU scratch holds D). Calls that overlap
    on one GPU race on that scratch. out = (dq, dk, dv) contiguous, else new."""
    lib = load_library()
    B, H, N, d = _bhnd(q)
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_tensor(n, t, torch.bfloat16, (B, H, N, d))
    _check_tensor("lse", lse, torch.float32, (B, H, N))
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            _check_tensor(n, t, torch.bfloat16, (B, H, N, d))
    st = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, int(bool(causal)),
                            _scale(scale, d), _stream())
    _raise(st, "fa_bwd_noalloc")
    return dq, dk, dv


def quant_fp8(x, signs=None):
    """Block quantisation (optional Hadamard rotation): returns (codes uint8, scales fp32)."""
    lib = load_library()
    B, H, N, d = _bhnd(x)
    _check_tensor("x", x, torch.bfloat16, (B, H, N, d))
    if signs is not None:
        _check_tensor("signs", signs, torch.int8, (128,))
    x8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    sc = torch.empty((B, H, (N + 127) // 128), dtype=torch.float32, device=x.device)
    st = lib.fa_quant_fp8(x.data_ptr(), x8.data_ptr(), sc.data_ptr(),
                          None if signs is None else signs.data_ptr(), B, H, N, d, _stream())
    _raise(st, "fa_quant_fp8")
    return x8, sc


def fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False, scale: float | None = None,
            out=None, lse=None, exp_mode: int = 0):
    """fp8 forward on quantised inputs: returns (O bf16, LSE fp32); out / lse
    are optional caller-owned contiguous outputs. exp_mode 1 (2) computes one
    in four (all) of the softmax exponentials with the software 2^x
    (fa_fwd_fp8_ext; d = 128 only); 0 uses the hardware exponential."""
    lib = load_library()
    B, H, N, d = _bhnd(q8)
    nb = (N + 127) // 128
    for n, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _check_tensor(n, t, torch.uint8, (B, H, N, d))
    for n, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check_tensor(n, t, torch.float32, (B, H, nb))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device) if lse is None else lse
    _check_tensor("out", o, torch.bfloat16, (B, H, N, d))
    _check_tensor("lse", lse, torch.float32, (B, H, N))
    ptrs = (q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_scale.data_ptr(),
            k_scale.data_ptr(), v_scale.data_ptr(), o.data_ptr(), lse.data_ptr())
    if exp_mode == 0:
        st = lib.fa_fwd_fp8(*ptrs, B, H, N, d, int(bool(causal)), _scale(scale, d), _stream())
        _raise(st, "fa_fwd_fp8")
    else:
        st = lib.fa_fwd_fp8_ext(*ptrs, B, H, N, d, int(bool(causal)), _scale(scale, d),
                                int(exp_mode), _stream())
        _raise(st, "fa_fwd_fp8_ext")
    return o, lse
