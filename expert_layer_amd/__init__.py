"""Python binding of libmoe355, the MI355X fused MoE layer forward.

Thin ctypes marshalling over the C ABI declared in ``include/moe355.h``: every
function here has the C entry point's name, takes caller-allocated torch
tensors (device memory), passes their pointers and torch's current stream, and
raises ``MoeError`` on a non-zero status.  All computation runs in the HIP
kernels of ``libmoe355.so``; if the library is not built, importing a function
raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE355_LIB may point at another build of the same library (e.g. a tuned variant)
LIB_PATH = os.environ.get("MOE355_LIB") or os.path.join(_PKG, "libmoe355.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EDEVICE = range(5)
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_W_BF16, MOE_W_FP8, MOE_W_MXFP8, MOE_W_FP8_TENSOR = 0, 1, 2, 3

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int
_SZ = ctypes.c_size_t


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({moe_status_string(status)})")


class moe_experts_t(ctypes.Structure):
    _fields_ = [("wtype", _I32), ("E", _I32), ("H", _I32), ("I", _I32), ("has_shared", _I32),
                ("w1", _P), ("w3", _P), ("w2", _P), ("s1", _P), ("s3", _P), ("s2", _P),
                ("sw1", _P), ("sw3", _P), ("sw2", _P), ("ss1", _P), ("ss3", _P), ("ss2", _P)]


class moe_forward_args_t(ctypes.Structure):
    _fields_ = [("T", _I64), ("k", _I32), ("y_dtype", _I32), ("x", _P), ("logits", _P),
                ("router_hi", _P), ("router_lo", _P), ("bias", _P), ("bias_rows", _P),
                ("out", _P), ("topk_ids", _P), ("topk_w", _P)]


_SIGS = {
    "moe_abi_version": (_I32, []),
    "moe_status_string": (ctypes.c_char_p, [_I32]),
    "moe_router_split": (_I32, [_P, _P, _P, _I32, _I32, _P]),
    "moe_router_gemm": (_I32, [_P, _P, _P, _P, _I64, _I32, _I32, _P]),
    "moe_route": (_I32, [_P, _P, _P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_align_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "moe_align": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_quant_rows_fp8": (_I32, [_P, _I64, _I32, _P, _P, _P]),
    "moe_quant_blocks_fp8": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_quant_rows_mxfp8": (_I32, [_P, _I64, _I32, _P, _P, _P]),
    "moe_tensor_amax": (_I32, [_P, _I32, _I64, _I64, _P, _P]),
    "moe_quant_tensor_fp8": (_I32, [_P, _I32, _I64, _I64, _P, _P, _P, _P]),
    "moe_gemm_workspace_bytes": (_SZ, [ctypes.POINTER(moe_experts_t), _I64, _I32]),
    "moe_gemm13": (_I32, [ctypes.POINTER(moe_experts_t), _P, _P, _P, _P, _I64, _I32, _P, _P, _P, _SZ, _P]),
    "moe_gemm2": (_I32, [ctypes.POINTER(moe_experts_t), _P, _P, _P, _I64, _I32, _P, _I32, _P, _SZ, _P]),
    "moe_combine": (_I32, [_P, _I32, _P, _P, _I64, _I32, _I32, _I32, _P, _P]),
    "moe_combine_rmsnorm": (_I32, [_P, _I32, _P, _P, _I64, _I32, _I32, _I32, _P, _P, ctypes.c_float, _P, _P, _P]),
    "moe_forward_workspace_bytes": (_SZ, [ctypes.POINTER(moe_experts_t), _I64, _I32, _I32]),
    "moe_forward": (_I32, [ctypes.POINTER(moe_experts_t), ctypes.POINTER(moe_forward_args_t), _P, _SZ, _P]),
    "moe_forward_persistent": (_I32, [ctypes.POINTER(moe_experts_t), ctypes.POINTER(moe_forward_args_t), _P, _SZ,
                                      _P]),
    "moe_forward_noalloc": (_I32, [ctypes.POINTER(moe_experts_t), ctypes.POINTER(moe_forward_args_t), _P]),
    "moe_forward_persistent_status": (_I32, [_P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe355.so (built in-tree by ``python -m expert_layer_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m expert_layer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


# ------------------------------------------------------------------ marshalling helpers
def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(*ts):
    for t in ts:
        if t is not None and t.is_cuda:
            return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return None


def _expect(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


def _check(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


# ------------------------------------------------------------------ router
def moe_router_split(w, w_hi, w_lo):
    _expect(w, torch.float32, "w")
    _expect(w_hi, torch.bfloat16, "w_hi")
    _expect(w_lo, torch.bfloat16, "w_lo")
    E, H = w.shape
    _check(lib().moe_router_split(_ptr(w), _ptr(w_hi), _ptr(w_lo), E, H, _stream(w)), "moe_router_split")


def moe_router_gemm(x, w_hi, w_lo, logits):
    _expect(x, torch.bfloat16, "x")
    _expect(logits, torch.float32, "logits")
    T, H = x.shape
    E = w_hi.shape[0]
    _check(lib().moe_router_gemm(_ptr(x), _ptr(w_hi), _ptr(w_lo), _ptr(logits), T, H, E, _stream(x)),
           "moe_router_gemm")


# ------------------------------------------------------------------ route / align
def moe_route(logits, k, topk_ids, topk_w, bias=None, bias_rows=None):
    _expect(logits, torch.float32, "logits")
    _expect(topk_ids, torch.int32, "topk_ids")
    _expect(topk_w, torch.float32, "topk_w")
    _expect(bias, torch.float32, "bias")
    _expect(bias_rows, torch.uint8, "bias_rows")
    T, E = logits.shape
    _check(lib().moe_route(_ptr(logits), _ptr(bias), _ptr(bias_rows), T, E, k, _ptr(topk_ids), _ptr(topk_w),
                           _stream(logits)), "moe_route")


def moe_align_workspace_bytes(T, E, k) -> int:
    return lib().moe_align_workspace_bytes(T, E, k)


def moe_align(topk_ids, E, shared, counts, offsets, slot_pair, pair_slot, ws=None):
    for t, n in ((topk_ids, "topk_ids"), (counts, "counts"), (offsets, "offsets"),
                 (slot_pair, "slot_pair"), (pair_slot, "pair_slot")):
        _expect(t, torch.int32, n)
    T, k = topk_ids.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_align(_ptr(topk_ids), T, E, k, int(shared), _ptr(counts), _ptr(offsets), _ptr(slot_pair),
                           _ptr(pair_slot), _ptr(ws), nbytes, _stream(topk_ids)), "moe_align")


# ------------------------------------------------------------------ fp8 helpers
def moe_quant_rows_fp8(x, q, s):
    _expect(x, torch.bfloat16, "x")
    _expect(s, torch.float32, "s")
    rows, cols = x.shape
    _check(lib().moe_quant_rows_fp8(_ptr(x), rows, cols, _ptr(q), _ptr(s), _stream(x)), "moe_quant_rows_fp8")


def moe_quant_blocks_fp8(w, q, s):
    _expect(w, torch.bfloat16, "w")
    _expect(s, torch.float32, "s")
    if w.dim() == 2:
        mats, (rows, cols) = 1, w.shape
    else:
        mats, rows, cols = w.shape
    _check(lib().moe_quant_blocks_fp8(_ptr(w), mats, rows, cols, _ptr(q), _ptr(s), _stream(w)),
           "moe_quant_blocks_fp8")


def moe_quant_rows_mxfp8(x, q, s):
    """MXFP8 of bf16 rows: x [..., cols] -> codes q (same shape, uint8), E8M0 bytes s [..., cols/32]."""
    _expect(x, torch.bfloat16, "x")
    _expect(s, torch.uint8, "s")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    _check(lib().moe_quant_rows_mxfp8(_ptr(x), rows, cols, _ptr(q), _ptr(s), _stream(x)), "moe_quant_rows_mxfp8")


def moe_tensor_amax(x, amax, mats=1):
    """amax[m] = max |x| over each of ``mats`` equal parts of x (bf16 or fp32)."""
    _expect(amax, torch.float32, "amax")
    dt = MOE_DTYPE_F32 if x.dtype == torch.float32 else MOE_DTYPE_BF16
    _check(lib().moe_tensor_amax(_ptr(x), dt, mats, x.numel() // mats, _ptr(amax), _stream(x)), "moe_tensor_amax")


def moe_quant_tensor_fp8(x, amax, q, s, mats=1):
    """Per-tensor FP8 of ``mats`` equal parts of x: s[m] = amax[m]/448, q = e4m3(x / s[m])."""
    _expect(amax, torch.float32, "amax")
    _expect(s, torch.float32, "s")
    dt = MOE_DTYPE_F32 if x.dtype == torch.float32 else MOE_DTYPE_BF16
    _check(lib().moe_quant_tensor_fp8(_ptr(x), dt, mats, x.numel() // mats, _ptr(amax), _ptr(q), _ptr(s),
                                      _stream(x)), "moe_quant_tensor_fp8")


# ------------------------------------------------------------------ experts
class Experts:
    """Holds the tensors of a layer's experts and the matching moe_experts_t.

    bf16: w1, w3 [E,I,H], w2 [E,H,I] (torch.bfloat16), shared sw1, sw3 [I,H], sw2 [H,I] or None.
    fp8:  the same shapes as uint8 / float8_e4m3fn codes plus fp32 block scales
          s1, s3 [E,I/128,H/128], s2 [E,H/128,I/128] (ss1, ss3, ss2 for the shared expert).
    mxfp8: codes plus uint8 E8M0 scales per weight row per 32 K: s1, s3 [E,I,H/32],
          s2 [E,H,I/32] (the scale dtype selects the format).
    per-tensor fp8: codes plus one fp32 scale per matrix, s1, s3, s2 [E] and ss1, ss3, ss2 [1]
          (one-dimensional scales select the format).
    """

    def __init__(self, w1, w3, w2, sw1=None, sw3=None, sw2=None, s1=None, s3=None, s2=None,
                 ss1=None, ss3=None, ss2=None):
        fp8 = w1.dtype in (torch.uint8, torch.float8_e4m3fn)
        self.tensors = dict(w1=w1, w3=w3, w2=w2, sw1=sw1, sw3=sw3, sw2=sw2, s1=s1, s3=s3, s2=s2,
                            ss1=ss1, ss3=ss3, ss2=ss2)
        E, I, H = w1.shape
        self.E, self.I, self.H = E, I, H
        self.has_shared = int(sw1 is not None)
        mx = fp8 and s1 is not None and s1.dtype == torch.uint8
        pt = fp8 and s1 is not None and s1.dim() == 1
        self.wtype = MOE_W_MXFP8 if mx else MOE_W_FP8_TENSOR if pt else MOE_W_FP8 if fp8 else MOE_W_BF16
        p = {n: _ptr(t) for n, t in self.tensors.items()}
        self.c = moe_experts_t(self.wtype, E, H, I, self.has_shared,
                               p["w1"], p["w3"], p["w2"], p["s1"], p["s3"], p["s2"],
                               p["sw1"], p["sw3"], p["sw2"], p["ss1"], p["ss3"], p["ss2"])

    @property
    def ref(self):
        return ctypes.byref(self.c)


def moe_gemm_workspace_bytes(ex: Experts, T, k) -> int:
    return lib().moe_gemm_workspace_bytes(ex.ref, T, k)


def moe_gemm13(ex: Experts, x, xs, offsets, slot_pair, T, k, h, hs=None, ws=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_gemm13(ex.ref, _ptr(x), _ptr(xs), _ptr(offsets), _ptr(slot_pair), T, k, _ptr(h), _ptr(hs),
                            _ptr(ws), nbytes, _stream(x)), "moe_gemm13")


def moe_gemm2(ex: Experts, h, hs, offsets, T, k, y, ws=None):
    y_dtype = MOE_DTYPE_F32 if y.dtype == torch.float32 else MOE_DTYPE_BF16
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_gemm2(ex.ref, _ptr(h), _ptr(hs), _ptr(offsets), T, k, _ptr(y), y_dtype, _ptr(ws), nbytes,
                           _stream(h)), "moe_gemm2")


def moe_combine(y, pair_slot, topk_w, T, k, has_shared, out):
    y_dtype = MOE_DTYPE_F32 if y.dtype == torch.float32 else MOE_DTYPE_BF16
    H = out.shape[1]
    _check(lib().moe_combine(_ptr(y), y_dtype, _ptr(pair_slot), _ptr(topk_w), T, k, H, int(has_shared), _ptr(out),
                             _stream(y)), "moe_combine")


def moe_combine_rmsnorm(y, pair_slot, topk_w, T, k, has_shared, residual, weight, eps, out, res_out=None):
    """Combine + residual add + RMSNorm: out = RMSNorm(combine + residual, weight); res_out = the sum."""
    _expect(residual, torch.bfloat16, "residual")
    _expect(weight, torch.bfloat16, "weight")
    _expect(out, torch.bfloat16, "out")
    _expect(res_out, torch.bfloat16, "res_out")
    y_dtype = MOE_DTYPE_F32 if y.dtype == torch.float32 else MOE_DTYPE_BF16
    H = out.shape[1]
    _check(lib().moe_combine_rmsnorm(_ptr(y), y_dtype, _ptr(pair_slot), _ptr(topk_w), T, k, H, int(has_shared),
                                     _ptr(residual), _ptr(weight), float(eps), _ptr(out), _ptr(res_out), _stream(y)),
           "moe_combine_rmsnorm")


# ------------------------------------------------------------------ whole chain
def moe_forward_workspace_bytes(ex: Experts, T, k, y_dtype=MOE_DTYPE_F32) -> int:
    return lib().moe_forward_workspace_bytes(ex.ref, T, k, y_dtype)


def moe_forward(ex: Experts, x, k, out, ws, logits=None, router_hi=None, router_lo=None, bias=None,
                bias_rows=None, y_dtype=MOE_DTYPE_F32, topk_ids=None, topk_w=None):
    T = x.shape[0]
    args = moe_forward_args_t(T, k, y_dtype, _ptr(x), _ptr(logits), _ptr(router_hi), _ptr(router_lo), _ptr(bias),
                              _ptr(bias_rows), _ptr(out), _ptr(topk_ids), _ptr(topk_w))
    nbytes = ws.numel() * ws.element_size()
    _check(lib().moe_forward(ex.ref, ctypes.byref(args), _ptr(ws), nbytes, _stream(x)), "moe_forward")


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(ex: Experts, x, k, out, logits=None, router_hi=None, router_lo=None, bias=None,
                        bias_rows=None, y_dtype=MOE_DTYPE_F32, topk_ids=None, topk_w=None):
    """moe_forward with its intermediates in the library's fixed device scratch (no workspace)."""
    T = x.shape[0]
    args = moe_forward_args_t(T, k, y_dtype, _ptr(x), _ptr(logits), _ptr(router_hi), _ptr(router_lo), _ptr(bias),
                              _ptr(bias_rows), _ptr(out), _ptr(topk_ids), _ptr(topk_w))
    _check(lib().moe_forward_noalloc(ex.ref, ctypes.byref(args), _stream(x)), "moe_forward_noalloc")


def moe_forward_persistent(ex: Experts, x, k, out, ws, logits=None, router_hi=None, router_lo=None, bias=None,
                           bias_rows=None, y_dtype=MOE_DTYPE_F32, topk_ids=None, topk_w=None):
    """moe_forward as one persistent kernel with device-side ready flags."""
    T = x.shape[0]
    args = moe_forward_args_t(T, k, y_dtype, _ptr(x), _ptr(logits), _ptr(router_hi), _ptr(router_lo), _ptr(bias),
                              _ptr(bias_rows), _ptr(out), _ptr(topk_ids), _ptr(topk_w))
    nbytes = ws.numel() * ws.element_size()
    _check(lib().moe_forward_persistent(ex.ref, ctypes.byref(args), _ptr(ws), nbytes, _stream(x)),
           "moe_forward_persistent")


def moe_forward_persistent_status(ws):
    """Waits for the stream; raises if the last persistent call on ws timed out on the device."""
    _check(lib().moe_forward_persistent_status(_ptr(ws), _stream(ws)), "moe_forward_persistent_status")
