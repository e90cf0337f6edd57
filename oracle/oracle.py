"""Oracle for the fused MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Python (ctypes + numpy) front end of ``moe_oracle.cpp``, a plain double
precision CPU implementation of the layer that shares no code with the HIP
path.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product package never does.

Every function takes and returns host numpy arrays.  bf16 data is carried as
``uint16`` bit patterns and e4m3 data as ``uint8`` codes.  See the C++ file for
the passages of the pages each function follows and for the readings taken
where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
# A build of a modified copy of the source, loaded instead of liboracle.so: the
# mutation test uses it to check that the pins catch planted mistakes.
_LIB_OVERRIDE = os.environ.get("MOE355_ORACLE_LIB")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int


def build() -> str:
    """Compile the oracle with the host C++ compiler (plain -O2, no fast-math)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
                           "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC])
    os.replace(tmp, _LIB)
    return _LIB


class _Layer(ctypes.Structure):
    _fields_ = [("wtype", _I32), ("E", _I32), ("H", _I32), ("I", _I32), ("has_shared", _I32),
                ("w1", _P), ("w3", _P), ("w2", _P), ("s1", _P), ("s3", _P), ("s2", _P),
                ("sw1", _P), ("sw3", _P), ("sw2", _P), ("ss1", _P), ("ss3", _P), ("ss2", _P),
                ("h_scale", _P)]


class _Trace(ctypes.Structure):
    _fields_ = [("h", _P), ("hq", _P), ("hs", _P), ("h_scale", _P)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            L = ctypes.CDLL(_LIB)
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_nearest.restype = ctypes.c_uint16
        L.orc_bf16_nearest.argtypes = [ctypes.c_float]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_code.restype = ctypes.c_uint8
        L.orc_e4m3_code.argtypes = [ctypes.c_float]
        L.orc_e4m3_code_array.argtypes = [_P, _I64, _P]
        L.orc_router_split.argtypes = [_P, _I64, _P, _P]
        L.orc_router_logits.argtypes = [_P, _P, _I64, _I32, _I32, _P, _I32]
        L.orc_route.argtypes = [_P, _P, _P, _I64, _I32, _I32, _P, _P]
        L.orc_align.argtypes = [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P]
        L.orc_quant_rows_fp8.argtypes = [_P, _I64, _I32, _P, _P]
        L.orc_mx_exponent.restype = ctypes.c_int
        L.orc_mx_exponent.argtypes = [ctypes.c_float]
        L.orc_quant_rows_mx.argtypes = [_P, _I64, _I32, _P, _P, _I32]
        L.orc_quant_rows_mx_f32.argtypes = [_P, _I64, _I32, _P, _P]
        L.orc_quant_blocks_fp8.argtypes = [_P, _I64, _I32, _I32, _P, _P, _I32]
        L.orc_quant_tensor_fp8.argtypes = [_P, _I32, _I64, _I64, _P, _P, _I32]
        L.orc_expert_bf16.argtypes = [_P, _P, _P, _P, _I32, _I32, _P, _P]
        L.orc_expert_fp8.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _P]
        L.orc_layer_rows.argtypes = [ctypes.POINTER(_Layer), _P, _P, _P, _P, _I32, _P, _I64, _P, _I32]
        L.orc_layer_rows_trace.argtypes = [ctypes.POINTER(_Layer), _P, _P, _P, _P, _I32, _P, _I64, _P, _I32,
                                           ctypes.POINTER(_Trace)]
        L.orc_pt_h.argtypes = [_P, _P, _I64, ctypes.c_double, ctypes.c_double, ctypes.c_double, _P]
        L.orc_combine.argtypes = [_P, _P, _P, _I64, _I32, _I32, _I32, _P]
        L.orc_add_rmsnorm.argtypes = [_P, _P, _P, ctypes.c_double, _I64, _I32, _P, _P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_P)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ------------------------------------------------------------------ codecs
def bf16_value(bits):
    bits = _c(bits, np.uint16)
    return np.array([lib().orc_bf16_value(int(b)) for b in bits.ravel()]).reshape(bits.shape)


def e4m3_value(codes):
    codes = _c(codes, np.uint8)
    return np.array([lib().orc_e4m3_value(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e4m3_code(values):
    v = _c(values, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_code_array(_ptr(v), v.size, _ptr(out))
    return out


# ------------------------------------------------------------------ router
def router_split(w):
    w = _c(w, np.float32)
    hi = np.empty(w.shape, np.uint16)
    lo = np.empty(w.shape, np.uint16)
    lib().orc_router_split(_ptr(w), w.size, _ptr(hi), _ptr(lo))
    return hi, lo


def router_logits(x_bits, w, nthreads=None):
    x_bits = _c(x_bits, np.uint16)
    w = _c(w, np.float32)
    T, H = x_bits.shape
    E = w.shape[0]
    out = np.empty((T, E), np.float64)
    lib().orc_router_logits(_ptr(x_bits), _ptr(w), T, H, E, _ptr(out), nthreads or default_threads())
    return out


# ------------------------------------------------------------------ route / align
def route(logits, k, bias=None, bias_rows=None):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    b = None if bias is None else _c(bias, np.float32)
    br = None if bias_rows is None else _c(bias_rows, np.uint8)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().orc_route(_ptr(logits), _ptr(b), _ptr(br), T, E, k, _ptr(ids), _ptr(w))
    return ids, w


def align(ids, E, shared):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 2, np.int32)
    slot_pair = np.empty(T * k, np.int32)
    pair_slot = np.empty(T * k, np.int32)
    lib().orc_align(_ptr(ids), T, E, k, int(shared), _ptr(counts), _ptr(offsets),
                    _ptr(slot_pair), _ptr(pair_slot))
    return counts, offsets, slot_pair, pair_slot


# ------------------------------------------------------------------ fp8
def quant_rows_fp8(x_bits):
    x_bits = _c(x_bits, np.uint16)
    rows, cols = x_bits.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    lib().orc_quant_rows_fp8(_ptr(x_bits), rows, cols, _ptr(q), _ptr(s))
    return q, s


def mx_exponent(amax: float) -> int:
    """Shared exponent X of an MXFP8 block whose largest magnitude is amax."""
    return lib().orc_mx_exponent(float(amax))


def quant_rows_mx(x_bits, nthreads=None):
    """MXFP8 of bf16 rows [..., cols]: codes (same shape) and E8M0 bytes [..., cols/32]."""
    x_bits = _c(x_bits, np.uint16)
    cols = x_bits.shape[-1]
    rows = x_bits.size // cols
    q = np.empty(x_bits.shape, np.uint8)
    s = np.empty(x_bits.shape[:-1] + (cols // 32,), np.uint8)
    lib().orc_quant_rows_mx(_ptr(x_bits), rows, cols, _ptr(q), _ptr(s), nthreads or default_threads())
    return q, s


def quant_rows_mx_f32(x):
    """The same MXFP8 rule on fp32 rows."""
    x = _c(x, np.float32)
    cols = x.shape[-1]
    q = np.empty(x.shape, np.uint8)
    s = np.empty(x.shape[:-1] + (cols // 32,), np.uint8)
    lib().orc_quant_rows_mx_f32(_ptr(x), x.size // cols, cols, _ptr(q), _ptr(s))
    return q, s


def quant_blocks_fp8(w_bits, nthreads=None):
    """w_bits: [mats, rows, cols] (or [rows, cols]) bf16 bit patterns."""
    w_bits = _c(w_bits, np.uint16)
    squeeze = w_bits.ndim == 2
    if squeeze:
        w_bits = w_bits[None]
    mats, rows, cols = w_bits.shape
    q = np.empty(w_bits.shape, np.uint8)
    s = np.empty((mats, rows // 128, cols // 128), np.float32)
    lib().orc_quant_blocks_fp8(_ptr(w_bits), mats, rows, cols, _ptr(q), _ptr(s), nthreads or default_threads())
    return (q[0], s[0]) if squeeze else (q, s)


def quant_tensor_fp8(x, mats=1, nthreads=None):
    """Per-tensor FP8 of ``mats`` equal parts of x (bf16 bit patterns as uint16,
    or fp32 values): codes shaped like x and one fp32 scale per part [mats]."""
    f32 = x.dtype == np.float32
    x = _c(x, np.float32 if f32 else np.uint16)
    n = x.size // mats
    q = np.empty(x.shape, np.uint8)
    s = np.empty(mats, np.float32)
    lib().orc_quant_tensor_fp8(_ptr(x), int(f32), mats, n, _ptr(q), _ptr(s), nthreads or default_threads())
    return q, s


_E4M3 = None


def e4m3_values():
    """Value of every E4M3 code (float64 [256], NaN for the two NaN codes), from the oracle's codec."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = e4m3_value(np.arange(256, dtype=np.uint8))
    return _E4M3


def pt_h_rows(xq, xsc, w1q, s1, w3q, s3):
    """Per-tensor FP8 h of one expert on the code rows xq [n, H]: fp32 [n, I].

    The code dot products are exact in double in any order of the additions
    (see ``tensor_dot`` in the C++ file), so they are taken as one float64
    matrix product of the decoded codes (a library matmul); the scaling, SiLU
    and the fp32 rounding are the layer's own (``orc_pt_h``)."""
    dec = e4m3_values()
    X = dec[_c(xq, np.uint8)]
    gdot = np.ascontiguousarray(X @ dec[_c(w1q, np.uint8)].T)
    udot = np.ascontiguousarray(X @ dec[_c(w3q, np.uint8)].T)
    h = np.empty(gdot.shape, np.float32)
    lib().orc_pt_h(_ptr(gdot), _ptr(udot), gdot.size, float(xsc), float(s1), float(s3), _ptr(h))
    return h


def pt_h_amax(xq, xsc, ids, E, has_shared, expert):
    """Per-tensor FP8: the largest |h| over the whole h tensor, i.e. over every
    (token, expert) pair of every token plus the shared expert's row of every
    token -- what the h scale amax/448 is taken from.

    xq [T, H] x codes, xsc the x scale, ids [T, k] the routing; expert(g)
    returns (w1q, s1, w3q, s3) of group g (g == E: the shared expert), so the
    weights can be streamed one expert at a time."""
    ids = _c(ids, np.int32)
    T = ids.shape[0]
    amax = np.float32(0.0)
    groups = [(g, np.nonzero((ids == g).any(axis=1))[0]) for g in range(E)]
    if has_shared:
        groups.append((E, np.arange(T)))
    for g, toks in groups:
        if toks.size == 0:
            continue
        w1q, s1, w3q, s3 = expert(g)
        h = pt_h_rows(xq[toks], xsc, w1q, s1, w3q, s3)
        amax = max(amax, np.float32(np.abs(h).max()))
    return float(amax)


# ------------------------------------------------------------------ experts / layer
def expert_bf16(x_bits, w1, w3, w2):
    x_bits, w1, w3, w2 = (_c(a, np.uint16) for a in (x_bits, w1, w3, w2))
    I, H = w1.shape
    h = np.empty(I, np.float64)
    y = np.empty(H, np.float64)
    lib().orc_expert_bf16(_ptr(x_bits), _ptr(w1), _ptr(w3), _ptr(w2), H, I, _ptr(h), _ptr(y))
    return h, y


def expert_fp8(xq, xs, w1q, s1, w3q, s3, w2q, s2):
    xq, w1q, w3q, w2q = (_c(a, np.uint8) for a in (xq, w1q, w3q, w2q))
    xs, s1, s3, s2 = (_c(a, np.float32) for a in (xs, s1, s3, s2))
    I, H = w1q.shape
    h = np.empty(I, np.float64)
    y = np.empty(H, np.float64)
    lib().orc_expert_fp8(_ptr(xq), _ptr(xs), _ptr(w1q), _ptr(s1), _ptr(w3q), _ptr(s3),
                         _ptr(w2q), _ptr(s2), H, I, _ptr(h), _ptr(y))
    return h, y


class Layer:
    """Host copies of the expert weights.

    bf16: ``Layer(w1, w3, w2, sw1=None, sw3=None, sw2=None)`` with uint16 arrays
    w1, w3 [E, I, H], w2 [E, H, I] and the shared expert [I, H] / [H, I].
    fp8: pass ``wtype=1`` plus uint8 codes and the fp32 block scales
    s1, s3 [E, I/128, H/128], s2 [E, H/128, I/128] (and ss1/ss3/ss2).
    MXFP8: ``wtype=2``, uint8 codes and uint8 E8M0 scales per weight row per
    32 K: s1, s3 [E, I, H/32], s2 [E, H, I/32] (and the shared ones).
    Per-tensor FP8: ``wtype=3``, uint8 codes and one fp32 scale per matrix,
    s1, s3, s2 [E] and ss1, ss3, ss2 [1]; ``h_scale`` fixes the scale of the
    whole h (None: computed from the h of the rows evaluated).
    """

    def __init__(self, w1, w3, w2, sw1=None, sw3=None, sw2=None, wtype=0,
                 s1=None, s3=None, s2=None, ss1=None, ss3=None, ss2=None, h_scale=None):
        dt = np.uint16 if wtype == 0 else np.uint8
        self.arrays = {}
        for name, a in (("w1", w1), ("w3", w3), ("w2", w2), ("sw1", sw1), ("sw3", sw3), ("sw2", sw2)):
            self.arrays[name] = None if a is None else _c(a, dt)
        sdt = np.uint8 if wtype == 2 else np.float32
        for name, a in (("s1", s1), ("s3", s3), ("s2", s2), ("ss1", ss1), ("ss3", ss3), ("ss2", ss2)):
            self.arrays[name] = None if a is None else _c(a, sdt)
        E, I, H = self.arrays["w1"].shape
        self.E, self.I, self.H, self.wtype = E, I, H, wtype
        self.has_shared = sw1 is not None
        a = self.arrays
        self.arrays["h_scale"] = None if h_scale is None else np.array([h_scale], np.float32)
        self.c = _Layer(wtype, E, H, I, int(self.has_shared),
                        *(_ptr(a[n]) for n in ("w1", "w3", "w2", "s1", "s3", "s2",
                                               "sw1", "sw3", "sw2", "ss1", "ss3", "ss2", "h_scale")))


def layer_rows(layer: Layer, x, ids, weights, rows, xs=None, nthreads=None, trace=False):
    """out[r] = sum_j w[t,j] FFN_{ids[t,j]}(x_t) + FFN_shared(x_t) for t = rows[r] (double).

    With trace=True returns (out, tr): tr["h"] [nrows, k+S, I] fp32 h of every
    pair (rank j < k, then the shared expert), and for the FP8 paths
    tr["hq"] (codes, same shape), tr["hs"] (block FP8: fp32 [nrows, k+S, I/128];
    MXFP8: E8M0 bytes [nrows, k+S, I/32]) and tr["h_scale"] (per-tensor FP8)."""
    dt = np.uint16 if layer.wtype == 0 else np.uint8
    x = _c(x, dt)
    xs = None if xs is None else _c(xs, np.uint8 if layer.wtype == 2 else np.float32)
    ids = _c(ids, np.int32)
    weights = _c(weights, np.float64)
    rows = _c(rows, np.int64)
    k = ids.shape[1]
    out = np.empty((rows.size, layer.H), np.float64)
    if not trace:
        lib().orc_layer_rows(ctypes.byref(layer.c), _ptr(x), _ptr(xs), _ptr(ids), _ptr(weights), k,
                             _ptr(rows), rows.size, _ptr(out), nthreads or default_threads())
        return out
    per = k + int(layer.has_shared)
    I = layer.I
    tr = {"h": np.empty((rows.size, per, I), np.float32)}
    hq = hs = hsc = None
    if layer.wtype != 0:
        tr["hq"] = hq = np.empty((rows.size, per, I), np.uint8)
    if layer.wtype == 1:
        tr["hs"] = hs = np.empty((rows.size, per, I // 128), np.float32)
    elif layer.wtype == 2:
        tr["hs"] = hs = np.empty((rows.size, per, I // 32), np.uint8)
    elif layer.wtype == 3:
        hsc = np.empty(1, np.float32)
    c = _Trace(_ptr(tr["h"]), _ptr(hq), _ptr(hs), _ptr(hsc))
    lib().orc_layer_rows_trace(ctypes.byref(layer.c), _ptr(x), _ptr(xs), _ptr(ids), _ptr(weights), k,
                               _ptr(rows), rows.size, _ptr(out), nthreads or default_threads(), ctypes.byref(c))
    if hsc is not None:
        tr["h_scale"] = float(hsc[0])
    return out, tr


# ------------------------------------------------------------------ combine / norm
def combine(y, pair_slot, w, T, k, has_shared):
    """Stage 5 on given expert outputs y [R,H] (fp32 values): double [T,H]."""
    y = _c(y, np.float32)
    pair_slot = _c(pair_slot, np.int32)
    w = _c(w, np.float32)
    H = y.shape[1]
    out = np.empty((T, H), np.float64)
    lib().orc_combine(_ptr(y), _ptr(pair_slot), _ptr(w), T, k, H, int(has_shared), _ptr(out))
    return out


def add_rmsnorm(x, residual_bits, weight_bits, eps):
    """s = x + residual, out = s / sqrt(mean(s^2) + eps) * weight, per row (double)."""
    x = _c(x, np.float64)
    residual_bits = _c(residual_bits, np.uint16)
    weight_bits = _c(weight_bits, np.uint16)
    rows, H = x.shape
    s = np.empty((rows, H), np.float64)
    out = np.empty((rows, H), np.float64)
    lib().orc_add_rmsnorm(_ptr(x), _ptr(residual_bits), _ptr(weight_bits), float(eps), rows, H, _ptr(s), _ptr(out))
    return s, out
