"""Host-side plumbing for one MoE layer call: device buffers plus the stage
calls in chain order.  Allocation uses torch; every computation is a call into
libmoe355.

    layer = Layer.from_weights(w1, w3, w2, sw1, sw3, sw2, fp8=False)
    bufs = Buffers(layer, T, k, y_dtype=torch.float32)
    run_chain(layer, bufs, x, k, logits=logits)          # or router_hi/lo=...
    bufs.out                                             # [T, H] bf16
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (Experts, moe_align, moe_align_workspace_bytes, moe_combine, moe_combine_rmsnorm, moe_gemm2,
               moe_gemm13,
               moe_gemm_workspace_bytes,
               moe_quant_blocks_fp8, moe_quant_rows_fp8, moe_quant_rows_mxfp8, moe_quant_tensor_fp8, moe_route,
               moe_router_gemm, moe_router_split, moe_tensor_amax)


@dataclass
class Layer:
    experts: Experts
    fp8: bool          # e4m3 codes (128x128 fp32 scales, or MXFP8 when mx)
    E: int
    H: int
    I: int
    shared: int
    mx: bool = False   # MXFP8: E8M0 scales per 32 K
    pt: bool = False   # per-tensor FP8: one fp32 scale per matrix

    @staticmethod
    def from_weights(w1, w3, w2, sw1=None, sw3=None, sw2=None, fp8=False, mx=False, pt=False):
        """bf16 weights as given; fp8 quantises them once with 128x128 block
        scales, mx once with MXFP8 (per weight row per 32 K), pt once with one
        scale per matrix."""
        E, I, H = w1.shape
        if pt:
            q = {}
            for name, w in (("w1", w1), ("w3", w3), ("w2", w2), ("sw1", sw1), ("sw3", sw3), ("sw2", sw2)):
                if w is None:
                    q[name] = (None, None)
                    continue
                mats = E if w.dim() == 3 else 1
                w = w.contiguous()
                amax = torch.empty(mats, dtype=torch.float32, device=w.device)
                qt = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
                st = torch.empty(mats, dtype=torch.float32, device=w.device)
                moe_tensor_amax(w, amax, mats=mats)
                moe_quant_tensor_fp8(w, amax, qt, st, mats=mats)
                q[name] = (qt, st)
            ex = Experts(*(q[n][0] for n in ("w1", "w3", "w2", "sw1", "sw3", "sw2")),
                         *(q[n][1] for n in ("w1", "w3", "w2", "sw1", "sw3", "sw2")))
            return Layer(ex, True, E, H, I, int(sw1 is not None), pt=True)
        if mx:
            q = {}
            for name, w in (("w1", w1), ("w3", w3), ("w2", w2), ("sw1", sw1), ("sw3", sw3), ("sw2", sw2)):
                if w is None:
                    q[name] = (None, None)
                    continue
                cols = w.shape[-1]
                qt = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
                st = torch.empty(w.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=w.device)
                moe_quant_rows_mxfp8(w.contiguous(), qt, st)
                q[name] = (qt, st)
            ex = Experts(*(q[n][0] for n in ("w1", "w3", "w2", "sw1", "sw3", "sw2")),
                         *(q[n][1] for n in ("w1", "w3", "w2", "sw1", "sw3", "sw2")))
            return Layer(ex, True, E, H, I, int(sw1 is not None), mx=True)
        if not fp8:
            ex = Experts(w1, w3, w2, sw1, sw3, sw2)
            return Layer(ex, False, E, H, I, int(sw1 is not None))
        q = {}
        for name, w in (("w1", w1), ("w3", w3), ("w2", w2), ("sw1", sw1), ("sw3", sw3), ("sw2", sw2)):
            if w is None:
                q[name] = None
                continue
            rows, cols = w.shape[-2:]
            qt = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
            st = torch.empty(w.shape[:-2] + (rows // 128, cols // 128), dtype=torch.float32, device=w.device)
            moe_quant_blocks_fp8(w.contiguous(), qt, st)
            q[name] = (qt, st)
        sc = lambda n: None if q[n] is None else q[n][1]   # noqa: E731
        co = lambda n: None if q[n] is None else q[n][0]   # noqa: E731
        ex = Experts(co("w1"), co("w3"), co("w2"), co("sw1"), co("sw3"), co("sw2"),
                     sc("w1"), sc("w3"), sc("w2"), sc("sw1"), sc("sw3"), sc("sw2"))
        return Layer(ex, True, E, H, I, int(sw1 is not None))


class Buffers:
    """Every intermediate of one layer call for T tokens, on the weights' device."""

    def __init__(self, layer: Layer, T: int, k: int, y_dtype=torch.float32, device=None, router=False):
        dev = device or layer.experts.tensors["w1"].device
        E, H, I = layer.E, layer.H, layer.I
        P = T * k
        R = P + layer.shared * T
        i32 = dict(dtype=torch.int32, device=dev)
        self.T, self.k, self.R = T, k, R
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev) if router else None
        self.ids = torch.empty((T, k), **i32)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 2, **i32)
        self.slot_pair = torch.empty(max(P, 1), **i32)
        self.pair_slot = torch.empty(max(P, 1), **i32)
        nws = moe_align_workspace_bytes(T, E, k)
        self.align_ws = torch.empty(max(nws // 4, 1), **i32)
        gws = moe_gemm_workspace_bytes(layer.experts, T, k)
        self.gemm_ws = torch.empty(max(gws // 4, 1), **i32)
        if layer.pt:
            # x and h each have one amax and one scale; h is kept in fp32 until
            # its tensor-wide scale is known, then quantised into hq
            f32 = dict(dtype=torch.float32, device=dev)
            self.xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
            self.x_amax = torch.empty(1, **f32)
            self.xs = torch.empty(1, **f32)
            self.h = torch.empty((R, I), **f32)
            self.h_amax = torch.empty(1, **f32)
            self.hq = torch.empty((R, I), dtype=torch.uint8, device=dev)
            self.hs = torch.empty(1, **f32)
        elif layer.mx:
            self.xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
            self.h = torch.empty((R, I), dtype=torch.uint8, device=dev)
            self.hs = torch.empty((R, I // 32), dtype=torch.uint8, device=dev)
        elif layer.fp8:
            self.xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
            self.h = torch.empty((R, I), dtype=torch.uint8, device=dev)
            self.hs = torch.empty((R, I // 128), dtype=torch.float32, device=dev)
        else:
            self.xq = self.xs = self.hs = None
            self.h = torch.empty((R, I), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((R, H), dtype=y_dtype, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)


def split_router(router_w):
    """Offline split of fp32 router weights [E,H] into bf16 hi / lo parts."""
    hi = torch.empty(router_w.shape, dtype=torch.bfloat16, device=router_w.device)
    lo = torch.empty_like(hi)
    moe_router_split(router_w.contiguous(), hi, lo)
    return hi, lo


def run_chain(layer: Layer, b: Buffers, x, k, logits=None, router_hi=None, router_lo=None, bias=None,
              bias_rows=None, stages=None, residual=None, norm_weight=None, eps=1e-6):
    """Enqueue the chain on torch's current stream.  ``stages`` (optional) maps a
    stage name to a (start_event, end_event) pair recorded around that stage.
    With ``residual`` (bf16 [T,H]) and ``norm_weight`` (bf16 [H]) the combine
    also adds the residual and applies RMSNorm: ``b.out`` receives the
    normalised rows and ``residual`` is updated in place to the sum."""
    def ev(name, i):
        if stages is not None and name in stages:
            stages[name][i].record()

    T = x.shape[0]
    if logits is None:
        ev("router", 0)
        moe_router_gemm(x, router_hi, router_lo, b.logits)
        ev("router", 1)
        logits = b.logits
    ev("route", 0)
    moe_route(logits, k, b.ids, b.w, bias=bias, bias_rows=bias_rows)
    ev("route", 1)
    ev("align", 0)
    moe_align(b.ids, layer.E, layer.shared, b.counts, b.offsets, b.slot_pair, b.pair_slot, b.align_ws)
    ev("align", 1)
    ex = layer.experts
    if layer.pt:
        ev("quant", 0)
        moe_tensor_amax(x, b.x_amax)
        moe_quant_tensor_fp8(x, b.x_amax, b.xq, b.xs)
        ev("quant", 1)
        ev("gemm13", 0)
        moe_gemm13(ex, b.xq, b.xs, b.offsets, b.slot_pair, T, k, b.h, b.h_amax, ws=b.gemm_ws)
        ev("gemm13", 1)
        ev("hquant", 0)
        moe_quant_tensor_fp8(b.h, b.h_amax, b.hq, b.hs)
        ev("hquant", 1)
    elif layer.fp8:
        ev("quant", 0)
        if layer.mx:
            moe_quant_rows_mxfp8(x, b.xq, b.xs)
        else:
            moe_quant_rows_fp8(x, b.xq, b.xs)
        ev("quant", 1)
        ev("gemm13", 0)
        moe_gemm13(ex, b.xq, b.xs, b.offsets, b.slot_pair, T, k, b.h, b.hs, ws=b.gemm_ws)
        ev("gemm13", 1)
    else:
        ev("gemm13", 0)
        moe_gemm13(ex, x, None, b.offsets, b.slot_pair, T, k, b.h, ws=b.gemm_ws)
        ev("gemm13", 1)
    ev("gemm2", 0)
    moe_gemm2(ex, b.hq if layer.pt else b.h, b.hs, b.offsets, T, k, b.y)
    ev("gemm2", 1)
    ev("combine", 0)
    if residual is None:
        moe_combine(b.y, b.pair_slot, b.w, T, k, layer.shared, b.out)
    else:
        moe_combine_rmsnorm(b.y, b.pair_slot, b.w, T, k, layer.shared, residual, norm_weight, eps, b.out,
                            res_out=residual)
    ev("combine", 1)
    return b
