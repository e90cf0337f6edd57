"""Shared GPU-vs-oracle checking for the parity tests.

The HIP chain runs through the C ABI (via the ctypes binding); the oracle runs
on the host copies of the identical input bytes.  Tolerances:
  * route ids, align outputs, fp8 codes/scales: bit-exact;
  * routing weights: |dw| <= 1e-6 (fp32 exp on the GPU vs fp64);
  * layer output: max|out - ref| <= 1e-2 max|ref| (bf16), 5e-2 max|ref| (fp8,
    against the oracle that emulates the quantisation steps exactly);
  * router logits: max|dl| <= 1e-5 max|ref| over [T,E] against fp64.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import workloads
from expert_layer_amd.chain import Buffers, Layer, run_chain, split_router
from oracle import oracle as orc

TOL = {"bf16": 1e-2, "fp8": 5e-2, "mxfp8": 5e-2, "fp8t": 5e-2}

# Requantised h (FP8 paths) against the oracle's on the checked rows.  The GPU
# forms h in fp32 from FP8 matrix-core dot products, the oracle in double
# rounded to fp32 once.  H_REL bounds the difference norm-wise: relative to
# the largest |h| of the quantisation group (a scale is that largest |h| / 448,
# so scales agree within H_REL relative), and a GPU code must be one that some
# value within H_REL * (group max) of the oracle's exact h rounds to.  Measured
# over every FP8 / MXFP8 / per-tensor test shape: up to 8.0e-5 of the group
# max (about 1.3 * 2^-14, more than fp32 sums alone give, so the FP8 dot
# products carry about 14 bits); H_REL = 2.5e-4 leaves a factor of 3.
H_REL = 2.5e-4


def log(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def host(t):
    return None if t is None else workloads.bits(t)


def run_gpu(wl, d, y_dtype=torch.float32):
    fp8 = wl.wtype == "fp8"
    layer = Layer.from_weights(d["w1"], d["w3"], d["w2"], d["sw1"], d["sw3"], d["sw2"], fp8=fp8,
                               mx=wl.wtype == "mxfp8", pt=wl.wtype == "fp8t")
    b = Buffers(layer, wl.T, wl.k, y_dtype=y_dtype, router=wl.router)
    hi = lo = None
    if wl.router:
        hi, lo = split_router(d["router_w"])
    run_chain(layer, b, d["x"], wl.k, logits=None if wl.router else d["logits"], router_hi=hi, router_lo=lo,
              bias=d["bias"], bias_rows=d["bias_rows"])
    torch.cuda.synchronize()
    return layer, b, (hi, lo)


def pair_slots(wl, rows, pair_slot):
    """Slot of every (checked token, rank) pair, ranks 0..k-1 then the shared expert: [nrows, k+S]."""
    P = wl.T * wl.k
    sl = pair_slot.reshape(wl.T, wl.k)[rows]
    if wl.shared:
        sl = np.concatenate([sl, (P + rows)[:, None]], axis=1)
    return sl


def check_codes(got_q, ref_q, v, slack, what):
    """got_q, ref_q: e4m3 codes; v: the oracle's h / scale (float64), same shape;
    slack: H_REL times the group's largest |v| (broadcastable).  Every GPU code
    must lie between the codes of v - slack and v + slack (rounding is
    monotonic, so those are the codes any h within the bound can take)."""
    dec = orc.e4m3_values()
    lo = orc.e4m3_code((v - slack).astype(np.float32))
    hi = orc.e4m3_code((v + slack).astype(np.float32))
    g = dec[got_q]
    ok = (dec[lo] <= g) & (g <= dec[hi])
    assert ok.all(), f"{what}: {int((~ok).sum())} codes outside the bound " \
                     f"(e.g. gpu {g[~ok][:4]}, ref {dec[ref_q[~ok]][:4]}, v {v[~ok][:4]})"
    # smallest h difference (in units of the slack) that explains each GPU code
    ag = np.abs(g)
    step = np.where(ag >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(ag, 2.0 ** -6))).astype(int) - 3),
                    2.0 ** -9)
    vs = np.clip(v, -448.0, 448.0)   # codes saturate at 448
    need = np.maximum(0.0, np.abs(vs - g) - 0.5 * step) / np.broadcast_to(slack, v.shape)
    return int((got_q != ref_q).sum()), float(need.max()) * H_REL


def check_requant(wl, b, tr, rows, pair_slot):
    """GPU requantised h (codes and scales) against the oracle's on the checked rows."""
    sl = pair_slots(wl, rows, pair_slot)
    I = wl.I
    href = tr["h"].astype(np.float64)                        # [n, k+S, I]
    gq = host(b.hq if wl.wtype == "fp8t" else b.h)[sl]        # [n, k+S, I]
    if wl.wtype == "fp8":
        gs = host(b.hs)[sl]                                    # [n, k+S, I/128]
        rs = tr["hs"]
        rel = np.abs(gs.astype(np.float64) - rs) / rs
        assert rel.max() <= H_REL, f"h scales: max relative difference {rel.max():.3e}"
        v = href / np.repeat(rs.astype(np.float64), 128, axis=-1)
        nbad, need = check_codes(gq, tr["hq"], v, H_REL * 448.0, "h codes")
        log(f"  h requant: scales max rel diff {rel.max():.2e}; codes differing {nbad} of {gq.size}, "
            f"implied h difference {need:.2e} of the group max")
    elif wl.wtype == "mxfp8":
        gs = host(b.hs)[sl]                                    # [n, k+S, I/32] E8M0
        rs = tr["hs"]
        amax = np.abs(href).reshape(*href.shape[:-1], I // 32, 32).max(axis=-1)
        lg = np.log2(np.maximum(amax, 1e-300))
        # the exponent is floor(log2(amax)) - 8: a byte may differ only where
        # the amax lies within H_REL of a power of two
        near_pow2 = np.abs(lg - np.round(lg)) <= 2.0 * H_REL
        diff = gs != rs
        assert not (diff & ~near_pow2).any(), "h MX scale bytes differ away from a power of two"
        assert np.all(np.abs(gs.astype(int) - rs.astype(int)) <= 1)
        same = np.repeat(~diff, 32, axis=-1)
        v = href * np.ldexp(1.0, 127 - np.repeat(rs.astype(np.int64), 32, axis=-1))
        vmax = np.repeat(np.abs(v).reshape(*v.shape[:-1], I // 32, 32).max(axis=-1), 32, axis=-1)
        nbad, need = check_codes(np.where(same, gq, tr["hq"]), tr["hq"], v, H_REL * vmax, "h MX codes")
        log(f"  h requant: scale bytes differing {int(diff.sum())}; codes differing {nbad} of {gq.size}, "
            f"implied h difference {need:.2e} of the block max")
    else:   # fp8t: the GPU keeps h in fp32 before its tensor-wide quantisation
        hg = host(b.h)[sl].astype(np.float64)
        dh = np.abs(hg - href).max()
        assert dh <= H_REL * np.abs(href).max(), f"h: max|diff| {dh:.3e} vs max|h| {np.abs(href).max():.3e}"
        v = href / tr["h_scale"]
        nbad, need = check_codes(gq, tr["hq"], v, H_REL * 448.0, "h codes")
        log(f"  h: max|diff| {dh:.2e} (max|h| {np.abs(href).max():.2e}); codes differing {nbad} of {gq.size}, "
            f"implied h difference {need:.2e} of the tensor max")


def checked_rows(wl, counts, offsets, slot_pair, nsample=256):
    """All rows for small T; else a seeded sample plus the first token of every touched expert."""
    if wl.T <= 512:
        return np.arange(wl.T, dtype=np.int64)
    rows = set(workloads.sample_rows(wl.T, nsample, wl.seed + 7).tolist())
    for e in range(wl.E):
        if counts[e] > 0:
            rows.add(int(slot_pair[offsets[e]]) // wl.k)
    return np.array(sorted(rows), dtype=np.int64)


def check_layer(wl, d, y_dtype=torch.float32, check_rows=None):
    """Run the chain on the GPU and compare every stage with the oracle."""
    t0 = time.time()
    log(f"{wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} S={wl.shared} {wl.wtype} y={y_dtype}")
    layer, b, (hi, lo) = run_gpu(wl, d, y_dtype)
    k, E = wl.k, wl.E
    x = host(d["x"])
    bias = host(d["bias"])
    bias_rows = host(d["bias_rows"])

    # ---- router front end
    if wl.router:
        w = host(d["router_w"])
        rhi, rlo = orc.router_split(w)
        assert np.array_equal(host(hi), rhi), "router split hi"
        assert np.array_equal(host(lo), rlo), "router split lo"
        glog = host(b.logits)
        ref = orc.router_logits(x, w)
        err = np.abs(glog.astype(np.float64) - ref).max()
        assert err <= 1e-5 * np.abs(ref).max(), f"router logits err {err} vs {np.abs(ref).max()}"
        logits = glog            # routing is evaluated on the GPU's logits
        ref_ids_exact, _ = orc.route(ref.astype(np.float32), k, bias, bias_rows)
    else:
        logits = host(d["logits"])

    # ---- route
    ids_ref, w_ref = orc.route(logits, k, bias, bias_rows)
    ids = host(b.ids)
    wts = host(b.w)
    assert np.array_equal(ids, ids_ref), f"route ids differ in {np.sum(ids != ids_ref)} entries"
    werr = np.abs(wts.astype(np.float64) - w_ref).max()
    assert werr <= 1e-6, f"route weights err {werr}"
    if wl.router:
        frac = np.mean(np.any(np.sort(ref_ids_exact, 1) != np.sort(ids_ref, 1), axis=1))
        log(f"  tokens whose top-k set differs under exact logits: {frac:.5f}")

    # ---- align
    counts, offsets, sp, ps = orc.align(ids_ref, E, wl.shared)
    assert np.array_equal(host(b.counts), counts), "align counts"
    assert np.array_equal(host(b.offsets), offsets), "align offsets"
    P = wl.T * k
    assert np.array_equal(host(b.slot_pair)[:P], sp), "align slot_pair"
    assert np.array_equal(host(b.pair_slot)[:P], ps), "align pair_slot"

    rows = checked_rows(wl, counts, offsets, sp) if check_rows is None else check_rows

    # ---- experts (oracle on the checked rows)
    if wl.wtype == "fp8":
        xq_ref, xs_ref = orc.quant_rows_fp8(x)
        assert np.array_equal(host(b.xq), xq_ref), "x quant codes"
        assert np.array_equal(host(b.xs), xs_ref), "x quant scales"
        used = np.unique(ids_ref[rows].ravel())
        ex = layer.experts.tensors
        qs = {}
        for name in ("w1", "w3", "w2"):
            src = d[name][torch.from_numpy(used).to(d[name].device)]
            q, s = orc.quant_blocks_fp8(host(src))
            assert np.array_equal(host(ex[name][torch.from_numpy(used).to(d[name].device)]), q), f"{name} codes"
            sname = "s" + name[1:]
            assert np.array_equal(host(ex[sname][torch.from_numpy(used).to(d[name].device)]), s), f"{name} scales"
            qs[name] = (q, s)
        sq = {}
        if wl.shared:
            for name in ("sw1", "sw3", "sw2"):
                q, s = orc.quant_blocks_fp8(host(d[name]))
                assert np.array_equal(host(ex[name]), q), f"{name} codes"
                assert np.array_equal(host(ex["ss" + name[2:]]), s), f"{name} scales"
                sq[name] = (q, s)
        remap = np.full(E, -1, np.int32)
        remap[used] = np.arange(used.size, dtype=np.int32)
        L = orc.Layer(qs["w1"][0], qs["w3"][0], qs["w2"][0],
                      sq["sw1"][0] if wl.shared else None, sq["sw3"][0] if wl.shared else None,
                      sq["sw2"][0] if wl.shared else None, wtype=1,
                      s1=qs["w1"][1], s3=qs["w3"][1], s2=qs["w2"][1],
                      ss1=sq["sw1"][1] if wl.shared else None, ss3=sq["sw3"][1] if wl.shared else None,
                      ss2=sq["sw2"][1] if wl.shared else None)
        ids_c = ids_ref.copy()
        ids_c[rows] = remap[ids_ref[rows]]
        ref, tr = orc.layer_rows(L, xq_ref, ids_c, w_ref, rows, xs=xs_ref, trace=True)
        check_requant(wl, b, tr, rows, ps)
    elif wl.wtype == "fp8t":
        # x: one scale; codes bit-exact
        xv = (x.astype(np.uint32) << 16).view(np.float32)   # the bf16 values, exactly
        assert float(host(b.x_amax)[0]) == float(np.abs(xv).max()), "x amax"
        xq_ref, xs_ref = orc.quant_tensor_fp8(x)
        assert np.array_equal(host(b.xq), xq_ref), "x codes"
        assert np.array_equal(host(b.xs), xs_ref), "x scale"
        # weights of the experts the checked rows use: one scale per matrix
        used = np.unique(ids_ref[rows].ravel())
        uidx = torch.from_numpy(used).to(d["w1"].device)
        ex = layer.experts.tensors
        qs = {}
        for name in ("w1", "w3", "w2"):
            q, s_ = orc.quant_tensor_fp8(host(d[name][uidx]), mats=used.size)
            assert np.array_equal(host(ex[name][uidx]), q), f"{name} codes"
            assert np.array_equal(host(ex["s" + name[1:]][uidx]), s_), f"{name} scales"
            qs[name] = (q, s_)
        sq = {}
        if wl.shared:
            for name in ("sw1", "sw3", "sw2"):
                q, s_ = orc.quant_tensor_fp8(host(d[name]))
                assert np.array_equal(host(ex[name]), q), f"{name} codes"
                assert np.array_equal(host(ex["ss" + name[2:]]), s_), f"{name} scales"
                sq[name] = (q, s_)
        # the GPU's h quantiser on its own fp32 h: amax and codes are exactly
        # the max and the per-tensor quantisation of those values
        hg = host(b.h)
        assert float(host(b.h_amax)[0]) == float(np.abs(hg).max()), "h amax"
        hq_g, hs_g = orc.quant_tensor_fp8(hg)
        assert np.array_equal(host(b.hq), hq_g), "h codes"
        assert np.array_equal(host(b.hs), hs_g), "h scale"
        del hg, hq_g
        remap = np.full(E, -1, np.int32)
        remap[used] = np.arange(used.size, dtype=np.int32)
        gs = lambda n, i: sq[n][i] if wl.shared else None   # noqa: E731
        h_scale = None
        if rows.size < wl.T:
            # a sample of the tokens: the h scale comes from the oracle's own
            # pass over the whole h tensor (every pair of every token), with
            # every expert's codes quantised by the oracle and checked against
            # the GPU's on the way
            t0 = time.time()
            xsc = float(xs_ref[0])

            def expert(g):
                if g == E:
                    return sq["sw1"][0], sq["sw1"][1][0], sq["sw3"][0], sq["sw3"][1][0]
                out = []
                for name in ("w1", "w3"):
                    q, s_ = orc.quant_tensor_fp8(host(d[name][g]))
                    assert np.array_equal(host(ex[name][g]), q), f"{name}[{g}] codes"
                    assert np.array_equal(host(ex["s" + name[1:]][g:g + 1]), s_), f"{name}[{g}] scale"
                    out += [q, float(s_[0])]
                return out
            amax = orc.pt_h_amax(xq_ref, xsc, ids_ref, E, wl.shared, expert)
            h_scale = float(np.float32(np.float32(amax) / np.float32(448.0))) if amax > 0 else 1.0
            gam = float(host(b.h_amax)[0])
            assert abs(gam - amax) <= H_REL * amax, f"h amax: gpu {gam} vs oracle {amax}"
            assert abs(float(host(b.hs)[0]) - h_scale) <= H_REL * h_scale, "h scale"
            log(f"  whole-h amax: oracle {amax:.6e}, gpu {gam:.6e} ({time.time() - t0:.1f}s)")
        L = orc.Layer(qs["w1"][0], qs["w3"][0], qs["w2"][0], gs("sw1", 0), gs("sw3", 0), gs("sw2", 0), wtype=3,
                      s1=qs["w1"][1], s3=qs["w3"][1], s2=qs["w2"][1],
                      ss1=gs("sw1", 1), ss3=gs("sw3", 1), ss2=gs("sw2", 1), h_scale=h_scale)
        ids_c = ids_ref.copy()
        ids_c[rows] = remap[ids_ref[rows]]
        ref, tr = orc.layer_rows(L, xq_ref, ids_c, w_ref, rows, xs=xs_ref, trace=True)
        if h_scale is None:
            gam = float(host(b.h_amax)[0])
            amax = float(np.abs(tr["h"]).max())
            assert abs(gam - amax) <= H_REL * amax, f"h amax: gpu {gam} vs oracle {amax}"
        check_requant(wl, b, tr, rows, ps)
    elif wl.wtype == "mxfp8":
        xq_ref, xs_ref = orc.quant_rows_mx(x)
        assert np.array_equal(host(b.xq), xq_ref), "x MX codes"
        assert np.array_equal(host(b.xs), xs_ref), "x MX scales"
        used = np.unique(ids_ref[rows].ravel())
        uidx = torch.from_numpy(used).to(d["w1"].device)
        ex = layer.experts.tensors
        qs = {}
        for name in ("w1", "w3", "w2"):
            q, s = orc.quant_rows_mx(host(d[name][uidx]))
            assert np.array_equal(host(ex[name][uidx]), q), f"{name} MX codes"
            assert np.array_equal(host(ex["s" + name[1:]][uidx]), s), f"{name} MX scales"
            qs[name] = (q, s)
        sq = {}
        if wl.shared:
            for name in ("sw1", "sw3", "sw2"):
                q, s = orc.quant_rows_mx(host(d[name]))
                assert np.array_equal(host(ex[name]), q), f"{name} MX codes"
                assert np.array_equal(host(ex["ss" + name[2:]]), s), f"{name} MX scales"
                sq[name] = (q, s)
        remap = np.full(E, -1, np.int32)
        remap[used] = np.arange(used.size, dtype=np.int32)
        gs = lambda n, i: sq[n][i] if wl.shared else None   # noqa: E731
        L = orc.Layer(qs["w1"][0], qs["w3"][0], qs["w2"][0], gs("sw1", 0), gs("sw3", 0), gs("sw2", 0), wtype=2,
                      s1=qs["w1"][1], s3=qs["w3"][1], s2=qs["w2"][1],
                      ss1=gs("sw1", 1), ss3=gs("sw3", 1), ss2=gs("sw2", 1))
        ids_c = ids_ref.copy()
        ids_c[rows] = remap[ids_ref[rows]]
        ref, tr = orc.layer_rows(L, xq_ref, ids_c, w_ref, rows, xs=xs_ref, trace=True)
        check_requant(wl, b, tr, rows, ps)
    else:
        L = orc.Layer(host(d["w1"]), host(d["w3"]), host(d["w2"]), host(d["sw1"]), host(d["sw3"]), host(d["sw2"]))
        ref = orc.layer_rows(L, x, ids_ref, w_ref, rows)
    out = b.out[torch.from_numpy(rows).to(b.out.device)].float().cpu().numpy()
    err = np.abs(out - ref).max()
    scale = np.abs(ref).max()
    tol = TOL[wl.wtype]
    log(f"  rows checked {rows.size}, max|err| {err:.3e}, max|ref| {scale:.3e}, ratio {err / scale:.3e} "
        f"(tol {tol}), {time.time() - t0:.1f}s")
    assert err <= tol * scale, f"layer output err {err} > {tol} * {scale}"
    return layer, b
