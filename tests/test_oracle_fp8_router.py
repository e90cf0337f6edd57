"""Pins for the oracle's FP8 codec/quantisers and the split-BF16 router (CPU only).

FP8: OCP E4M3FN (the pages say "FP8" with 128x128 blockwise weight scales, PR
#54160 report, implementation item 4).  Expected codes come from torch's own
float8_e4m3fn conversion (a library routine) and from hand-derived spec points.
Router: the HPC-Ops page ("Router GEMM" under main functions and technical
principles) splits fp32 weights into a high bf16 part plus a residual bf16
part with scale 1/256; expected bits come from torch's bf16 conversion, the
closed-form error bound and the page's accuracy claim (error 1/36 of TF32's,
"core advantages").
"""
import json
import os
import struct

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(nan, np.isnan(ours))
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_golden_points(orc):
    g = json.load(open(os.path.join(GOLDEN, "e4m3_points.json")))
    for code, val in g["decode"]:
        assert orc.e4m3_value(np.array([code]))[0] == val
    for c in g["encode"]:
        assert int(orc.e4m3_code(np.array([c["v"]]))[0]) == c["code"], c["why"]


def _finite_positive_values():
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return vals  # codes 0..126 (0x7F is NaN)


def test_e4m3_encode_vs_torch_boundaries(orc):
    vals = _finite_positive_values()
    mids = (vals[:-1] + vals[1:]) / 2.0
    pts = np.concatenate([vals, mids]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    allv = np.concatenate([pts, up, dn])
    allv = allv[np.abs(allv) <= 448.0]
    allv = np.concatenate([allv, -allv])
    np.testing.assert_array_equal(orc.e4m3_code(allv), _torch_e4m3(allv))


def test_e4m3_encode_vs_torch_random(orc):
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)]).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    np.testing.assert_array_equal(orc.e4m3_code(v), _torch_e4m3(v))


def test_e4m3_saturates(orc):
    v = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.0e38], np.float32)
    assert np.all(orc.e4m3_code(v) == 0x7E)
    assert np.all(orc.e4m3_code(-v) == 0xFE)


def _ref_group_quant(xf):
    """Per-row groups of 128: s = amax/448 (fp32 division), code = torch e4m3 of fp32(x/s)."""
    rows, cols = xf.shape
    g = xf.reshape(rows, cols // 128, 128)
    amax = np.abs(g).max(-1).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = _torch_e4m3((g / s[..., None]).astype(np.float32)).reshape(rows, cols)
    return q, s


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_float(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_quant_rows_vs_library(orc):
    rng = np.random.default_rng(5)
    x = _bf16_bits(rng.standard_normal((37, 512)) * np.array([1e-3, 1, 50, 1e3])[rng.integers(0, 4, (37, 1))])
    x[3, 128:256] = 0                       # all-zero group: scale 1, codes 0
    q, s = orc.quant_rows_fp8(x)
    rq, rs = _ref_group_quant(_bf16_float(x))
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(q, rq)
    assert s[3, 1] == 1.0 and np.all(q[3, 128:256] == 0)
    # the largest magnitude of a nonzero group maps to +-448 (code 0x7E / 0xFE)
    assert np.all((q.reshape(37, 4, 128) & 0x7F).max(-1)[s != 1.0] == 0x7E)


def test_quant_blocks_vs_library(orc):
    rng = np.random.default_rng(6)
    w = _bf16_bits(rng.standard_normal((2, 256, 384)) * 0.02)
    w[1, 128:, :128] = 0
    q, s = orc.quant_blocks_fp8(w)
    assert s.shape == (2, 2, 3)
    wf = _bf16_float(w)
    for m in range(2):
        for bi in range(2):
            for bj in range(3):
                blk = wf[m, bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
                amax = np.float32(np.abs(blk).max())
                sc = amax / np.float32(448.0) if amax > 0 else np.float32(1.0)
                assert s[m, bi, bj] == sc
                np.testing.assert_array_equal(q[m, bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128],
                                              _torch_e4m3((blk / sc).astype(np.float32)))


def test_expert_fp8_vs_dequantised_dense(orc):
    """Blockwise-scaled sums equal the dense product of dequantised operands."""
    rng = np.random.default_rng(8)
    H, I = 384, 256
    x = _bf16_bits(rng.standard_normal((1, H)))
    ws = [_bf16_bits(rng.standard_normal(sh) * 0.02) for sh in ((I, H), (I, H), (H, I))]
    xq, xs = orc.quant_rows_fp8(x)
    (w1q, s1), (w3q, s3), (w2q, s2) = (orc.quant_blocks_fp8(w) for w in ws)
    h, y = orc.expert_fp8(xq[0], xs[0], w1q, s1, w3q, s3, w2q, s2)

    dec = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xd = dec[xq[0]] * np.repeat(xs[0].astype(np.float64), 128)

    def deq(q, s):
        return dec[q] * np.kron(s.astype(np.float64), np.ones((128, 128)))

    g = deq(w1q, s1) @ xd
    u = deq(w3q, s3) @ xd
    href = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    np.testing.assert_array_equal(h.astype(np.float32), href)
    hq, hs = _ref_group_quant(href[None])
    hd = dec[hq[0]] * np.repeat(hs[0].astype(np.float64), 128)
    yref = deq(w2q, s2) @ hd
    np.testing.assert_allclose(y, yref, rtol=1e-11, atol=1e-12 * np.abs(yref).max())


# ------------------------------------------------------------------ router split
def test_split_golden(orc):
    for c in json.load(open(os.path.join(GOLDEN, "split_cases.json")))["cases"]:
        w = np.array([struct.unpack("<f", struct.pack("<I", int(c["w_bits"], 16)))[0]], np.float32)
        hi, lo = orc.router_split(w)
        assert int(hi[0]) == int(c["hi"], 16), c["why"]
        assert int(lo[0]) == int(c["lo"], 16), c["why"]


def test_split_vs_library_and_bound(orc):
    rng = np.random.default_rng(9)
    w = np.concatenate([rng.standard_normal(100000) * 0.01, rng.standard_normal(1000) * 1e3,
                        rng.standard_normal(1000) * 1e-6]).astype(np.float32)
    hi, lo = orc.router_split(w)
    np.testing.assert_array_equal(hi, _bf16_bits(w))
    resid = (w - _bf16_float(hi)).astype(np.float32)
    np.testing.assert_array_equal(lo, _bf16_bits(resid * np.float32(256.0)))
    # |w - (hi + lo/256)| <= 2^(e-17) with 2^e <= |w|
    approx = _bf16_float(hi).astype(np.float64) + _bf16_float(lo).astype(np.float64) / 256.0
    e = np.floor(np.log2(np.abs(w.astype(np.float64))))
    assert np.all(np.abs(w.astype(np.float64) - approx) <= np.exp2(e - 17))


def test_router_logits_vs_matmul(orc):
    rng = np.random.default_rng(10)
    x = _bf16_bits(rng.standard_normal((9, 256)))
    w = (rng.standard_normal((16, 256)) * 0.01).astype(np.float32)
    ref = _bf16_float(x).astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_allclose(orc.router_logits(x, w), ref, rtol=1e-13, atol=1e-16)


def _tf32(a):
    """Round fp32 to TF32 (10 explicit mantissa bits), nearest even."""
    u = a.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0xFFF + ((u >> 13) & 1)) & ~np.uint64(0x1FFF)
    return u.astype(np.uint32).view(np.float32)


def test_split_error_is_below_tf32_claim(orc):
    """HPC-Ops page ('core advantages'): split-BF16 error is 1/36 of TF32's."""
    rng = np.random.default_rng(12)
    x = _bf16_bits(rng.standard_normal((32, 2048)))
    w = (rng.standard_normal((64, 2048)) * 0.01).astype(np.float32)
    exact = orc.router_logits(x, w)
    hi, lo = orc.router_split(w)
    xf = _bf16_float(x).astype(np.float64)
    split = xf @ (_bf16_float(hi).astype(np.float64) + _bf16_float(lo).astype(np.float64) / 256.0).T
    tf32 = xf @ _tf32(w).astype(np.float64).T
    err_split = np.abs(split - exact).max()
    err_tf32 = np.abs(tf32 - exact).max()
    assert err_split <= err_tf32 / 36.0, (err_split, err_tf32)
