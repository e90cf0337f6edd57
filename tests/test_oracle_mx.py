"""Pins for the oracle's MXFP8 path (CPU only).

MXFP8 (listed with the FP8 blockwise 128x128 scales in the PR #54160 report,
implementation item 4) follows the OCP Microscaling definition: blocks of 32
values along K share an E8M0 power-of-two scale 2^X with X = floor(log2(amax))
- 8, elements are E4M3 codes of v / 2^X.  What pins it here, other than the
oracle itself:
* a property that fixes the exponent rule: the largest element magnitude of
  every nonzero block lands in [256, 448] (an off-by-one in X, or ceil instead
  of floor, moves it to [128, 256] or saturates half the block);
* given the scale, the element codes equal torch's float8_e4m3fn conversion
  of the clamped scaled values (a library routine);
* hand-derived blocks (tests/golden/mx_blocks.json);
* the layer against a dense numpy computation on dequantised operands (block
  scales applied elementwise, so block indexing and exponent sums are checked).
"""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _dequant(q, s):
    """codes [..., K], E8M0 bytes [..., K/32] -> float64 values."""
    v = _e4m3_values(q)
    sc = np.ldexp(1.0, s.astype(np.int64) - 127)
    return v * np.repeat(sc, 32, axis=-1)


def _random_blocks(rng, nblocks):
    """bf16 bit patterns of blocks whose magnitudes span many binades."""
    mag = np.ldexp(1.0, rng.integers(-60, 60, size=(nblocks, 1)))
    v = (rng.standard_normal((nblocks, 32)) * mag).astype(np.float32)
    return _bf16_bits(v)


def test_mx_exponent_places_block_max_in_top_binade(orc):
    rng = np.random.default_rng(5)
    x = _random_blocks(rng, 4000)
    q, s = orc.quant_rows_mx(x.reshape(-1, 32 * 8))
    q, s = q.reshape(-1, 32), s.reshape(-1)
    vals = np.abs(_e4m3_values(q))
    top = vals.max(axis=1)
    assert np.all(top >= 256) and np.all(top <= 448), (top.min(), top.max())
    # and the scale really is the power of two that the codes were divided by:
    # below 448 * 2^X an element is off by at most half an E4M3 step (<= 16 * 2^X
    # <= blockmax / 16); at or above it, it saturates to exactly 448 * 2^X
    deq = _dequant(q.reshape(-1, 32), s.reshape(-1, 1))
    xv = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy().reshape(-1, 32)
    scale = np.ldexp(1.0, s.astype(np.int64) - 127)[:, None]
    sat = np.abs(xv) >= 448.0 * scale
    blockmax = np.abs(xv).max(axis=1, keepdims=True)
    err = np.abs(deq - xv)
    assert np.all(err[~sat] <= np.broadcast_to(blockmax / 16.0, err.shape)[~sat])
    np.testing.assert_array_equal(deq[sat], np.sign(xv[sat]) * np.broadcast_to(448.0 * scale, xv.shape)[sat])
    assert sat.any()   # the saturating corner of the definition is exercised


def test_mx_elements_match_torch_given_the_scale(orc):
    rng = np.random.default_rng(6)
    x = _random_blocks(rng, 3000).reshape(-1, 64)
    q, s = orc.quant_rows_mx(x)
    xv = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    scaled = xv * np.repeat(np.ldexp(1.0, 127 - s.astype(np.int64)), 32, axis=1)
    ref = torch.from_numpy(np.clip(scaled, -448.0, 448.0).astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(q, ref.view(torch.uint8).numpy())


def test_mx_golden_blocks(orc):
    g = json.load(open(os.path.join(GOLDEN, "mx_blocks.json")))
    for blk in g["blocks"]:
        v = np.zeros(32, np.float32)
        v[: len(blk["values"])] = blk["values"]
        q, s = orc.quant_rows_mx(_bf16_bits(v)[None])
        assert int(s[0, 0]) == blk["scale_byte"], blk["why"]
        want = np.zeros(32, np.uint8)
        want[: len(blk["codes"])] = blk["codes"]
        np.testing.assert_array_equal(q[0], want, err_msg=blk["why"])


def test_mx_f32_rows_follow_the_same_rule(orc):
    rng = np.random.default_rng(7)
    x = _random_blocks(rng, 200).reshape(-1, 128)
    xv = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    q1, s1 = orc.quant_rows_mx(x)
    q2, s2 = orc.quant_rows_mx_f32(xv)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)


def _dense_mx_layer(orc, xq, xs, w1q, w1s, w3q, w3s, w2q, w2s, sw, ids, wts, rows):
    """The MXFP8 layer with every GEMM a dense numpy product of dequantised operands."""
    x = _dequant(xq, xs)
    W1, W3, W2 = _dequant(w1q, w1s), _dequant(w3q, w3s), _dequant(w2q, w2s)
    S1, S3, S2 = (_dequant(*t) for t in sw) if sw is not None else (None, None, None)
    k = ids.shape[1]
    out = np.zeros((len(rows), W2.shape[1]))

    def ffn(xr, a1, a3, a2):
        g, u = a1 @ xr, a3 @ xr
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        hq, hs = orc.quant_rows_mx_f32(h[None])
        return a2 @ _dequant(hq, hs)[0]

    for r, t in enumerate(rows):
        for j in range(k):
            e = ids[t, j]
            out[r] += wts[t, j] * ffn(x[t], W1[e], W3[e], W2[e])
        if S1 is not None:
            out[r] += ffn(x[t], S1, S3, S2)
    return out


def test_mx_layer_matches_dense_dequantised(orc):
    rng = np.random.default_rng(8)
    T, H, I, E, k = 12, 256, 128, 4, 2   # H, I multiples of 128 (the layer envelope)
    f = lambda *shape, sd: _bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))
    xq, xs = orc.quant_rows_mx(f(T, H, sd=1.0))
    w1q, w1s = orc.quant_rows_mx(f(E, I, H, sd=0.05))
    w3q, w3s = orc.quant_rows_mx(f(E, I, H, sd=0.05))
    w2q, w2s = orc.quant_rows_mx(f(E, H, I, sd=0.05))
    sw = [orc.quant_rows_mx(f(I, H, sd=0.05)), orc.quant_rows_mx(f(I, H, sd=0.05)),
          orc.quant_rows_mx(f(H, I, sd=0.05))]
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    wts = rng.random((T, k))
    rows = np.arange(T, dtype=np.int64)
    L = orc.Layer(w1q, w3q, w2q, sw[0][0], sw[1][0], sw[2][0], wtype=2, s1=w1s, s3=w3s, s2=w2s,
                  ss1=sw[0][1], ss3=sw[1][1], ss2=sw[2][1])
    got = orc.layer_rows(L, xq, ids, wts, rows, xs=xs)
    want = _dense_mx_layer(orc, xq, xs, w1q, w1s, w3q, w3s, w2q, w2s, sw, ids, wts, rows)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12 * np.abs(want).max())


def test_mx_layer_trace_is_the_requantised_h(orc):
    """The layer's traced h equals the dense dequantised h (fp32), and its traced
    codes and scale bytes are the MX rule applied to that h (quant_rows_mx_f32)."""
    rng = np.random.default_rng(9)
    T, H, I, E, k = 6, 256, 256, 3, 2
    f = lambda *shape, sd: _bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))
    xq, xs = orc.quant_rows_mx(f(T, H, sd=1.0))
    w1q, w1s = orc.quant_rows_mx(f(E, I, H, sd=0.05))
    w3q, w3s = orc.quant_rows_mx(f(E, I, H, sd=0.05))
    w2q, w2s = orc.quant_rows_mx(f(E, H, I, sd=0.05))
    sw = [orc.quant_rows_mx(f(I, H, sd=0.05)), orc.quant_rows_mx(f(I, H, sd=0.05)),
          orc.quant_rows_mx(f(H, I, sd=0.05))]
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    wts = rng.random((T, k))
    rows = np.arange(T, dtype=np.int64)
    L = orc.Layer(w1q, w3q, w2q, sw[0][0], sw[1][0], sw[2][0], wtype=2, s1=w1s, s3=w3s, s2=w2s,
                  ss1=sw[0][1], ss3=sw[1][1], ss2=sw[2][1])
    _, tr = orc.layer_rows(L, xq, ids, wts, rows, xs=xs, trace=True)
    x = _dequant(xq, xs)
    W1, W3 = _dequant(w1q, w1s), _dequant(w3q, w3s)
    S1, S3 = _dequant(*sw[0]), _dequant(*sw[1])
    for t in range(T):
        for j in range(k + 1):
            a1, a3 = (S1, S3) if j == k else (W1[ids[t, j]], W3[ids[t, j]])
            g, u = a1 @ x[t], a3 @ x[t]
            h = g / (1.0 + np.exp(-g)) * u
            np.testing.assert_allclose(tr["h"][t, j], h, rtol=2e-7, atol=1e-30)
    hq, hs = orc.quant_rows_mx_f32(tr["h"])
    np.testing.assert_array_equal(tr["hq"], hq)
    np.testing.assert_array_equal(tr["hs"], hs)
