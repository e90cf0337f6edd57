"""Pins of the oracle's per-tensor FP8 mode (HPC-Ops page, main functions:
GroupGEMM FP8 with per-tensor as well as block-wise scales) against facts
that do not come from the oracle's own per-tensor code:

* the quantiser: the largest magnitude maps to +-448, every code is within
  half an E4M3 step of its value, an all-zero tensor gets scale 1, and a tensor
  that is exactly one 128x128 block (or one 1x128 group) quantises exactly as
  the already pinned block (row) quantiser does;
* the layer: with every tensor a single block it equals the pinned
  block-scaled layer; with constant weights chosen so that every quantisation
  step is exact it equals a closed form built from the quantiser's scales;
* the h scale: passing the closed-form h scale explicitly gives the same
  result, and one that does not divide the h values into exact codes does not.
"""
import numpy as np
import pytest

from oracle import oracle as orc


def _bf16(values):
    """fp32 -> bf16 bit patterns by the pinned oracle rounding."""
    v = np.ascontiguousarray(values, np.float32)
    return np.array([orc.lib().orc_bf16_nearest(float(f)) for f in v.ravel()], np.uint16).reshape(v.shape)


def _rand_bf16(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)   # truncation: any bf16 values will do


def _check_codes(v, q, s):
    dec = orc.e4m3_value(q) * float(s)
    amax = np.abs(v).max()
    at_max = np.abs(v) == amax
    assert np.all(np.abs(orc.e4m3_value(q[at_max])) == 448.0)
    err = np.abs(dec - v)
    # normal E4M3 values have 3 mantissa bits: half a step is 2^-4 relative;
    # below 2^-6 (subnormal) the step is 2^-9, times the scale
    assert np.all(err <= np.maximum(np.abs(v) * 2.0 ** -4, float(s) * 2.0 ** -10) * (1 + 1e-6))


@pytest.mark.parametrize("f32", [False, True])
def test_quant_tensor_bounds_and_extremes(f32):
    xb = _rand_bf16((3, 40, 50), 1, scale=3.0)
    x = orc.bf16_value(xb).astype(np.float32) if f32 else xb
    q, s = orc.quant_tensor_fp8(x, mats=3)
    vals = orc.bf16_value(xb)
    for m in range(3):
        _check_codes(vals[m].ravel(), q[m].ravel(), s[m])
    z = np.zeros((2, 64), np.float32 if f32 else np.uint16)
    qz, sz = orc.quant_tensor_fp8(z, mats=2)
    assert np.all(sz == 1.0) and np.all(qz == 0)


def test_quant_tensor_one_block_is_the_block_quantiser():
    w = _rand_bf16((4, 128, 128), 2, scale=0.02)
    qt, st = orc.quant_tensor_fp8(w, mats=4)
    qb, sb = orc.quant_blocks_fp8(w)
    assert np.array_equal(qt, qb)
    assert np.array_equal(st, sb.reshape(4))
    x = _rand_bf16((1, 128), 3)
    qt, st = orc.quant_tensor_fp8(x)
    qr, sr = orc.quant_rows_fp8(x)
    assert np.array_equal(qt, qr) and np.array_equal(st, sr.reshape(1))


def test_layer_single_blocks_equal_block_layer():
    """T = 1, k = 1, H = I = 128: x, every weight matrix and h are each one
    block, so per-tensor and 128x128-block scaling are the same quantisation."""
    E, H, I = 3, 128, 128
    w1 = _rand_bf16((E, I, H), 4, 0.05)
    w3 = _rand_bf16((E, I, H), 5, 0.05)
    w2 = _rand_bf16((E, H, I), 6, 0.05)
    x = _rand_bf16((1, H), 7)
    q1, s1 = orc.quant_tensor_fp8(w1, E)
    q3, s3 = orc.quant_tensor_fp8(w3, E)
    q2, s2 = orc.quant_tensor_fp8(w2, E)
    xq, xs = orc.quant_tensor_fp8(x)
    ids = np.array([[2]], np.int32)
    wts = np.array([[0.75]])
    rows = np.array([0])
    Lt = orc.Layer(q1, q3, q2, wtype=3, s1=s1, s3=s3, s2=s2)
    out_t = orc.layer_rows(Lt, xq, ids, wts, rows, xs=xs)
    Lb = orc.Layer(q1, q3, q2, wtype=1, s1=s1.reshape(E, 1, 1), s3=s3.reshape(E, 1, 1), s2=s2.reshape(E, 1, 1))
    out_b = orc.layer_rows(Lb, xq, ids, wts, rows, xs=xs.reshape(1, 1))
    assert np.abs(out_b).max() > 0
    assert np.allclose(out_t, out_b, rtol=1e-12, atol=1e-12 * np.abs(out_b).max())


def _closed_form_case():
    """Constant weights: x = 1, w1[e] = c1 * 2^-a[e], w3 = c3, w2[e] = c2[e];
    every tensor is constant, so every code is 448 (0x7E); g is large enough
    that SiLU(g) = g in double; h values differ by powers of two only, so the
    h codes are exact too."""
    E, H, I, T, k = 4, 256, 128, 6, 2
    a = np.array([0, 1, 3, 2])
    a_sh = 1
    c1, c3 = 4.0, 0.25
    c2 = np.array([0.125, 0.0625, 0.375, 0.1875])
    c2_sh = 0.3125
    w1 = np.stack([np.full((I, H), c1 * 2.0 ** -a[e], np.float32) for e in range(E)])
    w3 = np.full((E, I, H), c3, np.float32)
    w2 = np.stack([np.full((H, I), c2[e], np.float32) for e in range(E)])
    sw1 = np.full((I, H), c1 * 2.0 ** -a_sh, np.float32)
    sw3 = np.full((I, H), c3, np.float32)
    sw2 = np.full((H, I), c2_sh, np.float32)
    b = {n: _bf16(v) for n, v in dict(w1=w1, w3=w3, w2=w2, sw1=sw1, sw3=sw3, sw2=sw2, x=np.ones((T, H))).items()}
    q = {}
    for n in ("w1", "w3", "w2"):
        q[n] = orc.quant_tensor_fp8(b[n], E)
    for n in ("sw1", "sw3", "sw2"):
        q[n] = orc.quant_tensor_fp8(b[n])
    xq, xs = orc.quant_tensor_fp8(b["x"])
    ids = np.array([[0, 1], [1, 2], [3, 0], [2, 3], [0, 2], [1, 3]], np.int32)
    wts = np.array([[0.6, 0.4], [0.3, 0.7], [0.55, 0.45], [0.2, 0.8], [0.9, 0.1], [0.5, 0.5]])
    for n in q:
        assert np.all(q[n][0] == 0x7E)
    assert np.all(xq == 0x7E)
    # closed form from the quantiser's scales
    xsc = float(xs[0])
    g = {e: H * 448.0 * 448.0 * xsc * float(q["w1"][1][e]) for e in range(E)}
    g["s"] = H * 448.0 * 448.0 * xsc * float(q["sw1"][1][0])
    u = {e: H * 448.0 * 448.0 * xsc * float(q["w3"][1][e]) for e in range(E)}
    u["s"] = H * 448.0 * 448.0 * xsc * float(q["sw3"][1][0])
    assert min(g.values()) > 40.0          # SiLU(g) = g exactly in double
    h = {e: np.float32(g[e] * u[e]) for e in g}
    hmax = max(h.values())
    sh = np.float32(hmax / np.float32(448.0))
    hcode = {e: float(h[e]) / float(sh) for e in h}
    for e in h:   # h / sh is 448 times a power of two within 2^-20: exact E4M3 code
        ratio = hcode[e] / 448.0
        assert abs(ratio - 2.0 ** np.round(np.log2(ratio))) < 1e-6
    hdec = {e: 448.0 * 2.0 ** np.round(np.log2(hcode[e] / 448.0)) for e in h}
    s2 = {e: float(q["w2"][1][e]) for e in range(E)}
    s2["s"] = float(q["sw2"][1][0])
    y = {e: I * hdec[e] * 448.0 * float(sh) * s2[e] for e in h}
    want = np.array([[sum(wts[t, j] * y[ids[t, j]] for j in range(k)) + y["s"]] * H for t in range(T)])
    return q, xq, xs, ids, wts, want, float(sh)


def test_layer_closed_form():
    q, xq, xs, ids, wts, want, sh = _closed_form_case()
    L = orc.Layer(q["w1"][0], q["w3"][0], q["w2"][0], q["sw1"][0], q["sw3"][0], q["sw2"][0], wtype=3,
                  s1=q["w1"][1], s3=q["w3"][1], s2=q["w2"][1], ss1=q["sw1"][1], ss3=q["sw3"][1], ss2=q["sw2"][1])
    rows = np.arange(ids.shape[0])
    got = orc.layer_rows(L, xq, ids, wts, rows, xs=xs)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


def test_layer_given_h_scale():
    q, xq, xs, ids, wts, want, sh = _closed_form_case()
    kw = dict(wtype=3, s1=q["w1"][1], s3=q["w3"][1], s2=q["w2"][1], ss1=q["sw1"][1], ss3=q["sw3"][1],
              ss2=q["sw2"][1])
    rows = np.arange(2)   # a subset of the tokens, with the whole tensor's h scale given
    L = orc.Layer(q["w1"][0], q["w3"][0], q["w2"][0], q["sw1"][0], q["sw3"][0], q["sw2"][0], h_scale=sh, **kw)
    got = orc.layer_rows(L, xq, ids, wts, rows, xs=xs)
    assert np.allclose(got, want[:2], rtol=1e-12, atol=0)
    L2 = orc.Layer(q["w1"][0], q["w3"][0], q["w2"][0], q["sw1"][0], q["sw3"][0], q["sw2"][0], h_scale=3 * sh, **kw)
    other = orc.layer_rows(L2, xq, ids, wts, rows, xs=xs)
    assert not np.allclose(other, want[:2], rtol=1e-3)


def test_whole_h_amax_closed_form():
    """The whole-tensor h pass (exact code dot products as one float64 matrix
    product, then the layer's own scaling) finds the closed-form largest h."""
    q, xq, xs, ids, wts, want, sh = _closed_form_case()
    E = q["w1"][0].shape[0]

    def expert(g):
        if g == E:
            return q["sw1"][0], q["sw1"][1][0], q["sw3"][0], q["sw3"][1][0]
        return q["w1"][0][g], q["w1"][1][g], q["w3"][0][g], q["w3"][1][g]
    amax = orc.pt_h_amax(xq, xs[0], ids, E, True, expert)
    assert np.float32(amax / np.float32(448.0)) == np.float32(sh)


def _random_pt_layer(seed, E=5, H=256, I=256, T=30, k=2):
    rng = np.random.default_rng(seed)
    b = {"w1": _rand_bf16((E, I, H), seed + 1, 0.05), "w3": _rand_bf16((E, I, H), seed + 2, 0.05),
         "w2": _rand_bf16((E, H, I), seed + 3, 0.05), "sw1": _rand_bf16((I, H), seed + 4, 0.05),
         "sw3": _rand_bf16((I, H), seed + 5, 0.05), "sw2": _rand_bf16((H, I), seed + 6, 0.05)}
    q = {n: orc.quant_tensor_fp8(b[n], E) for n in ("w1", "w3", "w2")}
    q.update({n: orc.quant_tensor_fp8(b[n]) for n in ("sw1", "sw3", "sw2")})
    xq, xs = orc.quant_tensor_fp8(_rand_bf16((T, H), seed + 7))
    ids, wts = orc.route(rng.standard_normal((T, E)).astype(np.float32), k)
    return q, xq, xs, ids, wts


def test_whole_h_pass_equals_layer_h():
    """The h of every pair from the whole-tensor pass equals, bit for bit, the
    h the layer's plain loops compute, and so do the amax and the h scale the
    layer takes when every token is evaluated."""
    q, xq, xs, ids, wts = _random_pt_layer(70)
    E, T, k = q["w1"][0].shape[0], ids.shape[0], ids.shape[1]
    kw = dict(wtype=3, s1=q["w1"][1], s3=q["w3"][1], s2=q["w2"][1], ss1=q["sw1"][1], ss3=q["sw3"][1],
              ss2=q["sw2"][1])
    L = orc.Layer(q["w1"][0], q["w3"][0], q["w2"][0], q["sw1"][0], q["sw3"][0], q["sw2"][0], **kw)
    rows = np.arange(T)
    out, tr = orc.layer_rows(L, xq, ids, wts, rows, xs=xs, trace=True)
    for t in range(T):
        for j in range(k + 1):
            g = E if j == k else ids[t, j]
            w1q, s1 = (q["sw1"][0], q["sw1"][1][0]) if g == E else (q["w1"][0][g], q["w1"][1][g])
            w3q, s3 = (q["sw3"][0], q["sw3"][1][0]) if g == E else (q["w3"][0][g], q["w3"][1][g])
            h = orc.pt_h_rows(xq[t:t + 1], xs[0], w1q, s1, w3q, s3)[0]
            assert np.array_equal(h, tr["h"][t, j]), (t, j)

    def expert(g):
        if g == E:
            return q["sw1"][0], q["sw1"][1][0], q["sw3"][0], q["sw3"][1][0]
        return q["w1"][0][g], q["w1"][1][g], q["w3"][0][g], q["w3"][1][g]
    amax = orc.pt_h_amax(xq, xs[0], ids, E, True, expert)
    assert amax == float(np.abs(tr["h"]).max())
    assert tr["h_scale"] == float(np.float32(np.float32(amax) / np.float32(448.0)))
    # a subset of the tokens with the whole tensor's scale given is the same rows of the whole
    sub = np.array([3, 11, 29])
    L2 = orc.Layer(q["w1"][0], q["w3"][0], q["w2"][0], q["sw1"][0], q["sw3"][0], q["sw2"][0],
                   h_scale=tr["h_scale"], **kw)
    assert np.array_equal(orc.layer_rows(L2, xq, ids, wts, sub, xs=xs), out[sub])
    # h codes of the trace are the quantisation of the trace's h with that scale
    hq, hs = orc.quant_tensor_fp8(tr["h"])
    assert np.array_equal(hq, tr["hq"]) and float(hs[0]) == tr["h_scale"]


def test_quant_tensor_thread_count_does_not_matter():
    x = _rand_bf16((3, 300000), 80, 2.0)
    q1, s1 = orc.quant_tensor_fp8(x, mats=3, nthreads=1)
    q8, s8 = orc.quant_tensor_fp8(x, mats=3, nthreads=8)
    assert np.array_equal(q1, q8) and np.array_equal(s1, s8)
