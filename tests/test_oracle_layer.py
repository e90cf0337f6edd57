"""Pins for the oracle's expert FFN and whole-layer combine (CPU only).

The layer (PR #54160 report, "features and motivation": routed experts plus a
shared expert; HPC-Ops page, FusedMoE: Gate-Up GEMM, Down GEMM, top-k weighted
combine) is checked against a dense formulation over every token-expert pair
with a gate matrix, computed with numpy/torch matrix products, and against
special cases that reduce to a textbook SwiGLU MLP.
"""
import numpy as np
import pytest
import torch

import workloads


def _f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _ffn_dense(X, w1, w3, w2):
    g = X @ _f(w1).T
    u = X @ _f(w3).T
    return (g / (1.0 + np.exp(-g)) * u) @ _f(w2).T


def _rand_layer(rng, E, H, I, shared, std=0.05):
    def b(shape):
        return torch.from_numpy(rng.standard_normal(shape) * std).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w1, w3, w2 = b((E, I, H)), b((E, I, H)), b((E, H, I))
    sw = (b((I, H)), b((I, H)), b((H, I))) if shared else (None, None, None)
    return w1, w3, w2, sw


def _dense_layer(X, ids, w, w1, w3, w2, sw):
    T = X.shape[0]
    E = w1.shape[0]
    G = np.zeros((T, E))
    for t in range(T):
        G[t, ids[t]] = w[t]
    out = np.zeros((T, w2.shape[1]))
    for e in range(E):
        out += G[:, e:e + 1] * _ffn_dense(X, w1[e], w3[e], w2[e])
    if sw[0] is not None:
        out += _ffn_dense(X, *sw)
    return out


@pytest.mark.parametrize("T,E,k,H,I,shared", [(16, 8, 2, 256, 128, 0), (12, 6, 3, 128, 256, 1), (5, 4, 4, 128, 128, 1)])
def test_layer_vs_dense_brute_force(orc, T, E, k, H, I, shared):
    rng = np.random.default_rng(T * E + H)
    w1, w3, w2, sw = _rand_layer(rng, E, H, I, shared)
    x = torch.from_numpy(rng.standard_normal((T, H))).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = orc.route(logits, k)
    L = orc.Layer(w1, w3, w2, *sw)
    out = orc.layer_rows(L, x, ids, w, np.arange(T))
    ref = _dense_layer(_f(x), ids, w, w1, w3, w2, sw)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    # a subset of rows gives the same rows
    sub = np.array([T - 1, 0, T // 2])
    np.testing.assert_array_equal(orc.layer_rows(L, x, ids, w, sub), out[sub])


def test_tiny_workload_vs_dense(orc):
    wl = workloads.WORKLOADS["tiny"]
    d = workloads.make_inputs(wl)
    bits = {k: workloads.bits(v) for k, v in d.items() if v is not None}
    ids, w = orc.route(bits["logits"], wl.k)
    L = orc.Layer(bits["w1"], bits["w3"], bits["w2"])
    out = orc.layer_rows(L, bits["x"], ids, w, np.arange(wl.T))
    ref = _dense_layer(_f(bits["x"]), ids, w, bits["w1"], bits["w3"], bits["w2"], (None, None, None))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_identical_experts_give_single_ffn(orc):
    rng = np.random.default_rng(1)
    T, E, k, H, I = 10, 5, 3, 128, 128
    w1, w3, w2, sw = _rand_layer(rng, 1, H, I, 1)
    W1, W3, W2 = (np.repeat(a, E, axis=0) for a in (w1, w3, w2))
    x = torch.from_numpy(rng.standard_normal((T, H))).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ids, w = orc.route(rng.standard_normal((T, E)).astype(np.float32), k)
    out = orc.layer_rows(orc.Layer(W1, W3, W2, *sw), x, ids, w, np.arange(T))
    ref = _ffn_dense(_f(x), w1[0], w3[0], w2[0]) + _ffn_dense(_f(x), *sw)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_single_expert_is_textbook_swiglu(orc):
    rng = np.random.default_rng(2)
    T, H, I = 7, 256, 128
    w1, w3, w2, _ = _rand_layer(rng, 1, H, I, 0)
    x = torch.from_numpy(rng.standard_normal((T, H))).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ids, w = orc.route(rng.standard_normal((T, 1)).astype(np.float32), 1)
    assert np.all(ids == 0) and np.all(w == 1.0)
    out = orc.layer_rows(orc.Layer(w1, w3, w2), x, ids, w, np.arange(T))
    X = torch.from_numpy(_f(x))
    W1, W3, W2 = (torch.from_numpy(_f(a[0])) for a in (w1, w3, w2))
    ref = (torch.nn.functional.silu(X @ W1.T) * (X @ W3.T)) @ W2.T
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12 * ref.abs().max().item())


def test_zero_down_weights_leave_shared_only(orc):
    rng = np.random.default_rng(4)
    T, E, k, H, I = 6, 4, 2, 128, 128
    w1, w3, w2, sw = _rand_layer(rng, E, H, I, 1)
    w2[:] = 0
    x = torch.from_numpy(rng.standard_normal((T, H))).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ids, w = orc.route(rng.standard_normal((T, E)).astype(np.float32), k)
    out = orc.layer_rows(orc.Layer(w1, w3, w2, *sw), x, ids, w, np.arange(T))
    np.testing.assert_allclose(out, _ffn_dense(_f(x), *sw), rtol=1e-12, atol=0)


def test_expert_bf16_intermediate(orc):
    rng = np.random.default_rng(3)
    H, I = 256, 384
    w1, w3, w2, _ = _rand_layer(rng, 1, H, I, 0)
    x = torch.from_numpy(rng.standard_normal((1, H))).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    h, y = orc.expert_bf16(x[0], w1[0], w3[0], w2[0])
    X = _f(x)
    g, u = X @ _f(w1[0]).T, X @ _f(w3[0]).T
    np.testing.assert_allclose(h, (g * scipy_expit(g) * u)[0], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(y, _ffn_dense(X, w1[0], w3[0], w2[0])[0], rtol=1e-11, atol=1e-14)


def scipy_expit(z):
    import scipy.special
    return scipy.special.expit(z)


def test_fp8_layer_rows_match_expert_calls(orc):
    """The fp8 layer combine equals sum_j w_j * expert_fp8(...) + shared, built from per-expert calls."""
    rng = np.random.default_rng(13)
    T, E, k, H, I = 4, 3, 2, 256, 128
    w1, w3, w2, sw = _rand_layer(rng, E, H, I, 1, std=0.02)
    x = torch.from_numpy(rng.standard_normal((T, H))).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xq, xs = orc.quant_rows_fp8(x)
    q1, s1 = orc.quant_blocks_fp8(w1)
    q3, s3 = orc.quant_blocks_fp8(w3)
    q2, s2 = orc.quant_blocks_fp8(w2)
    qs = [orc.quant_blocks_fp8(a) for a in sw]
    L = orc.Layer(q1, q3, q2, qs[0][0], qs[1][0], qs[2][0], wtype=1, s1=s1, s3=s3, s2=s2,
                  ss1=qs[0][1], ss3=qs[1][1], ss2=qs[2][1])
    ids, w = orc.route(rng.standard_normal((T, E)).astype(np.float32), k)
    out = orc.layer_rows(L, xq, ids, w, np.arange(T), xs=xs)
    for t in range(T):
        ref = orc.expert_fp8(xq[t], xs[t], qs[0][0], qs[0][1], qs[1][0], qs[1][1], qs[2][0], qs[2][1])[1]
        for j in range(k):
            e = ids[t, j]
            ref = ref + w[t, j] * orc.expert_fp8(xq[t], xs[t], q1[e], s1[e], q3[e], s3[e], q2[e], s2[e])[1]
        np.testing.assert_allclose(out[t], ref, rtol=1e-12, atol=1e-15)


def test_fp8_layer_trace_is_the_requantised_h(orc):
    """The block-FP8 layer's traced h equals the single-expert oracle's fp32 h,
    and its traced codes and scales are that h quantised per 128 columns (each
    128-column group as one tensor of the pinned per-tensor quantiser)."""
    rng = np.random.default_rng(14)
    T, E, k, H, I = 5, 3, 2, 256, 256
    w1, w3, w2, sw = _rand_layer(rng, E, H, I, 1, std=0.02)
    x = torch.from_numpy(rng.standard_normal((T, H))).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xq, xs = orc.quant_rows_fp8(x)
    q1, s1 = orc.quant_blocks_fp8(w1)
    q3, s3 = orc.quant_blocks_fp8(w3)
    q2, s2 = orc.quant_blocks_fp8(w2)
    qs = [orc.quant_blocks_fp8(a) for a in sw]
    L = orc.Layer(q1, q3, q2, qs[0][0], qs[1][0], qs[2][0], wtype=1, s1=s1, s3=s3, s2=s2,
                  ss1=qs[0][1], ss3=qs[1][1], ss2=qs[2][1])
    ids, w = orc.route(rng.standard_normal((T, E)).astype(np.float32), k)
    _, tr = orc.layer_rows(L, xq, ids, w, np.arange(T), xs=xs, trace=True)
    for t in range(T):
        for j in range(k + 1):
            if j == k:
                h = orc.expert_fp8(xq[t], xs[t], qs[0][0], qs[0][1], qs[1][0], qs[1][1], qs[2][0], qs[2][1])[0]
            else:
                e = ids[t, j]
                h = orc.expert_fp8(xq[t], xs[t], q1[e], s1[e], q3[e], s3[e], q2[e], s2[e])[0]
            np.testing.assert_array_equal(tr["h"][t, j], h.astype(np.float32))
    groups = tr["h"].reshape(-1, 128)
    hq, hs = orc.quant_tensor_fp8(groups, mats=groups.shape[0])
    np.testing.assert_array_equal(tr["hq"].reshape(-1, 128), hq)
    np.testing.assert_array_equal(tr["hs"].reshape(-1), hs)
