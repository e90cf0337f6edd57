"""Pins for the oracle's stage-5 combine on given expert outputs and for the
residual add + RMSNorm epilogue (CPU only).

The HPC-Ops page (technical principles, fused AllReduce+Norm) computes
RMSNorm(AllReduce(x) + residual, weight); on one GPU the all-reduce is the
identity.  Pinned against torch's rms_norm (a library routine) in float64,
a closed form for constant rows, and scale invariance.  The combine is pinned
against a dense gather-and-sum written with numpy indexing.
"""
import numpy as np
import torch


def _bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _vals(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_add_rmsnorm_matches_torch(orc):
    rng = np.random.default_rng(11)
    rows, H, eps = 7, 384, 1e-6
    x = rng.standard_normal((rows, H))
    res = _bits(rng.standard_normal((rows, H)).astype(np.float32))
    wgt = _bits((1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    s, out = orc.add_rmsnorm(x, res, wgt, eps)
    s_ref = x + _vals(res)
    np.testing.assert_array_equal(s, s_ref)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(s_ref), (H,), torch.from_numpy(_vals(wgt)), eps).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_add_rmsnorm_closed_forms(orc):
    H = 256
    wgt = _bits(np.linspace(0.5, 2.0, H).astype(np.float32))
    # constant row c (residual 0): out = weight * c / sqrt(c^2 + eps)
    for c, eps in ((3.0, 0.0), (-0.25, 1e-3)):
        x = np.full((1, H), c)
        _, out = orc.add_rmsnorm(x, np.zeros((1, H), np.uint16), wgt, eps)
        np.testing.assert_allclose(out[0], _vals(wgt) * c / np.sqrt(c * c + eps), rtol=1e-14)
    # scale invariance with eps = 0
    rng = np.random.default_rng(12)
    x = rng.standard_normal((3, H))
    _, o1 = orc.add_rmsnorm(x, np.zeros((3, H), np.uint16), wgt, 0.0)
    _, o2 = orc.add_rmsnorm(8.0 * x, np.zeros((3, H), np.uint16), wgt, 0.0)
    np.testing.assert_allclose(o1, o2, rtol=1e-14)


def test_combine_matches_gather_sum(orc):
    rng = np.random.default_rng(13)
    T, k, H, shared = 9, 3, 128, 1
    R = T * k + shared * T
    y = rng.standard_normal((R, H)).astype(np.float32)
    pair_slot = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out = orc.combine(y, pair_slot, w, T, k, shared)
    ref = (w.astype(np.float64)[:, :, None] * y.astype(np.float64)[pair_slot.reshape(T, k)]).sum(axis=1)
    ref += y[T * k:].astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-14)
