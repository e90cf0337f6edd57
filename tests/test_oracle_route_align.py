"""Pins for the oracle's route and align stages (CPU only).

Route: top-k by (value desc, id asc), weights = softmax over the k selected
logits (HPC-Ops page, main functions: FusedMoE routing index stage; the gate
function is a reading, see the oracle's header).  Align: per-expert counts and
contiguous, stable intervals (HPC-Ops page, technical principles: FusedMoE
pipeline).  Each expected value below comes from an independent formulation:
hand-derived fixtures, an O(E^2) rank count, a library softmax or a library
stable sort.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_route(logits, k, bias=None, bias_rows=None):
    """Rank of expert e = number of experts that beat it; selected iff rank < k."""
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k))
    for t in range(T):
        row = logits[t].astype(np.float32)
        if bias is not None and (bias_rows is None or bias_rows[t]):
            row = (row + bias.astype(np.float32)).astype(np.float32)
        for e in range(E):
            rank = sum(1 for f in range(E) if row[f] > row[e] or (row[f] == row[e] and f < e))
            if rank < k:
                ids[t, rank] = e
        w[t] = scipy.special.softmax(row[ids[t]].astype(np.float64))
    return ids, w


def test_route_golden(orc):
    cases = json.load(open(os.path.join(GOLDEN, "route_cases.json")))["cases"]
    for c in cases:
        logits = np.array(c["logits"], np.float32)
        bias = workloads.zipf_bias(logits.shape[1]) if c.get("bias") == "zipf" else None
        ids, w = orc.route(logits, c["k"], bias=bias)
        np.testing.assert_array_equal(ids, np.array(c["ids"]), err_msg=c["why"])
        np.testing.assert_allclose(w, np.array(c["w"]), rtol=0, atol=c.get("w_tol", 1e-15), err_msg=c["why"])


@pytest.mark.parametrize("T,E,k,integer", [(40, 8, 2, False), (30, 16, 4, True), (20, 64, 8, False),
                                           (25, 7, 7, True), (10, 5, 1, True), (12, 33, 5, True)])
def test_route_vs_rank_count(orc, T, E, k, integer):
    rng = np.random.default_rng(T * 1000 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if integer:  # many exact ties
        logits = np.round(logits * 1.5).astype(np.float32)
    ids, w = orc.route(logits, k)
    bids, bw = _brute_route(logits, k)
    np.testing.assert_array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=1e-13, atol=1e-15)
    # invariants: distinct ids, weights sum to one and follow rank order
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-13)
    assert np.all(np.diff(w, axis=1) <= 1e-15)


def test_route_bias_rows(orc):
    rng = np.random.default_rng(7)
    T, E, k = 50, 32, 8
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = workloads.zipf_bias(E)
    rows = (rng.random(T) < 0.3).astype(np.uint8)
    ids, w = orc.route(logits, k, bias=bias, bias_rows=rows)
    bids, bw = _brute_route(logits, k, bias=bias, bias_rows=rows)
    np.testing.assert_array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=1e-13)
    ids_all, _ = orc.route(logits, k, bias=bias)
    bids_all, _ = _brute_route(logits, k, bias=bias)
    np.testing.assert_array_equal(ids_all, bids_all)


def test_route_k_equals_E_is_full_softmax(orc):
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((9, 12)).astype(np.float32)
    ids, w = orc.route(logits, 12)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    for t in range(9):
        np.testing.assert_allclose(w[t], full[t, ids[t]], rtol=1e-13)
        assert sorted(ids[t].tolist()) == list(range(12))


def test_align_golden(orc):
    cases = json.load(open(os.path.join(GOLDEN, "align_cases.json")))["cases"]
    for c in cases:
        counts, offsets, sp, ps = orc.align(np.array(c["ids"], np.int32), c["E"], c["shared"])
        np.testing.assert_array_equal(counts, c["counts"], err_msg=c["why"])
        np.testing.assert_array_equal(offsets, c["offsets"], err_msg=c["why"])
        np.testing.assert_array_equal(sp, c["slot_pair"], err_msg=c["why"])
        np.testing.assert_array_equal(ps, c["pair_slot"], err_msg=c["why"])


@pytest.mark.parametrize("T,E,k,shared", [(100, 8, 2, 0), (257, 64, 8, 1), (64, 256, 8, 1), (33, 3, 3, 1)])
def test_align_vs_stable_sort(orc, T, E, k, shared):
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[: T // 3] += workloads.zipf_bias(E)  # skew part of the batch
    ids, _ = orc.route(logits, k)
    counts, offsets, sp, ps = orc.align(ids, E, shared)
    flat = ids.ravel()
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets[: E + 1], np.concatenate([[0], np.cumsum(counts)]))
    assert offsets[E + 1] == T * k + shared * T
    np.testing.assert_array_equal(sp, np.argsort(flat, kind="stable"))   # library stable sort
    np.testing.assert_array_equal(ps[sp], np.arange(T * k))              # mutually inverse
    np.testing.assert_array_equal(sp[ps], np.arange(T * k))
    for e in range(E):  # ascending token inside each interval
        toks = sp[offsets[e]:offsets[e + 1]] // k
        assert np.all(np.diff(toks) > 0)
    # each token appears in exactly k slots
    np.testing.assert_array_equal(np.bincount(sp // k, minlength=T), np.full(T, k))
