"""GPU parity of moe_forward_persistent: route, align, Gate-Up, Down and
combine as phases of one persistent kernel with device-side ready flags.

Its phases run the five-kernel chain's arithmetic, so the output, routing ids
and routing weights must equal moe_forward's bit for bit.  The output is also
checked against the oracle on every row: route ids bit-exact and weights
within 1e-6 (when the router runs on the device: on its logits, which are
first checked against the exact logits within 1e-5 of their largest
magnitude), layer output within 1e-2 of max|ref|.  After every call the device-side
status word must report that no wait ran out of time.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import TOL, host, log

import expert_layer_amd as moe
from expert_layer_amd.chain import Layer, split_router
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

W = workloads.Workload

CASES = [
    workloads.WORKLOADS["tiny"],
    workloads.WORKLOADS["decode"],
    # ragged chunks; Gate-Up K loop of depth 2, Down of depth 4
    W("p-ragged", T=37, H=384, E=8, k=3, I=256, shared=1, seed=61),
    W("p-single-token", T=1, H=256, E=16, k=4, I=256, shared=1, seed=62),
    # a single chunk; the combine item is narrower than a wave's 512 columns
    W("p-one-expert", T=16, H=128, E=1, k=1, I=128, shared=0, seed=63),
    # 16 logits per lane in the route phase
    W("p-wide-E", T=50, H=128, E=1000, k=32, I=128, shared=1, seed=64),
    W("p-max-E", T=40, H=128, E=1024, k=32, I=128, shared=1, seed=67),
    W("p-mixed-bias", T=60, H=256, E=32, k=8, I=128, shared=1, bias="mix", bias_frac=0.3, seed=65),
    W("p-router", T=100, H=512, E=64, k=8, I=128, shared=1, router=True, bias="mix", bias_frac=0.3, seed=66),
]


def _layer(d):
    return Layer.from_weights(d["w1"], d["w3"], d["w2"], d["sw1"], d["sw3"], d["sw2"])


def _forward(fn, layer, wl, d, ydt, hi=None, lo=None, ws=None):
    if ws is None:
        nbytes = moe.moe_forward_workspace_bytes(layer.experts, wl.T, wl.k, ydt)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda")
    fn(layer.experts, d["x"], wl.k, out, ws, logits=None if wl.router else d["logits"], router_hi=hi,
       router_lo=lo, bias=d["bias"], bias_rows=d["bias_rows"], y_dtype=ydt, topk_ids=ids, topk_w=w)
    return out, ids, w, ws


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
@pytest.mark.parametrize("ydt", [moe.MOE_DTYPE_F32, moe.MOE_DTYPE_BF16], ids=["yf32", "ybf16"])
def test_persistent_matches_chain_and_oracle(wl, ydt):
    log(f"persistent {wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} S={wl.shared} y={ydt}")
    d = workloads.make_inputs(wl, device="cuda")
    layer = _layer(d)
    hi = lo = None
    if wl.router:
        hi, lo = split_router(d["router_w"])
    out_c, ids_c, w_c, _ = _forward(moe.moe_forward, layer, wl, d, ydt, hi, lo)
    out_p, ids_p, w_p, ws = _forward(moe.moe_forward_persistent, layer, wl, d, ydt, hi, lo)
    moe.moe_forward_persistent_status(ws)
    assert torch.equal(ids_p, ids_c), "routing ids differ from moe_forward"
    assert torch.equal(w_p, w_c), "routing weights differ from moe_forward"
    assert torch.equal(out_p, out_c), "output differs from moe_forward"

    ids = host(ids_p)
    wts = host(w_p)
    if wl.router:
        # the logits the chain routes on come from the router GEMM kernel it
        # launches first; the same call on the same inputs gives the same bits.
        # They are checked against the exact logits, and routing is evaluated
        # on them (a legitimate 1e-6 logit difference could flip a near-tie)
        glog = torch.empty((wl.T, wl.E), dtype=torch.float32, device="cuda")
        moe.moe_router_gemm(d["x"], hi, lo, glog)
        torch.cuda.synchronize()
        exact = orc.router_logits(host(d["x"]), host(d["router_w"]))
        lerr = np.abs(host(glog).astype(np.float64) - exact).max()
        assert lerr <= 1e-5 * np.abs(exact).max(), f"router logits err {lerr} vs {np.abs(exact).max()}"
        logits = host(glog)
    else:
        logits = host(d["logits"])
    ids_ref, w_ref = orc.route(logits, wl.k, host(d["bias"]), host(d["bias_rows"]))
    assert np.array_equal(ids, ids_ref), f"route ids differ in {np.sum(ids != ids_ref)} entries"
    assert np.abs(wts.astype(np.float64) - w_ref).max() <= 1e-6
    L = orc.Layer(host(d["w1"]), host(d["w3"]), host(d["w2"]), host(d["sw1"]), host(d["sw3"]), host(d["sw2"]))
    rows = np.arange(wl.T, dtype=np.int64)
    ref = orc.layer_rows(L, host(d["x"]), ids_ref, w_ref, rows)
    err = np.abs(out_p.float().cpu().numpy() - ref).max()
    scale = np.abs(ref).max()
    log(f"  max|err| {err:.3e}, max|ref| {scale:.3e}")
    assert err <= TOL["bf16"] * scale


def test_persistent_repeats_and_graph_replay():
    """The control words are cleared by every call: back-to-back calls on one
    workspace, and a captured graph replayed with eager calls in between, all
    give the first call's bits."""
    wl = W("p-graph", T=64, H=512, E=64, k=8, I=256, shared=1, bias="mix", bias_frac=0.3, seed=67)
    d = workloads.make_inputs(wl, device="cuda")
    layer = _layer(d)
    ydt = moe.MOE_DTYPE_F32
    want, _, _, ws = _forward(moe.moe_forward_persistent, layer, wl, d, ydt)
    moe.moe_forward_persistent_status(ws)
    ref_chain, _, _, _ = _forward(moe.moe_forward, layer, wl, d, ydt)
    assert torch.equal(want, ref_chain)
    out = torch.empty_like(want)
    kw = dict(logits=d["logits"], bias=d["bias"], bias_rows=d["bias_rows"], y_dtype=ydt)
    for i in range(3):
        out.zero_()
        moe.moe_forward_persistent(layer.experts, d["x"], wl.k, out, ws, **kw)
        moe.moe_forward_persistent_status(ws)
        assert torch.equal(out, want), f"repeat {i}"
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        moe.moe_forward_persistent(layer.experts, d["x"], wl.k, out, ws, **kw)
    stream.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_forward_persistent(layer.experts, d["x"], wl.k, out, ws, **kw)
    for i in range(3):
        out.zero_()
        graph.replay()
        moe.moe_forward_persistent_status(ws)
        assert torch.equal(out, want), f"replay {i}"
        out.zero_()
        moe.moe_forward_persistent(layer.experts, d["x"], wl.k, out, ws, **kw)    # eager between replays
        moe.moe_forward_persistent_status(ws)
        assert torch.equal(out, want), f"eager after replay {i}"


def _random_shapes(n, seed):
    """Seeded random shapes inside the persistent kernel's envelope (bf16,
    T*k <= 16*E): expert count, top-k, widths, shared expert, bias mode and
    the device router drawn at random."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 5, 16, 48, 64, 200]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 16 * E // k + 1))
        H = 128 * int(rng.integers(1, 6))
        I = 128 * int(rng.integers(1, 5))
        shared = int(rng.integers(0, 2))
        bias = str(rng.choice(["none", "all", "mix"]))
        router = bool(rng.integers(0, 4) == 0)
        out.append(W(f"prand{i}-T{T}-E{E}-k{k}-H{H}-I{I}-S{shared}-{bias}{'-router' if router else ''}", T=T,
                     H=H, E=E, k=k, I=I, shared=shared, bias=bias, bias_frac=0.3, router=router, seed=7000 + i))
    return out


RANDOM = _random_shapes(16, 2025)


@pytest.mark.parametrize("wl", RANDOM, ids=[w.name for w in RANDOM])
def test_persistent_random_shapes(wl):
    test_persistent_matches_chain_and_oracle(wl, moe.MOE_DTYPE_F32 if wl.T % 2 else moe.MOE_DTYPE_BF16)


def test_persistent_chains_on_two_streams():
    """Two persistent chains enqueued on two streams at once: the library orders
    them on the device, so both complete (status OK) with their serial bits."""
    shapes = [W("pc-a", T=64, H=1024, E=64, k=8, I=256, shared=1, seed=91),
              W("pc-b", T=48, H=512, E=32, k=4, I=384, shared=1, bias="mix", bias_frac=0.3, seed=92)]
    runs = []
    for wl in shapes:
        log(f"two-stream persistent {wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I}")
        d = workloads.make_inputs(wl, device="cuda")
        layer = _layer(d)
        want, _, _, ws = _forward(moe.moe_forward_persistent, layer, wl, d, moe.MOE_DTYPE_F32)
        moe.moe_forward_persistent_status(ws)
        runs.append((wl, layer, d, ws, torch.empty_like(want), want))
    streams = [torch.cuda.Stream() for _ in runs]
    for rep in range(3):
        for s, (wl, layer, d, ws, out, _) in zip(streams, runs):
            out.zero_()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                moe.moe_forward_persistent(layer.experts, d["x"], wl.k, out, ws, logits=d["logits"], bias=d["bias"],
                                           bias_rows=d["bias_rows"], y_dtype=moe.MOE_DTYPE_F32)
        torch.cuda.synchronize()
        for (wl, _, _, ws, out, want) in runs:
            moe.moe_forward_persistent_status(ws)
            assert torch.equal(out, want), f"{wl.name}, repeat {rep}"
