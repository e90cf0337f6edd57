"""GPU parity: the HIP chain (through the C ABI) against the oracle.

Stage-by-stage on every configuration: route ids and align permutations
bit-exact, fp8 codes/scales bit-exact, routing weights within 1e-6, layer
output within 1e-2 (bf16) / 5e-2 (fp8) of max|ref|.  Small and medium shapes
check every row; the full-size layer shapes check a seeded 256-token sample
plus the first token of every touched expert.
"""
import gc

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import check_layer, log, run_gpu

from expert_layer_amd.chain import run_chain

pytestmark = pytest.mark.gpu

W = workloads.Workload


def _inputs(wl, **mut):
    d = workloads.make_inputs(wl, device="cuda")
    return d


def _free():
    gc.collect()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- small / medium (all rows)
SMALL = [
    W("tiny", T=16, H=256, E=8, k=2, I=128, shared=0, seed=1001),
    W("ragged", T=37, H=384, E=8, k=3, I=256, shared=1, seed=11),
    W("medium", T=300, H=512, E=16, k=4, I=256, shared=1, seed=12),
    W("multiblock-align", T=1500, H=256, E=64, k=8, I=128, shared=1, seed=13),
    W("k-equals-E", T=40, H=256, E=8, k=8, I=128, shared=1, seed=14),
    W("single-expert", T=33, H=128, E=1, k=1, I=128, shared=0, seed=15),
    W("single-token", T=1, H=256, E=16, k=4, I=256, shared=1, seed=16),
    W("wide-E", T=50, H=128, E=1000, k=32, I=128, shared=1, seed=17),
    # the largest expert count and top-k the ABI accepts
    W("max-E", T=40, H=128, E=1024, k=32, I=128, shared=1, seed=44),
    W("zipf-bias", T=200, H=256, E=32, k=8, I=128, shared=1, bias="all", seed=18),
    W("mixed-bias", T=200, H=256, E=32, k=8, I=128, shared=1, bias="mix", bias_frac=0.3, seed=19),
    W("router-small", T=100, H=512, E=64, k=8, I=128, shared=1, router=True, bias="mix", bias_frac=0.3, seed=20),
    # router tiles of 128 tokens x 128 experts: ragged in both, two expert tiles
    W("router-ragged", T=300, H=384, E=200, k=8, I=128, shared=1, router=True, bias="mix", bias_frac=0.3, seed=21),
    # 224 to 288 rows per expert on average: 288-row tiles, with remainders
    # where the Zipf-biased experts overflow them
    W("tall-tiles", T=500, H=256, E=16, k=8, I=128, shared=1, bias="mix", bias_frac=0.3, seed=38),
    # Zipf ranks permuted: the hot experts sit at scattered indices, some late in the item order
    W("zipf-perm", T=500, H=256, E=32, k=8, I=128, shared=1, bias="all", bias_perm=5, seed=39),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16], ids=["yf32", "ybf16"])
def test_small_bf16(wl, ydt):
    check_layer(wl, _inputs(wl), y_dtype=ydt)


FP8_SMALL = [
    W("fp8-medium", T=300, H=512, E=16, k=4, I=256, shared=1, wtype="fp8", seed=21),
    W("fp8-ragged", T=37, H=384, E=8, k=3, I=384, shared=0, wtype="fp8", seed=22),
    W("fp8-zipf", T=400, H=256, E=32, k=8, I=256, shared=1, wtype="fp8", bias="all", seed=23),
    W("fp8-zipf-perm", T=500, H=256, E=32, k=8, I=256, shared=1, wtype="fp8", bias="all", bias_perm=6, seed=28),
    # weight-streaming kernels (up to 16 rows per expert on average) at each
    # K-blocks-in-flight depth: Gate-Up KB 8 / 5, Down KB 6 / 4
    W("fp8-stream", T=33, H=1024, E=40, k=6, I=768, shared=1, wtype="fp8", bias="mix", bias_frac=0.3, seed=47),
    W("fp8-stream2", T=20, H=640, E=24, k=4, I=512, shared=1, wtype="fp8", seed=49),
]


@pytest.mark.parametrize("wl", FP8_SMALL, ids=[w.name for w in FP8_SMALL])
def test_small_fp8(wl):
    check_layer(wl, _inputs(wl), y_dtype=torch.float32)


MX_SMALL = [
    W("mx-medium", T=300, H=512, E=16, k=4, I=256, shared=1, wtype="mxfp8", seed=24),
    W("mx-ragged", T=37, H=256, E=8, k=3, I=384, shared=0, wtype="mxfp8", seed=25),
    W("mx-zipf", T=400, H=256, E=32, k=8, I=256, shared=1, wtype="mxfp8", bias="all", seed=26),
    W("mx-tiny-groups", T=16, H=512, E=64, k=8, I=256, shared=1, wtype="mxfp8", seed=27),
    # weight-streaming kernels (up to 16 rows per expert on average), ragged K and chunks
    W("mx-stream", T=33, H=768, E=40, k=6, I=384, shared=1, wtype="mxfp8", bias="mix", bias_frac=0.3, seed=29),
    # streaming kernels with the scale rows staged in LDS (K % 512 == 0): one
    # partly used group of 16 K blocks, and a second, partly used group
    W("mx-stream-staged", T=40, H=1536, E=48, k=6, I=1536, shared=1, wtype="mxfp8", seed=45),
    W("mx-stream-staged2", T=24, H=2560, E=32, k=4, I=2048, shared=1, wtype="mxfp8", bias="all", seed=46),
]


@pytest.mark.parametrize("wl", MX_SMALL, ids=[w.name for w in MX_SMALL])
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16], ids=["yf32", "ybf16"])
def test_small_mxfp8(wl, ydt):
    check_layer(wl, _inputs(wl), y_dtype=ydt)


def test_mxfp8_quantiser_exhaustive_over_bf16():
    """Every finite bf16 value through the GPU MXFP8 quantiser, as given and
    scaled to hit saturation, ties and the clamped exponent range: codes and
    scale bytes equal the oracle's bit for bit."""
    import expert_layer_amd as moe
    from oracle import oracle as orc
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    expo = (allbits >> 7) & 0xFF
    finite = allbits[expo != 0xFF]
    n = finite.size - finite.size % 256
    rng = np.random.default_rng(9)
    rows = rng.permutation(finite[:n]).reshape(-1, 256)
    # plus a row of bf16 subnormals (clamped exponent) and an all-zero row
    rows = np.concatenate([rows, np.arange(1, 257, dtype=np.uint16)[None], np.zeros((1, 256), np.uint16)])
    vals = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).float().numpy()
    with np.errstate(over="ignore"):
        scaled = vals * np.ldexp(1.0, rng.integers(-40, 40, size=(vals.shape[0], 1))).astype(np.float32)
    scaled = np.where(np.abs(scaled) < 3.0e38, scaled, 0.0).astype(np.float32)   # finite inputs only
    scaled_bits = torch.from_numpy(scaled).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for data in (rows, scaled_bits):
        xg = torch.from_numpy(data.view(np.int16)).view(torch.bfloat16).cuda()
        q = torch.empty(data.shape, dtype=torch.uint8, device="cuda")
        s = torch.empty((data.shape[0], data.shape[1] // 32), dtype=torch.uint8, device="cuda")
        moe.moe_quant_rows_mxfp8(xg, q, s)
        torch.cuda.synchronize()
        rq, rs = orc.quant_rows_mx(data)
        assert np.array_equal(s.cpu().numpy(), rs), "scale bytes differ"
        bad = np.sum(q.cpu().numpy() != rq)
        assert bad == 0, f"{bad} codes differ"


PT_SMALL = [
    W("pt-medium", T=300, H=512, E=16, k=4, I=256, shared=1, wtype="fp8t", seed=34),
    W("pt-ragged", T=37, H=256, E=8, k=3, I=384, shared=0, wtype="fp8t", seed=35),
    W("pt-zipf", T=400, H=256, E=32, k=8, I=256, shared=1, wtype="fp8t", bias="all", seed=36),
    W("pt-tiny-groups", T=16, H=512, E=64, k=8, I=256, shared=1, wtype="fp8t", seed=37),
    W("pt-stream", T=33, H=768, E=40, k=6, I=384, shared=1, wtype="fp8t", bias="mix", bias_frac=0.3, seed=48),
]


@pytest.mark.parametrize("wl", PT_SMALL, ids=[w.name for w in PT_SMALL])
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16], ids=["yf32", "ybf16"])
def test_small_fp8_per_tensor(wl, ydt):
    check_layer(wl, _inputs(wl), y_dtype=ydt)


def test_per_tensor_quantiser_over_bf16_and_f32():
    """Every finite bf16 value through the GPU per-tensor amax + quantiser, as
    256-value tensors (one scale each) as given and scaled across the exponent
    range, and the same for fp32 tensors: amax, scales and codes equal the
    oracle's bit for bit."""
    import expert_layer_amd as moe
    from oracle import oracle as orc
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    expo = (allbits >> 7) & 0xFF
    finite = allbits[expo != 0xFF]
    n = finite.size - finite.size % 256
    rng = np.random.default_rng(10)
    rows = rng.permutation(finite[:n]).reshape(-1, 256)
    rows = np.concatenate([rows, np.arange(1, 257, dtype=np.uint16)[None], np.zeros((1, 256), np.uint16)])
    vals = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).float().numpy()
    with np.errstate(over="ignore"):
        scaled = vals * np.ldexp(1.0, rng.integers(-40, 40, size=(vals.shape[0], 1))).astype(np.float32)
    scaled = np.where(np.abs(scaled) < 3.0e38, scaled, 0.0).astype(np.float32)
    scaled_bits = torch.from_numpy(scaled).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    keep = np.abs(scaled) < 1e30
    small = np.where(keep, scaled, 0.0).astype(np.float32)     # so the product cannot overflow
    f32 = np.where(keep, small * rng.standard_normal(scaled.shape).astype(np.float32), 0.0).astype(np.float32)
    for data in (rows, scaled_bits, f32):
        mats = data.shape[0]
        if data.dtype == np.float32:
            xg = torch.from_numpy(data).cuda()
            amax_ref = np.abs(data).max(axis=1)
        else:
            xg = torch.from_numpy(data.view(np.int16)).view(torch.bfloat16).cuda()
            amax_ref = np.abs((data.astype(np.uint32) << 16).view(np.float32)).max(axis=1)
        amax = torch.empty(mats, dtype=torch.float32, device="cuda")
        q = torch.empty(data.shape, dtype=torch.uint8, device="cuda")
        s = torch.empty(mats, dtype=torch.float32, device="cuda")
        moe.moe_tensor_amax(xg, amax, mats=mats)
        moe.moe_quant_tensor_fp8(xg, amax, q, s, mats=mats)
        torch.cuda.synchronize()
        assert np.array_equal(amax.cpu().numpy(), amax_ref.astype(np.float32)), "amax differs"
        rq, rs = orc.quant_tensor_fp8(data, mats=mats)
        assert np.array_equal(s.cpu().numpy(), rs), "scales differ"
        bad = np.sum(q.cpu().numpy() != rq)
        assert bad == 0, f"{bad} codes differ"


def test_forced_ties_and_one_hot():
    """Integer logits (many exact ties) and a batch where every token picks expert 5 first."""
    wl = W("ties", T=128, H=256, E=16, k=4, I=128, shared=1, seed=30)
    d = _inputs(wl)
    d["logits"] = torch.round(d["logits"] * 1.5)
    check_layer(wl, d)
    wl2 = W("one-hot", T=200, H=256, E=8, k=1, I=128, shared=0, seed=31)
    d2 = _inputs(wl2)
    d2["logits"][:, 5] += 100.0
    _, b = check_layer(wl2, d2)
    counts = b.counts.cpu().numpy()
    assert counts[5] == 200 and counts.sum() == 200


def test_empty_experts_and_all_equal_logits():
    wl = W("all-equal", T=64, H=256, E=32, k=4, I=128, shared=1, seed=32)
    d = _inputs(wl)
    d["logits"].zero_()
    _, b = check_layer(wl, d)
    ids = b.ids.cpu().numpy()
    assert np.all(ids == np.arange(4)[None, :])
    assert np.allclose(b.w.cpu().numpy(), 0.25)
    counts = b.counts.cpu().numpy()
    assert np.all(counts[4:] == 0) and np.all(counts[:4] == 64)


def test_determinism_and_forward_entry_point():
    """Two runs give identical bits; moe_forward gives the same bits as the stages."""
    import expert_layer_amd as moe
    wl = W("det", T=500, H=512, E=32, k=8, I=256, shared=1, bias="mix", bias_frac=0.3, seed=33)
    d = _inputs(wl)
    _, b1, _ = run_gpu(wl, d)
    _, b2, _ = run_gpu(wl, d)
    for name in ("ids", "w", "counts", "offsets", "slot_pair", "pair_slot", "h", "y", "out"):
        assert torch.equal(getattr(b1, name), getattr(b2, name)), name
    # the same buffers again: the Gate-Up workspace still holds the previous
    # call's round counters, which the call must clear before use
    layer, b3, _ = run_gpu(wl, d)
    first = b3.out.clone()
    run_chain(layer, b3, d["x"], wl.k, logits=d["logits"], bias=d["bias"], bias_rows=d["bias_rows"])
    torch.cuda.synchronize()
    assert torch.equal(b3.out, first)
    assert torch.equal(first, b1.out)
    ws = torch.empty(moe.moe_forward_workspace_bytes(layer.experts, wl.T, wl.k), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda")
    moe.moe_forward(layer.experts, d["x"], wl.k, out, ws, logits=d["logits"], bias=d["bias"],
                    bias_rows=d["bias_rows"], topk_ids=ids)
    torch.cuda.synchronize()
    assert torch.equal(out, b1.out)
    assert torch.equal(ids, b1.ids)


def test_zero_tokens_is_a_no_op():
    import expert_layer_amd as moe
    logits = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    moe.moe_route(logits, 2, ids, w)
    torch.cuda.synchronize()


def test_fp8_codec_exhaustive_over_bf16():
    """Every finite bf16 value through the GPU row quantiser: groups whose amax
    is 448 have scale 1, so the codes are the conversion of the values
    themselves; other groups exercise fp32 quotients."""
    import expert_layer_amd as moe
    from oracle import oracle as orc
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (allv.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    v = allv[keep]
    v = np.concatenate([v, np.zeros((-v.size) % 127, np.uint16)])
    groups = v.reshape(-1, 127)
    anchor = np.full((groups.shape[0], 1), 0x43E0, np.uint16)      # bf16 448.0
    rows = np.concatenate([groups, anchor], axis=1).reshape(-1, 128 * 4) if groups.shape[0] % 4 == 0 else None
    if rows is None:
        pad = (-groups.shape[0]) % 4
        groups = np.concatenate([groups, np.zeros((pad, 127), np.uint16)])
        anchor = np.full((groups.shape[0], 1), 0x43E0, np.uint16)
        rows = np.concatenate([groups, anchor], axis=1).reshape(-1, 128 * 4)
    rng = np.random.default_rng(40)
    scaled = (rows.view(np.uint16).astype(np.uint32) << 16).view(np.float32) * rng.choice(
        np.array([1.0, 3.0, 0.37, 1e-3], np.float32), size=(rows.shape[0], 1))
    scaled_bits = torch.from_numpy(scaled.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for data in (rows, scaled_bits):
        xg = torch.from_numpy(data.view(np.int16)).view(torch.bfloat16).cuda()
        q = torch.empty(data.shape, dtype=torch.uint8, device="cuda")
        s = torch.empty((data.shape[0], data.shape[1] // 128), dtype=torch.float32, device="cuda")
        moe.moe_quant_rows_fp8(xg, q, s)
        torch.cuda.synchronize()
        rq, rs = orc.quant_rows_fp8(data)
        assert np.array_equal(s.cpu().numpy(), rs)
        bad = np.sum(q.cpu().numpy() != rq)
        assert bad == 0, f"{bad} codes differ"


# ---------------------------------------------------------------- the five layer configurations
@pytest.mark.parametrize("name,ydt", [("tiny", torch.float32), ("decode", torch.float32),
                                      ("prefill", torch.bfloat16), ("fp8", torch.float32),
                                      ("mxfp8", torch.float32), ("fp8t", torch.float32),
                                      ("router", torch.bfloat16), ("decode_fp8", torch.float32),
                                      ("decode_mxfp8", torch.float32), ("decode_fp8t", torch.bfloat16)])
def test_layer_configs(name, ydt):
    wl = workloads.WORKLOADS[name]
    d = _inputs(wl)
    check_layer(wl, d, y_dtype=ydt)
    del d
    _free()


def test_rows_past_32bit_element_offsets():
    """x with more than 2^31 elements (600000 tokens of H = 4096).  The tiled
    kernels address gathered rows with 32-bit element offsets, so such shapes
    take the weight-streaming kernels, which address in 64 bits.  Checked on
    a sample that includes the last tokens, whose x rows start past element
    2^31."""
    wl = W("huge-x", T=600000, H=4096, E=8, k=1, I=128, shared=0, seed=43)
    assert wl.T * wl.H > 2 ** 31
    d = _inputs(wl)
    edge = [0, (1 << 31) // wl.H - 1, (1 << 31) // wl.H, (1 << 31) // wl.H + 1, wl.T - 2, wl.T - 1]
    rows = np.unique(np.concatenate([workloads.sample_rows(wl.T, 64, wl.seed), edge])).astype(np.int64)
    check_layer(wl, d, y_dtype=torch.bfloat16, check_rows=rows)
    del d
    _free()


GRAPH_SHAPES = {
    "streaming": W("graph-s", T=64, H=512, E=64, k=8, I=256, shared=1, seed=41),
    "tiled": W("graph-t", T=500, H=512, E=32, k=8, I=256, shared=1, bias="mix", bias_frac=0.3, seed=42),
    # the fp8 chains add the quantisation passes and their cleared counters
    "fp8": W("graph-f8", T=500, H=512, E=32, k=8, I=256, shared=1, wtype="fp8", bias="mix", bias_frac=0.3, seed=45),
    "mxfp8": W("graph-mx", T=500, H=512, E=32, k=8, I=256, shared=1, wtype="mxfp8", seed=46),
    "fp8t": W("graph-pt", T=500, H=512, E=32, k=8, I=256, shared=1, wtype="fp8t", seed=47),
    # the weight-streaming FP8 kernels (decode-sized groups; MX with its scale rows staged in LDS)
    "fp8-stream": W("graph-f8s", T=64, H=1024, E=64, k=8, I=512, shared=1, wtype="fp8", seed=50),
    "mxfp8-stream": W("graph-mxs", T=64, H=1024, E=64, k=8, I=512, shared=1, wtype="mxfp8", seed=51),
    "fp8t-stream": W("graph-pts", T=64, H=1024, E=64, k=8, I=512, shared=1, wtype="fp8t", seed=52),
}


def _random_shapes(n, seed):
    """Seeded random layer shapes across weight types, sizes, top-k, shared
    expert and bias mode (every row checked when T <= 512)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        wtype = ["bf16", "fp8", "mxfp8", "fp8t"][i % 4]
        E = int(rng.choice([1, 3, 8, 16, 40, 64]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 7, 64, 200, 513]))
        step = 256 if wtype in ("mxfp8", "fp8t") else 128
        H = step * int(rng.integers(1, 5))
        I = 128 * int(rng.integers(1, 4))
        shared = int(rng.integers(0, 2))
        bias = str(rng.choice(["none", "all", "mix"]))
        out.append(W(f"rand{i}-{wtype}-T{T}-E{E}-k{k}-H{H}-I{I}-S{shared}-{bias}", T=T, H=H, E=E, k=k, I=I,
                     shared=shared, wtype=wtype, bias=bias, bias_frac=0.3, seed=5000 + i))
    return out


RANDOM = _random_shapes(48, 2024)


@pytest.mark.parametrize("wl", RANDOM, ids=[w.name for w in RANDOM])
def test_random_shapes(wl):
    check_layer(wl, _inputs(wl), y_dtype=torch.float32 if wl.T < 200 else torch.bfloat16)


@pytest.mark.parametrize("shape", list(GRAPH_SHAPES))
def test_graph_replay_matches_eager(shape):
    """The chain captured as a HIP graph: every replay, with eager launches and
    synchronisations between replays, gives the eager result bit for bit."""
    wl = GRAPH_SHAPES[shape]
    d = _inputs(wl)
    layer, b, _ = run_gpu(wl, d)
    want = b.out.clone()
    kw = dict(logits=d["logits"], bias=d["bias"], bias_rows=d["bias_rows"])
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        run_chain(layer, b, d["x"], wl.k, **kw)
    stream.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_chain(layer, b, d["x"], wl.k, **kw)
    for i in range(3):
        b.out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(b.out, want), f"replay {i}"
        run_chain(layer, b, d["x"], wl.k, **kw)     # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(b.out, want), f"eager after replay {i}"


def test_concurrent_streams_match_serial():
    """The library keeps no state between calls: two layers (tiled kernels with
    the per-XCD round barrier, whose counters live in the workspace, and
    weight-streaming kernels) run at the same time on two streams, each with
    its own workspace, and give their serial outputs bit for bit."""
    import expert_layer_amd as moe
    from expert_layer_amd.chain import Layer
    shapes = [W("cc-tiled", T=4096, H=512, E=8, k=4, I=256, shared=1, bias="mix", bias_frac=0.3, seed=81),
              W("cc-stream", T=64, H=1024, E=64, k=8, I=256, shared=1, seed=82),
              # streaming MX (scale rows staged in LDS) and per-tensor FP8 (its h amax word in the workspace)
              W("cc-mx-stream", T=64, H=1024, E=64, k=8, I=512, shared=1, wtype="mxfp8", seed=83),
              W("cc-pt-stream", T=64, H=1024, E=64, k=8, I=512, shared=1, wtype="fp8t", seed=84)]
    runs = []
    for wl in shapes:
        log(f"concurrent {wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} {wl.wtype}")
        d = _inputs(wl)
        layer = Layer.from_weights(d["w1"], d["w3"], d["w2"], d["sw1"], d["sw3"], d["sw2"], fp8=wl.wtype == "fp8",
                                   mx=wl.wtype == "mxfp8", pt=wl.wtype == "fp8t")
        ydt = moe.MOE_DTYPE_F32
        ws = torch.empty(moe.moe_forward_workspace_bytes(layer.experts, wl.T, wl.k, ydt), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
        kw = dict(logits=d["logits"], bias=d["bias"], bias_rows=d["bias_rows"], y_dtype=ydt,
                  topk_ids=torch.empty((wl.T, wl.k), dtype=torch.int32, device="cuda"),
                  topk_w=torch.empty((wl.T, wl.k), dtype=torch.float32, device="cuda"))
        runs.append((wl, layer, d["x"], ws, out, kw))
    want = []
    for wl, layer, x, ws, out, kw in runs:
        moe.moe_forward(layer.experts, x, wl.k, out, ws, **kw)
        torch.cuda.synchronize()
        want.append(out.clone())
    streams = [torch.cuda.Stream() for _ in runs]
    for rep in range(3):
        for run in runs:
            run[4].zero_()
        for s, (wl, layer, x, ws, out, kw) in zip(streams, runs):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                moe.moe_forward(layer.experts, x, wl.k, out, ws, **kw)
        torch.cuda.synchronize()
        for (wl, _, _, _, out, _), ref in zip(runs, want):
            assert torch.equal(out, ref), f"{wl.name}, repeat {rep}"


@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16], ids=["yf32", "ybf16"])
def test_combine_rmsnorm_stage(ydt):
    """combine + residual + RMSNorm on the GPU's own y against the oracle's
    combine and add+RMSNorm in double; in place equals out of place bit for bit."""
    import expert_layer_amd as moe
    from oracle import oracle as orc
    wl = W("norm", T=300, H=512, E=16, k=4, I=256, shared=1, seed=51)
    d = _inputs(wl)
    _, b, _ = run_gpu(wl, d, y_dtype=ydt)
    g = torch.Generator(device="cuda").manual_seed(52)
    residual = torch.randn((wl.T, wl.H), generator=g, device="cuda").to(torch.bfloat16)
    weight = (1.0 + 0.1 * torch.randn(wl.H, generator=g, device="cuda")).to(torch.bfloat16)
    eps = 1e-6
    out = torch.empty_like(residual)
    res_out = torch.empty_like(residual)
    moe.moe_combine_rmsnorm(b.y, b.pair_slot, b.w, wl.T, wl.k, wl.shared, residual, weight, eps, out, res_out)
    res_in_place = residual.clone()
    out2 = torch.empty_like(residual)
    moe.moe_combine_rmsnorm(b.y, b.pair_slot, b.w, wl.T, wl.k, wl.shared, res_in_place, weight, eps, out2,
                            res_in_place)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(res_out, res_in_place)
    x = orc.combine(b.y.float().cpu().numpy(), b.pair_slot.cpu().numpy(), b.w.cpu().numpy(), wl.T, wl.k, wl.shared)
    s_ref, out_ref = orc.add_rmsnorm(x, workloads.bits(residual), workloads.bits(weight), eps)
    got_s = res_out.double().cpu().numpy()
    got = out.double().cpu().numpy()
    # bf16 rounding of the stored value (<= 2^-9 relative) plus fp32 vs double arithmetic
    assert np.all(np.abs(got_s - s_ref) <= 2.0 ** -8 * np.abs(s_ref) + 1e-6 * np.abs(s_ref).max())
    assert np.all(np.abs(got - out_ref) <= 2.0 ** -8 * np.abs(out_ref) + 1e-6 * np.abs(out_ref).max())
    log(f"  combine+rmsnorm: max|out-ref| {np.abs(got - out_ref).max():.3e}, max|ref| {np.abs(out_ref).max():.3e}")


@pytest.mark.parametrize("T,H,E", [(1100, 256, 200), (1, 128, 1000), (2049, 384, 64), (8 * 128 + 1, 128, 129)],
                         ids=["T1100-E200", "T1-E1000", "T2049-E64", "T1025-E129"])
def test_router_gemm_tile_map(T, H, E):
    """Split-BF16 router GEMM on its own, at token-tile counts past one per XCD
    and expert-tile counts 1..8: every logit written once (the buffer starts as
    NaN), split bits equal to the oracle's, logits within 1e-5 max|ref| of fp64."""
    import expert_layer_amd as moe
    from oracle import oracle as orc
    g = torch.Generator(device="cuda").manual_seed(T * 7 + E)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    w = 0.01 * torch.randn((E, H), generator=g, device="cuda")
    hi = torch.empty((E, H), dtype=torch.bfloat16, device="cuda")
    lo = torch.empty_like(hi)
    logits = torch.full((T, E), float("nan"), device="cuda")
    moe.moe_router_split(w, hi, lo)
    moe.moe_router_gemm(x, hi, lo, logits)
    torch.cuda.synchronize()
    rhi, rlo = orc.router_split(w.cpu().numpy())
    assert np.array_equal(workloads.bits(hi), rhi) and np.array_equal(workloads.bits(lo), rlo)
    got = logits.double().cpu().numpy()
    assert not np.isnan(got).any(), "logits left unwritten"
    ref = orc.router_logits(workloads.bits(x), w.cpu().numpy())
    err = np.abs(got - ref).max()
    log(f"  router T={T} H={H} E={E}: max|d| {err:.3e}, max|ref| {np.abs(ref).max():.3e}")
    assert err <= 1e-5 * np.abs(ref).max()
