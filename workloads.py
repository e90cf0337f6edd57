"""Seeded synthetic inputs for the fused MoE layer forward.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no routing, quantisation or products).  Both the HIP path
and the oracle are fed the identical bytes it produces.

Workloads (shapes and distributions of the five layer configurations):
  tiny     T=16    H=256  E=8   k=2 I=128  no shared expert, bf16
  decode   T=64    H=4096 E=256 k=8 I=1536 + shared expert, bf16
  prefill  T=8192  H=4096 E=256 k=8 I=1536 + shared expert, bf16
  fp8      T=4096  H=6144 E=256 k=8 I=2048 + shared expert, e4m3 weights
           (128x128 block scales), Zipf-skewed routing
  mxfp8    the fp8 shape and routing with MXFP8 weights and activations
           (E8M0 scales per 32 values along K)
  fp8t     the fp8 shape and routing with per-tensor FP8 (one scale per
           expert matrix, per x, per h)
  router   T=16384 H=6144 E=256 k=8 I=2048 + shared expert, bf16, fp32 router
           weights [E,H], 30% of tokens carry the Zipf logit bias
  fp8perm  the fp8 workload with the Zipf ranks permuted (seeded), so the hot
           experts sit at scattered expert indices instead of 0, 1, 2, ...
  decode_fp8, decode_mxfp8, decode_fp8t
           the decode shape and routing with 128x128-block, MXFP8 and
           per-tensor FP8 weights
Distributions: weights bf16 ~N(0, 0.02), activations bf16 ~N(0, 1), router
logits fp32 ~N(0, 1), router weights fp32 ~N(0, 0.01).  Values are drawn in
fp32 and rounded to bf16 by torch's round-to-nearest-even conversion.  The
Zipf bias is b_e = 2 ln(1 / rank(e)) with rank(e) = e + 1, or with
rank(e) = perm[e] + 1 for a seeded permutation perm of [0, E) when the
workload sets bias_perm.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    shared: int
    wtype: str = "bf16"          # "bf16", "fp8" (128x128 scales), "mxfp8" or "fp8t" (per tensor)
    bias: str = "none"           # "none", "all" (every row biased) or "mix"
    bias_frac: float = 0.0       # fraction of biased rows for "mix"
    router: bool = False         # logits come from the split-bf16 router GEMM
    bias_perm: int = 0           # nonzero: seed of a permutation of the Zipf ranks
    seed: int = 0
    w_std: float = 0.02
    x_std: float = 1.0
    router_std: float = 0.01
    extra: dict = field(default_factory=dict)

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def R(self) -> int:
        return self.T * self.k + self.shared * self.T


WORKLOADS = {
    "tiny": Workload("tiny", T=16, H=256, E=8, k=2, I=128, shared=0, seed=1001),
    "decode": Workload("decode", T=64, H=4096, E=256, k=8, I=1536, shared=1, seed=1002),
    "prefill": Workload("prefill", T=8192, H=4096, E=256, k=8, I=1536, shared=1, seed=1003),
    "fp8": Workload("fp8", T=4096, H=6144, E=256, k=8, I=2048, shared=1, wtype="fp8",
                    bias="all", seed=1004),
    "mxfp8": Workload("mxfp8", T=4096, H=6144, E=256, k=8, I=2048, shared=1, wtype="mxfp8",
                      bias="all", seed=1006),
    "fp8t": Workload("fp8t", T=4096, H=6144, E=256, k=8, I=2048, shared=1, wtype="fp8t",
                     bias="all", seed=1007),
    "router": Workload("router", T=16384, H=6144, E=256, k=8, I=2048, shared=1, bias="mix",
                       bias_frac=0.3, router=True, seed=1005),
    "fp8perm": Workload("fp8perm", T=4096, H=6144, E=256, k=8, I=2048, shared=1, wtype="fp8",
                        bias="all", bias_perm=77, seed=1004),
    "decode_fp8": Workload("decode_fp8", T=64, H=4096, E=256, k=8, I=1536, shared=1, wtype="fp8", seed=1002),
    "decode_mxfp8": Workload("decode_mxfp8", T=64, H=4096, E=256, k=8, I=1536, shared=1, wtype="mxfp8",
                             seed=1002),
    "decode_fp8t": Workload("decode_fp8t", T=64, H=4096, E=256, k=8, I=1536, shared=1, wtype="fp8t",
                            seed=1002),
}


def workload(name: str, **overrides) -> Workload:
    return replace(WORKLOADS[name], **overrides)


def zipf_bias(E: int, perm_seed: int = 0) -> np.ndarray:
    """b_e = 2 ln(1/rank(e)) as fp32: rank(e) = e + 1 (expert 0 is the hottest),
    or perm[e] + 1 for a permutation of [0, E) drawn from perm_seed."""
    rank = np.arange(E) + 1
    if perm_seed:
        rank = np.random.default_rng(perm_seed).permutation(E) + 1
    return np.array([2.0 * math.log(1.0 / int(r)) for r in rank], dtype=np.float32)


def _normal(shape, std, gen, device, dtype):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_inputs(wl: Workload, device="cpu", seed: int | None = None, weights: bool = True):
    """Draw every input of one layer call.  Returns a dict of torch tensors on ``device``.

    keys: x [T,H] bf16; logits [T,E] fp32 (absent when wl.router); router_w [E,H]
    fp32 (wl.router only); bias [E] fp32 or None; bias_rows [T] uint8 or None;
    w1, w3 [E,I,H] bf16; w2 [E,H,I] bf16; sw1, sw3 [I,H], sw2 [H,I] bf16 (shared).
    """
    seed = wl.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    T, H, E, I = wl.T, wl.H, wl.E, wl.I
    d = {}
    d["x"] = _normal((T, H), wl.x_std, gen, device, torch.bfloat16)
    if wl.router:
        d["router_w"] = _normal((E, H), wl.router_std, gen, device, torch.float32)
    else:
        d["logits"] = _normal((T, E), 1.0, gen, device, torch.float32)
    d["bias"] = None
    d["bias_rows"] = None
    if wl.bias in ("all", "mix"):
        d["bias"] = torch.from_numpy(zipf_bias(E, wl.bias_perm)).to(device)
    if wl.bias == "mix":
        cpu_gen = torch.Generator()
        cpu_gen.manual_seed(seed + 1)
        perm = torch.randperm(T, generator=cpu_gen)
        rows = torch.zeros(T, dtype=torch.uint8)
        rows[perm[: int(math.floor(wl.bias_frac * T))]] = 1
        d["bias_rows"] = rows.to(device)
    if weights:
        w1 = torch.empty((E, I, H), dtype=torch.bfloat16, device=device)
        w3 = torch.empty((E, I, H), dtype=torch.bfloat16, device=device)
        w2 = torch.empty((E, H, I), dtype=torch.bfloat16, device=device)
        for e in range(E):
            w1[e] = _normal((I, H), wl.w_std, gen, device, torch.bfloat16)
            w3[e] = _normal((I, H), wl.w_std, gen, device, torch.bfloat16)
            w2[e] = _normal((H, I), wl.w_std, gen, device, torch.bfloat16)
        d["w1"], d["w3"], d["w2"] = w1, w3, w2
        if wl.shared:
            d["sw1"] = _normal((I, H), wl.w_std, gen, device, torch.bfloat16)
            d["sw3"] = _normal((I, H), wl.w_std, gen, device, torch.bfloat16)
            d["sw2"] = _normal((H, I), wl.w_std, gen, device, torch.bfloat16)
        else:
            d["sw1"] = d["sw3"] = d["sw2"] = None
    return d


def bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor's raw bits (bf16 -> uint16, fp8 -> uint8)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def sample_rows(T: int, n: int, seed: int) -> np.ndarray:
    """Seeded uniform sample of n distinct token indices (sorted)."""
    rng = np.random.default_rng(seed)
    n = min(n, T)
    return np.sort(rng.choice(T, size=n, replace=False)).astype(np.int64)
