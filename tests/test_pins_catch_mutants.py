"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant below is the oracle source with one planted mistake: a copy of
``oracle/moe_oracle.cpp`` with one fragment replaced, compiled with the
oracle's own flags into a temporary directory.  The oracle pin suite
(``tests/test_oracle_*.py``) then runs against that build, selected through
``MOE355_ORACLE_LIB``, and must fail.  A mutant it passes would be a mistake
the pins cannot see.  The oracle itself is never modified.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.cpp")
PINS = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))

# (name, fragment of the oracle source, the mistake put in its place)
MUTANTS = [
    # route: ranks and weights
    ("tie-to-higher-id", "return a.second < b.second;", "return a.second > b.second;"),
    ("softmax-over-all-E", "for (int j = 0; j < k; ++j) denom +=", "for (int j = 0; j < E; ++j) denom +="),
    ("weights-unnormalised", "- top) / denom;", "- top);"),
    ("bias-subtracted", "if (biased) l = l + bias[e];", "if (biased) l = l - bias[e];"),
    ("bias-rows-inverted", "bias_rows[t] != 0", "bias_rows[t] == 0"),
    # align
    ("slot-holds-token", "slot_pair[s] = static_cast<int32_t>(p);", "slot_pair[s] = static_cast<int32_t>(p / k);"),
    ("shared-group-dropped", "offsets[E] + (shared ? static_cast<int32_t>(T) : 0)", "offsets[E]"),
    # codecs
    ("e4m3-ties-away", "std::nearbyint(a / quantum)", "std::round(a / quantum)"),
    ("e4m3-saturates-at-240", "if (a >= 448.0) return sign | 0x7E;", "if (a >= 240.0) return sign | 0x77;"),
    ("e4m3-subnormal-step", "quantum = std::ldexp(1.0, -9);", "quantum = std::ldexp(1.0, -10);"),
    ("bf16-ties-down", "return (down & 1u) ? up : down;", "return down;"),
    ("mx-exponent-off-by-one", "e - 1 - 8", "e - 1 - 7"),
    # router split
    ("split-factor-128", "lo[i] = bf16_nearest(resid * 256.0f);", "lo[i] = bf16_nearest(resid * 128.0f);"),
    # quantisers
    ("row-scale-240", "      float sc = amax > 0.0f ? amax / 448.0f : 1.0f;\n      s[r * groups + g] = sc;",
     "      float sc = amax > 0.0f ? amax / 240.0f : 1.0f;\n      s[r * groups + g] = sc;"),
    ("block-scale-240", "    float sc = amax > 0.0f ? amax / 448.0f : 1.0f;\n    s[b] = sc;",
     "    float sc = amax > 0.0f ? amax / 240.0f : 1.0f;\n    s[b] = sc;"),
    ("tensor-scale-240", "    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;\n    s[m] = sc;",
     "    const float sc = amax > 0.0f ? amax / 240.0f : 1.0f;\n    s[m] = sc;"),
    # expert arithmetic
    ("silu-sign", "return z / (1.0 + std::exp(-z));", "return z / (1.0 + std::exp(z));"),
    ("expert-up-reads-gate", "u += xv[i] * bf16_value(w3[(int64_t)n * H + i]);",
     "u += xv[i] * bf16_value(w1[(int64_t)n * H + i]);"),
    ("layer-up-reads-gate", "uv += xi * bf16_value(w3[i]);", "uv += xi * bf16_value(w1[i]);"),
    ("block-scale-index", "acc += static_cast<double>(xs[kb]) * static_cast<double>(ws[kb]) * part;",
     "acc += static_cast<double>(xs[0]) * static_cast<double>(ws[kb]) * part;"),
    ("mx-weight-exponent", "(static_cast<int>(ws[b]) - 127)", "(static_cast<int>(ws[b]) - 128)"),
    ("swiglu-operands-swapped", "h[n] = static_cast<float>(silu(g) * u);", "h[n] = static_cast<float>(silu(u) * g);"),
    ("layer-h-scale-240", "        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;\n        hs[q * ib + gi] = sc;",
     "        const float sc = amax > 0.0f ? amax / 240.0f : 1.0f;\n        hs[q * ib + gi] = sc;"),
    ("layer-h-tensor-scale-240", "h_tensor_scale = amax > 0.0f ? amax / 448.0f : 1.0f;",
     "h_tensor_scale = amax > 0.0f ? amax / 240.0f : 1.0f;"),
    ("layer-mx-h-blocks-of-64", "for (int b = 0; b < im; ++b) mx_quant_block(hv.data() + b * 32, 32,",
     "for (int b = 0; b < im / 2; ++b) mx_quant_block(hv.data() + b * 64, 64,"),
    # combine and norm
    ("combine-rank0-weight", "const double wt = j == k ? 1.0 : weights[t * k + j];",
     "const double wt = j == k ? 1.0 : weights[t * k];"),
    ("combine-shared-row", "if (has_shared) acc += y[(P + t) * H + m];", "if (has_shared) acc += y[t * H + m];"),
    ("rmsnorm-mean-over-H-1", "std::sqrt(ssq / H + eps)", "std::sqrt(ssq / (H - 1) + eps)"),
    ("rmsnorm-weight-dropped", "out[r * H + m] = s[r * H + m] * inv * bf16_value(weight[m]);",
     "out[r * H + m] = s[r * H + m] * inv;"),
]


def _build(name, old, new, out_dir):
    src = open(SRC).read()
    assert src.count(old) == 1, f"{name}: fragment must occur exactly once in the oracle source"
    path = os.path.join(out_dir, f"{name}.cpp")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(out_dir, f"lib{name}.so")
    # the oracle's own compiler flags (oracle.build)
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
                           "-ffp-contract=off", "-o", lib, path])
    return lib


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("mutants"))
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as pool:
        futs = {name: pool.submit(_build, name, old, new, out) for name, old, new in MUTANTS}
        return {name: f.result() for name, f in futs.items()}


@pytest.fixture(scope="module")
def pin_runs(mutant_libs):
    """Exit status and output of the pin suite against every mutant (4 at a time)."""
    def run(name):
        env = dict(os.environ, MOE355_ORACLE_LIB=mutant_libs[name], OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                            *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        return r.returncode, r.stdout[-3000:]
    with cf.ThreadPoolExecutor(4) as pool:
        futs = {name: pool.submit(run, name) for name, _, _ in MUTANTS}
        return {name: f.result() for name, f in futs.items()}


def test_unmodified_source_passes_the_pins(tmp_path):
    """Control: the same build route with no change gives a library the pins pass."""
    lib = _build("identity", "int orc_version(void) { return 1; }", "int orc_version(void) { return 1; }",
                 str(tmp_path))
    env = dict(os.environ, MOE355_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:]


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, pin_runs):
    rc, out = pin_runs[name]
    # exit status 1: tests ran and at least one failed (not a crash or a collection error)
    assert rc == 1 and " failed" in out, f"mutant {name} not caught (exit {rc}):\n{out}"
