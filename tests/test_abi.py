"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/moe355.h, and refuses bad arguments with the documented
status codes before anything is launched (fake, never-dereferenced device
pointers are enough because validation is host-only)."""
import ctypes
import os
import re

import pytest

import expert_layer_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe355.h")

A = 0x100000      # fake 16-byte aligned "device" addresses
B = 0x900000
C = 0x1100000
D = 0x1900000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe355.so not built")
    return moe.lib()


def test_every_declared_symbol_is_exported_and_bound(L):
    names = declared_functions()
    assert len(names) == 22
    for n in names:
        assert hasattr(L, n), n
    assert sorted(moe.exported_symbols()) == names


def test_version_and_status_strings(L):
    assert L.moe_abi_version() == 4
    assert moe.moe_status_string(0) == "ok"
    for s in range(1, 5):
        assert moe.moe_status_string(s) not in ("ok", "unknown status")
    assert moe.moe_status_string(99) == "unknown status"


def test_route_validation(L):
    r = L.moe_route
    assert r(A, None, None, -1, 8, 2, B, C, None) == moe.MOE_EINVAL
    assert r(A, None, None, 4, 8, 9, B, C, None) == moe.MOE_EINVAL          # k > E
    assert r(A, None, None, 4, 2000, 8, B, C, None) == moe.MOE_EUNSUPPORTED  # E > 1024
    assert r(A, None, None, 4, 64, 33, B, C, None) == moe.MOE_EUNSUPPORTED   # k > 32
    assert r(None, None, None, 4, 8, 2, B, C, None) == moe.MOE_EINVAL
    assert r(A, None, D, 4, 8, 2, B, C, None) == moe.MOE_EINVAL              # rows flag without bias
    assert r(A, None, None, 4, 8, 2, B, B + 8, None) == moe.MOE_EINVAL      # outputs overlap
    assert r(A, None, None, 0, 8, 2, B, C, None) == moe.MOE_OK               # T == 0: no-op
    assert r(None, None, None, 0, 8, 2, None, None, None) == moe.MOE_OK


def test_align_validation(L):
    al = L.moe_align
    assert al(A, 4, 8, 2, 2, B, C, D, D + 4096, None, 0, None) == moe.MOE_EINVAL       # shared not 0/1
    assert al(A, 4, 8, 2, 1, None, C, D, D + 4096, None, 0, None) == moe.MOE_EINVAL
    assert al(A, 4, 8, 2, 1, B, B, D, D + 4096, None, 0, None) == moe.MOE_EINVAL       # counts/offsets alias
    T, E, k = 2000, 64, 8
    need = L.moe_align_workspace_bytes(T, E, k)
    assert need == 2 * E * 4
    base = 0x10000000
    ps = base + 0x100000
    assert al(A, T, E, k, 1, B, C, base, ps, None, 0, None) == moe.MOE_EWORKSPACE
    assert al(A, T, E, k, 1, B, C, base, ps, D, need - 1, None) == moe.MOE_EWORKSPACE
    assert L.moe_align_workspace_bytes(64, 256, 8) == 0                               # single workgroup
    assert al(A, 0, E, k, 1, B, C, base, ps, None, 0, None) == moe.MOE_OK


def test_quant_validation(L):
    assert L.moe_quant_rows_fp8(A, 4, 100, B, C, None) == moe.MOE_EUNSUPPORTED
    assert L.moe_quant_rows_fp8(A + 2, 4, 128, B, C, None) == moe.MOE_EINVAL           # misaligned x
    assert L.moe_quant_rows_fp8(A, 0, 128, B, C, None) == moe.MOE_OK
    assert L.moe_quant_blocks_fp8(A, 2, 100, 128, B, C, None) == moe.MOE_EUNSUPPORTED
    assert L.moe_quant_blocks_fp8(A, -1, 128, 128, B, C, None) == moe.MOE_EINVAL


def test_quant_mxfp8_validation(L):
    qm = L.moe_quant_rows_mxfp8
    assert qm(A, 4, 48, B, C, None) == moe.MOE_EUNSUPPORTED          # cols % 32
    assert qm(A, -1, 64, B, C, None) == moe.MOE_EINVAL
    assert qm(A + 2, 4, 64, B, C, None) == moe.MOE_EINVAL             # x misaligned
    assert qm(A, 4, 64, B + 4, C, None) == moe.MOE_EINVAL             # q misaligned
    assert qm(A, 4, 64, B, B + 8, None) == moe.MOE_EINVAL             # s overlaps q
    assert qm(A, 4, 64, None, C, None) == moe.MOE_EINVAL
    assert qm(A, 0, 64, B, C, None) == moe.MOE_OK


def _experts(**kw):
    d = dict(wtype=0, E=8, H=256, I=128, has_shared=0, w1=A, w3=B, w2=C)
    d.update(kw)
    c = moe.moe_experts_t()
    for k, v in d.items():
        setattr(c, k, v)
    return c


def test_gemm_validation(L):
    g13 = L.moe_gemm13
    x, off, sp, h = 0x20000000, 0x21000000, 0x22000000, 0x23000000
    ok = _experts()
    assert g13(ctypes.byref(_experts(H=100)), x, None, off, sp, 4, 2, h, None, None, 0, None) == moe.MOE_EUNSUPPORTED
    assert g13(ctypes.byref(_experts(I=200)), x, None, off, sp, 4, 2, h, None, None, 0, None) == moe.MOE_EUNSUPPORTED
    assert g13(ctypes.byref(_experts(wtype=7)), x, None, off, sp, 4, 2, h, None, None, 0, None) == moe.MOE_EUNSUPPORTED
    assert g13(ctypes.byref(_experts(wtype=1)), x, None, off, sp, 4, 2, h, None, None, 0, None) == moe.MOE_EINVAL
    assert g13(ctypes.byref(_experts(has_shared=1)), x, None, off, sp, 4, 2, h, None, None, 0, None) == moe.MOE_EINVAL
    assert g13(ctypes.byref(_experts(w2=C + 4)), x, None, off, sp, 4, 2, h, None, None, 0, None) == moe.MOE_EINVAL
    assert g13(ctypes.byref(ok), x, None, off, sp, 4, 9, h, None, None, 0, None) == moe.MOE_EINVAL       # k > E
    assert g13(ctypes.byref(ok), x, None, off, sp, 4, 2, x, None, None, 0, None) == moe.MOE_EINVAL       # h aliases x
    assert g13(ctypes.byref(ok), x, None, off, sp, 0, 2, h, None, None, 0, None) == moe.MOE_OK
    assert g13(None, x, None, off, sp, 4, 2, h, None, None, 0, None) == moe.MOE_EINVAL
    mx = _experts(wtype=2, s1=A, s3=B, s2=C)
    assert g13(ctypes.byref(mx), x, None, off, sp, 4, 2, h, None, None, 0, None) == moe.MOE_EINVAL   # no xs/hs
    assert g13(ctypes.byref(_experts(wtype=2)), x, D, off, sp, 4, 2, h, D + 4096, None, 0, None) == moe.MOE_EINVAL
    assert g13(ctypes.byref(_experts(wtype=2, s1=A, s3=B, s2=C, H=384)), x, D, off, sp, 4, 2, h, D + 4096,
               None, 0, None) == moe.MOE_EUNSUPPORTED                                           # MX needs H % 256
    assert g13(ctypes.byref(mx), x, D + 2, off, sp, 4, 2, h, D + 4096, D + 8192, 256, None) == moe.MOE_EINVAL
    assert g13(ctypes.byref(_experts(wtype=2, s1=A + 2, s3=B, s2=C)), x, D, off, sp, 4, 2, h, D + 4096,
               D + 8192, 256, None) == moe.MOE_EINVAL                                           # scales misaligned
    need = L.moe_gemm_workspace_bytes(ctypes.byref(ok), 4, 2)
    assert need > 0
    assert g13(ctypes.byref(ok), x, None, off, sp, 4, 2, h, None, None, 0, None) == moe.MOE_EWORKSPACE
    assert g13(ctypes.byref(ok), x, None, off, sp, 4, 2, h, None, D, need - 4, None) == moe.MOE_EWORKSPACE
    assert g13(ctypes.byref(ok), x, None, off, sp, 4, 2, h, None, D + 2, need, None) == moe.MOE_EINVAL   # misaligned
    assert g13(ctypes.byref(ok), x, None, off, sp, 4, 2, h, None, h + 64, need, None) == moe.MOE_EINVAL  # ws inside h
    g2 = L.moe_gemm2
    assert g2(ctypes.byref(ok), h, None, off, 4, 2, x, 3, None, 0, None) == moe.MOE_EUNSUPPORTED          # y dtype
    assert g2(ctypes.byref(_experts(wtype=1, s1=A, s3=B, s2=C)), h, None, off, 4, 2, x, 0, None, 0, None) == moe.MOE_EINVAL
    assert g2(ctypes.byref(ok), h, None, off, 0, 2, x, 0, None, 0, None) == moe.MOE_OK


def test_combine_validation(L):
    cb = L.moe_combine
    assert cb(A, 2, B, C, 4, 2, 256, 0, D, None) == moe.MOE_EUNSUPPORTED
    assert cb(A, 0, B, C, 4, 2, 200, 0, D, None) == moe.MOE_EUNSUPPORTED
    assert cb(A, 0, B, C, 4, 2, 256, 3, D, None) == moe.MOE_EINVAL
    assert cb(A, 0, B, C, 4, 2, 256, 0, A + 16, None) == moe.MOE_EINVAL    # out overlaps y
    assert cb(A, 0, B, C, 0, 2, 256, 0, D, None) == moe.MOE_OK


def test_combine_rmsnorm_validation(L):
    cr = L.moe_combine_rmsnorm
    F = ctypes.c_float
    E_ = 0x2100000   # another fake buffer
    args = lambda **kw: {**dict(y=A, yd=0, ps=B, w=C, T=4, k=2, H=256, sh=0, res=D, wt=E_, eps=F(1e-6),
                                out=0x2900000, ro=None), **kw}
    call = lambda a: cr(a["y"], a["yd"], a["ps"], a["w"], a["T"], a["k"], a["H"], a["sh"], a["res"], a["wt"],
                        a["eps"], a["out"], a["ro"], None)
    assert call(args(eps=F(-1.0))) == moe.MOE_EINVAL
    assert call(args(eps=F(float("nan")))) == moe.MOE_EINVAL
    assert call(args(H=200)) == moe.MOE_EUNSUPPORTED
    assert call(args(H=65536)) == moe.MOE_EUNSUPPORTED
    assert call(args(res=None)) == moe.MOE_EINVAL
    assert call(args(out=D + 64)) == moe.MOE_EINVAL                # out overlaps residual
    assert call(args(ro=D + 64)) == moe.MOE_EINVAL                 # partial overlap with residual
    assert call(args(T=0)) == moe.MOE_OK


def test_forward_validation(L):
    ex = _experts(has_shared=0)
    need = L.moe_forward_workspace_bytes(ctypes.byref(ex), 16, 2, 0)
    assert need > 0
    args = moe.moe_forward_args_t(16, 2, 0, A, B, None, None, None, None, C, None, None)
    ws = 0x40000000
    assert L.moe_forward(ctypes.byref(ex), ctypes.byref(args), ws, need - 1, None) == moe.MOE_EWORKSPACE
    args2 = moe.moe_forward_args_t(16, 2, 0, A, None, None, None, None, None, C, None, None)
    assert L.moe_forward(ctypes.byref(ex), ctypes.byref(args2), ws, need, None) == moe.MOE_EINVAL   # no logits, no router
    args3 = moe.moe_forward_args_t(16, 2, 5, A, B, None, None, None, None, C, None, None)
    assert L.moe_forward(ctypes.byref(ex), ctypes.byref(args3), ws, need, None) == moe.MOE_EUNSUPPORTED
    assert L.moe_forward(ctypes.byref(ex), None, ws, need, None) == moe.MOE_EINVAL
    args0 = moe.moe_forward_args_t(0, 2, 0, None, B, None, None, None, None, None, None, None)
    assert L.moe_forward(ctypes.byref(ex), ctypes.byref(args0), None, 0, None) == moe.MOE_OK


def test_forward_noalloc_validation(L):
    """Host-only checks of the workspace-free chain: argument errors as for
    moe_forward, and shapes whose intermediates exceed the fixed scratch are
    refused with MOE_EUNSUPPORTED before anything touches the device."""
    fn = L.moe_forward_noalloc
    ex = _experts(has_shared=0)
    args2 = moe.moe_forward_args_t(16, 2, 0, A, None, None, None, None, None, C, None, None)
    assert fn(ctypes.byref(ex), ctypes.byref(args2), None) == moe.MOE_EINVAL   # no logits, no router
    args3 = moe.moe_forward_args_t(16, 2, 5, A, B, None, None, None, None, C, None, None)
    assert fn(ctypes.byref(ex), ctypes.byref(args3), None) == moe.MOE_EUNSUPPORTED
    assert fn(ctypes.byref(ex), None, None) == moe.MOE_EINVAL
    big_T = 1 << 16
    assert L.moe_forward_workspace_bytes(ctypes.byref(ex), big_T, 2, 0) > moe.MOE_NOALLOC_SCRATCH_BYTES
    big = moe.moe_forward_args_t(big_T, 2, 0, A, B, None, None, None, None, C, None, None)
    assert fn(ctypes.byref(ex), ctypes.byref(big), None) == moe.MOE_EUNSUPPORTED
    args0 = moe.moe_forward_args_t(0, 2, 0, None, B, None, None, None, None, None, None, None)
    assert fn(ctypes.byref(ex), ctypes.byref(args0), None) == moe.MOE_OK


def test_forward_persistent_validation(L):
    """Same argument rules as moe_forward, plus the envelope (bf16 weights, T*k <= 16*E);
    every call here stops at host validation (or T == 0), so nothing is launched."""
    fp = L.moe_forward_persistent
    ex = _experts(has_shared=0)
    need = L.moe_forward_workspace_bytes(ctypes.byref(ex), 16, 2, 0)
    ws = 0x40000000
    args = moe.moe_forward_args_t(16, 2, 0, A, B, None, None, None, None, C, None, None)
    assert fp(ctypes.byref(ex), ctypes.byref(args), ws, need - 1, None) == moe.MOE_EWORKSPACE
    assert fp(ctypes.byref(ex), ctypes.byref(args), None, need, None) == moe.MOE_EWORKSPACE
    args2 = moe.moe_forward_args_t(16, 2, 0, A, None, None, None, None, None, C, None, None)
    assert fp(ctypes.byref(ex), ctypes.byref(args2), ws, need, None) == moe.MOE_EINVAL   # no logits, no router
    args3 = moe.moe_forward_args_t(16, 2, 5, A, B, None, None, None, None, C, None, None)
    assert fp(ctypes.byref(ex), ctypes.byref(args3), ws, need, None) == moe.MOE_EUNSUPPORTED
    assert fp(ctypes.byref(ex), None, ws, need, None) == moe.MOE_EINVAL
    assert fp(ctypes.byref(ex), ctypes.byref(args), C, need, None) == moe.MOE_EINVAL     # workspace holds out
    # outside the envelope: fp8 weights, and more than 16 routed rows per expert on average
    ex8 = _experts(wtype=1, s1=D, s3=D, s2=D)
    need8 = L.moe_forward_workspace_bytes(ctypes.byref(ex8), 16, 2, 0)
    assert fp(ctypes.byref(ex8), ctypes.byref(args), ws, need8, None) == moe.MOE_EUNSUPPORTED
    big = moe.moe_forward_args_t(128, 2, 0, A, B, None, None, None, None, C, None, None)   # 256 > 16 * 8 rows
    need_big = L.moe_forward_workspace_bytes(ctypes.byref(ex), 128, 2, 0)
    assert fp(ctypes.byref(ex), ctypes.byref(big), ws, need_big, None) == moe.MOE_EUNSUPPORTED
    args0 = moe.moe_forward_args_t(0, 2, 0, None, B, None, None, None, None, None, None, None)
    assert fp(ctypes.byref(ex), ctypes.byref(args0), None, 0, None) == moe.MOE_OK
    assert L.moe_forward_persistent_status(None, None) == moe.MOE_EINVAL


def test_tiled_only_types_refuse_past_32bit_offsets(L):
    """MXFP8 and per-tensor FP8 have only tiled kernels, whose gathered-row
    offsets are 32-bit: x [T,H] or h [R,I] with 2^31 elements or more is
    refused before anything is launched (bf16 and block fp8 take such shapes
    on the weight-streaming kernels instead)."""
    g13, g2 = L.moe_gemm13, L.moe_gemm2
    x, off, sp, h, ws = 0x20000000, 0x21000000, 0x22000000, 0x23000000, 0x30000000
    T_big = (1 << 31) // 4096 + 1                    # x has more than 2^31 elements at H = 4096
    for ex in (_experts(wtype=2, H=4096, s1=A, s3=B, s2=C), _experts(wtype=3, H=4096, s1=D, s3=D, s2=D)):
        assert g13(ctypes.byref(ex), x, D, off, sp, T_big, 1, h, D + 64, ws, 256, None) == moe.MOE_EUNSUPPORTED
        assert g2(ctypes.byref(ex), h, D, off, T_big, 1, x, 1, None, 0, None) == moe.MOE_EUNSUPPORTED
        assert L.moe_forward_workspace_bytes(ctypes.byref(ex), T_big, 1, 1) == 0
    # h [R, I] past 2^31 elements with x inside the range: R = T (k = 1), I = 2^14
    ex = _experts(wtype=2, H=256, I=1 << 14, s1=A, s3=B, s2=C)
    T_h = (1 << 31) // (1 << 14) + 1
    assert g2(ctypes.byref(ex), h, D, off, T_h, 1, x, 1, None, 0, None) == moe.MOE_EUNSUPPORTED


def test_per_tensor_validation(L):
    """Per-tensor FP8: the quantiser entry points and weight type 3 refuse bad
    arguments before launching anything."""
    amax = L.moe_tensor_amax
    qt = L.moe_quant_tensor_fp8
    F32, BF16 = moe.MOE_DTYPE_F32, moe.MOE_DTYPE_BF16
    assert amax(A, 7, 1, 256, B, None) == moe.MOE_EUNSUPPORTED              # unknown dtype
    assert amax(A, BF16, 1, 200, B, None) == moe.MOE_EUNSUPPORTED           # n % 128
    assert amax(A, BF16, 70000, 128, B, None) == moe.MOE_EUNSUPPORTED       # too many tensors
    assert amax(A, BF16, -1, 128, B, None) == moe.MOE_EINVAL
    assert amax(A, BF16, 1, 256, None, None) == moe.MOE_EINVAL
    assert amax(A + 2, BF16, 1, 256, B, None) == moe.MOE_EINVAL             # x not 16-byte aligned
    assert amax(A, F32, 1, 256, A + 16, None) == moe.MOE_EINVAL             # amax inside x
    assert amax(A, BF16, 0, 256, B, None) == moe.MOE_OK                     # nothing to do
    assert qt(A, BF16, 1, 256, B, A + 64, D, None) == moe.MOE_EINVAL        # codes overlap x
    assert qt(A, BF16, 1, 256, B, C, C + 8, None) == moe.MOE_EINVAL         # scale inside the codes
    assert qt(A, BF16, 1, 256, B, C + 4, D, None) == moe.MOE_EINVAL         # codes not 8-byte aligned
    assert qt(A, BF16, 1, 256, None, C, D, None) == moe.MOE_EINVAL
    assert qt(A, BF16, 1, 0, B, C, D, None) == moe.MOE_OK
    g13 = L.moe_gemm13
    x, off, sp, h = 0x20000000, 0x21000000, 0x22000000, 0x23000000
    pt = lambda **kw: _experts(wtype=3, H=256, s1=D, s3=D, s2=D, **kw)   # noqa: E731
    assert g13(ctypes.byref(_experts(wtype=3, H=256)), x, B, off, sp, 4, 2, h, C, None, 0, None) == moe.MOE_EINVAL
    assert g13(ctypes.byref(pt(I=128)), x, B + 2, off, sp, 4, 2, h, C, 0x30000000, 256, None) == moe.MOE_EINVAL
    assert g13(ctypes.byref(_experts(wtype=3, H=128, s1=D, s3=D, s2=D)), x, B, off, sp, 4, 2, h, C, 0x30000000,
               256, None) == moe.MOE_EUNSUPPORTED                                # H % 256 for the Down tiles
    assert g13(ctypes.byref(pt()), x, None, off, sp, 4, 2, h, C, 0x30000000, 256, None) == moe.MOE_EINVAL


def test_router_validation(L):
    assert L.moe_router_gemm(A, B, C, D, 4, 100, 8, None) == moe.MOE_EUNSUPPORTED
    assert L.moe_router_gemm(A, B, C, D, 4, 128, 2048, None) == moe.MOE_EUNSUPPORTED
    assert L.moe_router_gemm(A, B, C, D, 0, 128, 8, None) == moe.MOE_OK
    assert L.moe_router_split(A, B, B, 4, 4, None) == moe.MOE_EINVAL     # hi/lo alias
    assert L.moe_router_split(A, B, C, 0, 4, None) == moe.MOE_OK


def test_missing_library_fails_loudly(tmp_path):
    """With no built library the binding raises on first use; there is no
    other code path that could compute a result instead."""
    import subprocess
    import sys
    code = ("import expert_layer_amd as moe\n"
            "try:\n"
            "    moe.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    raise SystemExit('loaded a library that does not exist')\n")
    env = dict(os.environ, MOE355_LIB=str(tmp_path / "libmoe355.so"))
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "raised:" in r.stdout and "is not built" in r.stdout
