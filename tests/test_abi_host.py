"""Host-side tests of libox (no GPU needed): the library loads and exports every
symbol include/ox.h declares; every validation error is reported before
anything is enqueued (these calls never reach the HIP runtime); the offline
helpers (BatchNorm fold, int8 parameter block) match the oracle or their
definitions."""
import ctypes as C
import os
import re
import struct

import numpy as np
import pytest

import oracle
import synth
from kernel_rules import dwr_applies

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ox():
    import conv_implicit_gemm_amd as ox
    return ox


def header_symbols():
    src = open(os.path.join(ROOT, "include", "ox.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ox_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(ox):
    syms = header_symbols()
    assert set(syms) == set(ox.EXPORTS), syms
    for s in syms:
        assert hasattr(ox.lib, s), s
    assert ox.ox_version().startswith("ox ")


def test_package_has_no_oracle_dependency():
    pkg = os.path.join(ROOT, "conv_implicit_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower().replace("no oracle", ""), f
                assert "oxref" not in text, f


# ------------------------------------------------------------ error paths --

def raw(ox):
    return ox.lib


def desc(ox, **kw):
    base = dict(N=1, Cin=4, H=8, W=8, M=8, kH=3, kW=3, stride=(1, 1), pads=(1, 1, 1, 1),
                dilation=(1, 1), group=1)
    base.update(kw)
    return ox.conv_desc(base["N"], base["Cin"], base["H"], base["W"], base["M"], base["kH"],
                        base["kW"], base["stride"], base["pads"], base["dilation"], base["group"])


FAKE = 0x1000   # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,status,needle", [
    (dict(group=3), 2, "group=3 does not divide C=4"),
    (dict(Cin=4, M=6, group=4), 2, "does not divide M=6"),
    (dict(H=2, W=2, kH=5, kW=5, pads=(0, 0, 0, 0)), 2, "output size"),
    (dict(kH=0), 1, "kH=0"),
    (dict(stride=(0, 1)), 1, "s_h=0"),
    (dict(dilation=(1, 0)), 1, "d_w=0"),
    (dict(pads=(0, -1, 0, 0)), 1, "p_l=-1"),
    (dict(N=-1), 1, "N=-1"),
    (dict(H=1 << 24), 3, "2^24"),
    (dict(N=1 << 20, Cin=1 << 12, H=1, W=1, kH=1, kW=1, pads=(0, 0, 0, 0)), 3, "X has >= 2^31"),
])
def test_conv_shape_errors(ox, kw, status, needle):
    d = desc(ox, **kw)
    st = raw(ox).ox_conv2d_fused(ox.OX_F32, C.byref(d), FAKE, FAKE, None, 0, FAKE, None)
    assert st == status and needle in ox.ox_last_error(), ox.ox_last_error()


def test_conv_argument_errors(ox):
    L = raw(ox)
    d = desc(ox)
    assert L.ox_conv2d_fused(ox.OX_I8, C.byref(d), FAKE, FAKE, None, 0, FAKE, None) == 3
    assert L.ox_conv2d_fused(ox.OX_F32, C.byref(d), FAKE, FAKE, None, 7, FAKE, None) == 1
    assert "activation" in ox.ox_last_error()
    assert L.ox_conv2d_fused(ox.OX_F32, None, FAKE, FAKE, None, 0, FAKE, None) == 1
    for args, name in (((None, FAKE, FAKE), "X"), ((FAKE, None, FAKE), "W"), ((FAKE, FAKE, None), "Y")):
        st = L.ox_conv2d_fused(ox.OX_BF16, C.byref(d), args[0], args[1], None, 0, args[2], None)
        assert st == 1 and ("%s is NULL" % name) in ox.ox_last_error()
    # int8 entry
    assert L.ox_conv2d_int8(C.byref(d), FAKE, FAKE, None, ox.OX_I8, FAKE, None) == 1
    assert "int8_params" in ox.ox_last_error()
    assert L.ox_conv2d_int8(C.byref(d), FAKE, FAKE, FAKE, ox.OX_F32, FAKE, None) == 3


def test_forced_variant_must_apply(ox, monkeypatch):
    L = raw(ox)
    d = desc(ox)   # a 3x3 conv, not depthwise
    monkeypatch.setenv("OX_FORCE_KERNEL", "dw")
    assert L.ox_conv2d_fused(ox.OX_F32, C.byref(d), FAKE, FAKE, None, 0, FAKE, None) == 3
    monkeypatch.setenv("OX_FORCE_KERNEL", "1x1")
    assert L.ox_conv2d_fused(ox.OX_F32, C.byref(d), FAKE, FAKE, None, 0, FAKE, None) == 3
    monkeypatch.setenv("OX_FORCE_KERNEL", "gemv")
    assert L.ox_conv2d_fused(ox.OX_F32, C.byref(d), FAKE, FAKE, None, 0, FAKE, None) == 1
    monkeypatch.setenv("OX_FORCE_KERNEL", "igemm,tile=7x7")
    assert L.ox_conv2d_fused(ox.OX_F32, C.byref(d), FAKE, FAKE, None, 0, FAKE, None) == 1
    assert "unknown tile" in ox.ox_last_error()
    monkeypatch.setenv("OX_FORCE_KERNEL", "gemv")
    st = L.ox_gemm_fused(ox.OX_F32, 4, 8, 8, 0, 1, 1.0, FAKE, FAKE, 1.0, None, 0, FAKE, None, None)
    assert st == 3 and "M=1" in ox.ox_last_error()


def test_variant_selection_sweep(ox, monkeypatch):
    # host-side planning of every kernel over many geometries (no launches):
    # each call returns a name and the expected kernels are chosen
    import numpy as np
    r = np.random.default_rng(2024)
    for _ in range(600):
        dt = str(r.choice(["f32", "bf16", "i8"]))
        k = int(r.choice([1, 1, 3, 3, 5, 7]))
        g = 1
        C = int(r.choice([1, 3, 4, 16, 32, 64, 96, 128, 256, 512, 2048]))
        M = int(r.choice([1, 5, 64, 130, 256, 2048]))
        if r.random() < 0.15:
            g, M = C, C
        N = int(r.integers(1, 40))
        H, W = int(r.integers(k, 60)), int(r.integers(k, 60))
        s = int(r.choice([1, 2]))
        p = k // 2
        name = ox.ox_conv2d_variant(dt, N, C, H, W, M, k, k, (s, s), (p, p, p, p), (1, 1), g)
        assert "/" in name
        if dt == "bf16" and g == 1 and k == 1 and s == 1 and C % 32 == 0:
            # the DMA-staged kernel where the plane has an even pixel count
            # (the fake pointers are aligned) and C is a multiple of 64 or the
            # layer has at least 65536 pixels, else the register-staged one,
            # except on an odd plane with C <= 192 or M <= 384 (the tile
            # engine's 1x1)
            if (H * W) % 2 == 0 and (C % 64 == 0 or N * H * W >= 65536):
                want = "pwd/"
            elif (H * W) % 2 == 1 and (C <= 192 or M <= 384):
                want = "1x1/"
            else:
                want = "pw/"
            assert name.startswith(want), (name, C, M, H, W)
        if dt == "bf16" and g == 1 and k == 3 and C % 32 == 0:
            assert name.startswith("patch/"), (name, C, M, H, W, s)
        if dt == "bf16" and g == 1 and C <= 4 and k > 1 and not (C == 1 and M == 1):
            assert name.startswith("smallc/"), (name, C, k, s)
        if g == C and M == C and k == 3 and dt != "i8":
            # depthwise 3x3, pads 1: the row-segment kernel where it applies
            assert name.startswith("dwr/") == dwr_applies(dt, W, s), (name, dt, H, W, s)
    # pinned split-K counts, including more slices than chunks (short K on
    # this odd plane takes the tile engine unless pw is asked for)
    for splits in ("1", "2", "7", "64"):
        monkeypatch.setenv("OX_PW_SPLITS", splits)
        for C in (32, 64, 96, 2048):
            want = "pw/" if C > 192 else "1x1/"
            assert ox.ox_conv2d_variant("bf16", 2, C, 7, 7, 512, 1, 1).startswith(want)
        monkeypatch.setenv("OX_FORCE_KERNEL", "pw")
        for C in (32, 64, 96):
            assert ox.ox_conv2d_variant("bf16", 2, C, 7, 7, 512, 1, 1).startswith("pw/")
        monkeypatch.delenv("OX_FORCE_KERNEL")


def test_workspace_entry_point(ox):
    # split-K scratch: sized by the library, brought by the caller; the
    # checks run before anything is enqueued
    L = raw(ox)
    assert ox.ox_conv2d_workspace_bytes("bf16", 32, 2048, 7, 7, 512, 1, 1) > 0      # 104 tiles x 32 chunks
    assert ox.ox_conv2d_workspace_bytes("bf16", 32, 512, 7, 7, 512, 3, 3, (1, 1), (1, 1, 1, 1)) > 0
    assert ox.ox_conv2d_workspace_bytes("bf16", 32, 64, 56, 56, 256, 1, 1) == 0      # many tiles
    assert ox.ox_conv2d_workspace_bytes("f32", 32, 2048, 7, 7, 512, 1, 1) == 0
    d = ox.conv_desc(32, 2048, 7, 7, 512, 1, 1)
    need = ox.ox_conv2d_workspace_bytes("bf16", 32, 2048, 7, 7, 512, 1, 1)
    f = L.ox_conv2d_fused_ws
    assert f(ox.OX_BF16, C.byref(d), FAKE, FAKE, 0, None, 0, FAKE, FAKE + 8, need, None) == 1
    assert "16-byte aligned" in ox.ox_last_error()
    assert f(ox.OX_BF16, C.byref(d), FAKE, FAKE, 0, None, 0, FAKE, FAKE, need - 16, None) == 1
    assert "workspace_bytes" in ox.ox_last_error()
    assert f(ox.OX_BF16, C.byref(d), FAKE, FAKE, 2, None, 0, FAKE, FAKE, need, None) == 1
    assert "w_packed" in ox.ox_last_error()
    assert f(ox.OX_I8, C.byref(d), FAKE, FAKE, 0, None, 0, FAKE, FAKE, need, None) == 3


def test_residual_entry_point_errors(ox, monkeypatch):
    # the fused residual call validates before anything is enqueued: dtype,
    # the residual's alignment, forced kernels without a residual epilogue
    L = raw(ox)
    f = L.ox_conv2d_fused_res
    d = ox.conv_desc(2, 64, 8, 8, 64, 3, 3, (1, 1), (1, 1, 1, 1))
    assert f(ox.OX_I8, C.byref(d), FAKE, FAKE, None, FAKE, 0, FAKE, None, 0, None) == 3
    assert f(ox.OX_BF16, C.byref(d), FAKE, FAKE, None, FAKE + 1, 0, FAKE, None, 0, None) == 1
    assert "R is not aligned" in ox.ox_last_error()
    assert f(ox.OX_F32, C.byref(d), FAKE, FAKE, None, FAKE + 2, 0, FAKE, None, 0, None) == 1
    assert f(ox.OX_BF16, C.byref(d), FAKE, FAKE, None, FAKE, 7, FAKE, None, 0, None) == 1
    assert f(ox.OX_BF16, C.byref(d), FAKE, FAKE, None, FAKE, 0, None, None, 0, None) == 1
    assert "Y is NULL" in ox.ox_last_error()
    for v in ("patch", "dw", "smallc"):
        monkeypatch.setenv("OX_FORCE_KERNEL", v)
        assert f(ox.OX_BF16, C.byref(d), FAKE, FAKE, None, FAKE, 0, FAKE, None, 0, None) == 3
    monkeypatch.delenv("OX_FORCE_KERNEL")


def test_gemm_workspace_plan_and_errors(ox):
    # split-K is planned only for float Gemms too small to fill the GPU with a long K
    assert ox.ox_gemm_workspace_bytes("bf16", 64, 1024, 4096) == 8 * 64 * 1024 * 4
    assert ox.ox_gemm_workspace_bytes("bf16", 1000, 4096, 1024) == 0      # fills the chip
    assert ox.ox_gemm_workspace_bytes("f32", 16, 64, 128) == 0            # K too short
    assert ox.ox_gemm_workspace_bytes("bf16", 1, 4096, 4096) == 0         # one row: GEMV
    L = raw(ox)
    g = L.ox_gemm_fused_ws
    assert g(ox.OX_I8, 64, 1024, 4096, 0, 1, 1.0, FAKE, FAKE, 1.0, None, 0, FAKE, FAKE, 1 << 30, None) == 3
    need = ox.ox_gemm_workspace_bytes("bf16", 64, 1024, 4096)
    assert g(ox.OX_BF16, 64, 1024, 4096, 0, 1, 1.0, FAKE, FAKE, 1.0, None, 0, FAKE, FAKE, need - 4, None) == 1
    assert "workspace" in ox.ox_last_error()
    assert g(ox.OX_BF16, 64, 1024, 4096, 0, 1, 1.0, FAKE, FAKE, 1.0, None, 0, FAKE, FAKE + 8, need, None) == 1


def test_matmul_nbits_argument_errors(ox):
    L = raw(ox)
    nb = L.ox_matmul_nbits
    assert nb(ox.OX_F32, 2, 4, 64, 4, 32, FAKE, FAKE, FAKE, None, None, FAKE, None) == 3   # dtype
    assert nb(ox.OX_BF16, 2, 4, 64, 8, 32, FAKE, FAKE, FAKE, None, None, FAKE, None) == 3  # bits
    assert nb(ox.OX_BF16, 2, 4, 64, 4, 64, FAKE, FAKE, FAKE, None, None, FAKE, None) == 3  # block size
    assert nb(ox.OX_BF16, -2, 4, 64, 4, 32, FAKE, FAKE, FAKE, None, None, FAKE, None) == 2
    assert nb(ox.OX_BF16, 2, 4, 64, 4, 32, FAKE, None, FAKE, None, None, FAKE, None) == 1  # B NULL
    assert nb(ox.OX_BF16, 2, 4, 64, 4, 32, FAKE, FAKE + 2, FAKE, None, None, FAKE, None) == 1
    assert nb(ox.OX_BF16, 2, 4, 64, 4, 32, FAKE + 1, FAKE, FAKE, None, None, FAKE, None) == 1
    assert nb(ox.OX_BF16, 0, 4, 64, 4, 32, None, None, None, None, None, None, None) == 0  # empty


def test_dynamic_quantize_argument_errors(ox):
    L = raw(ox)
    need = L.ox_dynamic_quantize_workspace_bytes()
    assert need >= 16
    dq = L.ox_dynamic_quantize_linear
    assert dq(-1, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == 2
    assert dq(8, FAKE, FAKE, None, FAKE, FAKE, need, None) == 1                 # y_scale NULL
    assert dq(8, None, FAKE, FAKE, FAKE, FAKE, need, None) == 1                 # X NULL
    assert dq(8, FAKE + 2, FAKE, FAKE, FAKE, FAKE, need, None) == 1             # X misaligned
    assert dq(8, FAKE, FAKE, FAKE, FAKE, FAKE, need - 4, None) == 1             # workspace too small
    assert "workspace" in ox.ox_last_error()
    assert dq(8, FAKE, FAKE, FAKE, FAKE, FAKE + 8, need, None) == 1             # workspace misaligned
    assert dq(8, FAKE, FAKE, FAKE, FAKE, None, need, None) == 1


def test_pool_and_batchnorm_argument_errors(ox):
    L = raw(ox)
    bn = L.ox_batchnorm_act
    assert bn(ox.OX_I8, 1, 2, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-5, 0, FAKE, None) == 3
    assert bn(ox.OX_F32, -1, 2, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-5, 0, FAKE, None) == 2
    assert bn(ox.OX_F32, 1, 2, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, 0, FAKE, None) == 1
    assert "eps" in ox.ox_last_error()
    assert bn(ox.OX_F32, 1, 2, 4, FAKE, None, FAKE, FAKE, FAKE, 1e-5, 0, FAKE, None) == 1
    assert bn(ox.OX_BF16, 1, 2, 4, FAKE + 1, FAKE, FAKE, FAKE, FAKE, 1e-5, 0, FAKE, None) == 1
    assert bn(ox.OX_F32, 1, 2, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-5, 9, FAKE, None) == 1
    assert bn(ox.OX_F32, 0, 2, 4, None, None, None, None, None, 1e-5, 0, None, None) == 0   # empty: nothing to do
    mp = L.ox_maxpool2d
    d_bad = ox.conv_desc(1, 4, 8, 8, 5, 3, 3, (2, 2), (1, 1, 1, 1))
    assert mp(ox.OX_F32, C.byref(d_bad), FAKE, FAKE, None) == 1
    assert "M == C" in ox.ox_last_error()
    d_pad = ox.conv_desc(1, 4, 8, 8, 4, 2, 2, (1, 1), (2, 0, 0, 0))
    assert mp(ox.OX_F32, C.byref(d_pad), FAKE, FAKE, None) == 1
    assert "pad reaches" in ox.ox_last_error()
    d_small = ox.conv_desc(1, 4, 2, 2, 4, 5, 5)
    assert mp(ox.OX_F32, C.byref(d_small), FAKE, FAKE, None) == 2
    gap = L.ox_global_avgpool
    assert gap(ox.OX_F32, 1, 2, 0, FAKE, FAKE, None) == 2
    assert gap(ox.OX_I8, 1, 2, 4, FAKE, FAKE, None) == 3
    assert gap(ox.OX_F32, 1, 2, 4, None, FAKE, None) == 1


def test_gemm_argument_errors(ox):
    L = raw(ox)
    g = L.ox_gemm_fused
    assert g(ox.OX_F32, -1, 4, 4, 0, 0, 1.0, FAKE, FAKE, 1.0, None, 0, FAKE, None, None) == 1
    assert g(ox.OX_F32, 4, 4, 4, 2, 0, 1.0, FAKE, FAKE, 1.0, None, 0, FAKE, None, None) == 1
    assert g(ox.OX_F32, 4, 4, 4, 0, 0, float("inf"), FAKE, FAKE, 1.0, None, 0, FAKE, None, None) == 1
    assert g(ox.OX_F32, 4, 4, 4, 0, 0, 1.0, None, FAKE, 1.0, None, 0, FAKE, None, None) == 1
    assert "A is NULL" in ox.ox_last_error()
    assert g(ox.OX_F32, 4, 4, 4, 0, 0, 1.0, FAKE, FAKE, 1.0, None, 0, None, None, None) == 1
    assert g(ox.OX_F32, 4, 4, 4, 0, 0, 1.0, FAKE, FAKE, 1.0, None, 0, FAKE, FAKE, None) == 1
    assert "int8_params must be NULL" in ox.ox_last_error()
    # int8 constraints
    assert g(ox.OX_I8, 4, 4, 4, 0, 0, 1.0, FAKE, FAKE, 1.0, None, 0, FAKE, FAKE, None) == 3
    assert "transB=1" in ox.ox_last_error()
    assert g(ox.OX_I8, 4, 4, 4, 0, 1, 1.0, FAKE, FAKE, 1.0, FAKE, 0, FAKE, FAKE, None) == 1
    assert g(ox.OX_I8, 4, 4, 4, 0, 1, 2.0, FAKE, FAKE, 1.0, None, 0, FAKE, FAKE, None) == 3
    assert g(ox.OX_I8, 4, 4, 4, 0, 1, 1.0, FAKE, FAKE, 1.0, None, 1, FAKE, FAKE, None) == 3
    assert g(ox.OX_I8, 4, 4, 4, 0, 1, 1.0, FAKE, FAKE, 1.0, None, 0, FAKE, None, None) == 1
    assert g(ox.OX_F32, 1 << 16, 1 << 16, 4, 0, 0, 1.0, FAKE, FAKE, 1.0, None, 0, FAKE, None, None) == 3


def test_matmul_argument_errors(ox):
    L = raw(ox)
    m = L.ox_matmul_batched
    assert m(ox.OX_I8, 2, 4, 4, 4, FAKE, 16, FAKE, 16, FAKE, None) == 3
    assert m(ox.OX_F32, 2, 4, 4, 4, FAKE, 8, FAKE, 16, FAKE, None) == 1
    assert "sA=8" in ox.ox_last_error()
    assert m(ox.OX_F32, 2, 4, 4, 4, FAKE, 16, FAKE, 5, FAKE, None) == 1
    assert m(ox.OX_F32, 2, 4, 4, 4, FAKE, 16, FAKE, 16, None, None) == 1


def test_empty_shapes_enqueue_nothing_and_succeed(ox):
    L = raw(ox)
    # zero-sized outputs return OX_OK without touching any pointer or the GPU
    assert L.ox_matmul_batched(ox.OX_F32, 0, 4, 4, 4, None, 16, None, 16, None, None) == 0
    assert L.ox_matmul_batched(ox.OX_F32, 3, 0, 4, 4, None, 0, None, 16, None, None) == 0
    assert L.ox_gemm_fused(ox.OX_F32, 0, 4, 4, 0, 0, 1.0, None, None, 1.0, None, 0, None, None, None) == 0
    d = desc(ox, N=0)
    assert L.ox_conv2d_fused(ox.OX_F32, C.byref(d), None, None, None, 0, None, None) == 0


# --------------------------------------------------------- offline helpers --

def test_fold_batchnorm_matches_oracle_fold(ox):
    layer = synth.ConvLayer("t", 1, 16, 5, 5, 24, 3, 1, 1, 1, "relu")
    t = synth.conv_inputs(layer, 3, 5)
    W32 = t["W"].astype(np.float32)
    prm = [t[k].astype(np.float32) for k in ("gamma", "beta", "mean", "var")]
    b0 = np.random.default_rng(0).standard_normal(24).astype(np.float32)
    Wg, bg = ox.ox_fold_batchnorm(W32, *prm, eps=1e-5, b0=b0)
    Wr, br = oracle.fold_batchnorm(W32.astype(np.float64), *[p.astype(np.float64) for p in prm],
                                   eps=float(np.float32(1e-5)), b0=b0.astype(np.float64))
    # the library folds in fp64 and rounds once to fp32
    assert np.array_equal(Wg, Wr.astype(np.float32))
    assert np.array_equal(bg, br.astype(np.float32))


def test_fold_batchnorm_errors(ox):
    L = raw(ox)
    z = np.zeros(4, np.float32)
    var = np.array([1, 1, -2, 1], np.float32)
    st = L.ox_fold_batchnorm(4, 3, np.zeros(12, np.float32).ctypes.data, None, z.ctypes.data,
                             z.ctypes.data, z.ctypes.data, var.ctypes.data, 1e-5,
                             np.zeros(12, np.float32).ctypes.data, np.zeros(4, np.float32).ctypes.data)
    assert st == 1 and "var[2]" in ox.ox_last_error()


def test_int8_params_block_layout(ox):
    r = np.random.default_rng(1)
    M, K = 6, 37
    wq = r.integers(-127, 128, (M, K)).astype(np.int8)
    ws = r.uniform(1e-3, 1e-2, M).astype(np.float32)
    bq = r.integers(-5000, 5000, M).astype(np.int32)
    xs, ys, xzp, yzp = np.float32(0.05), np.float32(0.7), -9, 4
    blk = ox.ox_int8_prepare(wq, ws, xs, xzp, ys, yzp, bq)
    assert blk.size == ox.ox_int8_params_bytes(M) == 32 + 16 * M
    magic, ver, m, xz, yz, flags = struct.unpack_from("<iiqiii", blk.tobytes(), 0)
    assert (magic, ver, m, xz, yz, flags) == (0x3849584F, 2, M, xzp, yzp, 0)
    assert not np.frombuffer(blk.tobytes(), np.int32, M, 32 + 12 * M).any()    # w_zp all 0
    mult = np.frombuffer(blk.tobytes(), np.float64, M, 32)
    bfold = np.frombuffer(blk.tobytes(), np.int32, M, 32 + 8 * M)
    # multiplier: ((double)x_s * (double)w_s) / (double)y_s, as the oracle defines it
    assert np.array_equal(mult, (np.float64(xs) * ws.astype(np.float64)) / np.float64(ys))
    # zero-point fold: bias_q - x_zp * sum_k w
    assert np.array_equal(bfold, bq.astype(np.int64) - xzp * wq.astype(np.int64).sum(1))
    # and the fold reproduces the oracle's accumulator on a Gemm
    x = r.integers(-128, 128, (5, K)).astype(np.int8)
    acc, _ = oracle.gemm_int8(x, wq, bq, xzp, xs, ws, ys, yzp)
    folded = x.astype(np.int64) @ wq.astype(np.int64).T + bfold[None, :]
    assert np.array_equal(acc, folded)


def test_int8_prepare_errors(ox):
    wq = np.zeros((2, 3), np.int8)
    with pytest.raises(ox.OxError):
        ox.ox_int8_prepare(wq, [0.01, 0.0], 0.1, 0, 0.2, 0)       # w_scale 0
    with pytest.raises(ox.OxError):
        ox.ox_int8_prepare(wq, [0.01, 0.01], 0.1, 200, 0.2, 0)    # x_zp out of range
    with pytest.raises(ox.OxError):
        ox.ox_int8_prepare(wq, [0.01, 0.01], float("nan"), 0, 0.2, 0)


def test_int8_params_block_unsigned_and_weight_zero_points(ox):
    # uint8 activations / outputs are read as int8 with the top bit flipped:
    # the block stores their zero points minus 128, folds with that x_zp, and
    # records the weight zero points and the flags
    r = np.random.default_rng(2)
    M, K = 5, 29
    wq = r.integers(-128, 128, (M, K)).astype(np.int8)
    ws = r.uniform(1e-3, 1e-2, M).astype(np.float32)
    bq = r.integers(-5000, 5000, M).astype(np.int32)
    wz = np.array([3, 0, -128, 127, -1], np.int32)
    xs, ys, xzp, yzp = np.float32(0.05), np.float32(0.7), 201, 17
    blk = ox.ox_int8_prepare(wq, ws, xs, xzp, ys, yzp, bq, w_zp=wz, x_unsigned=True, y_unsigned=True)
    magic, ver, m, xz, yz, flags = struct.unpack_from("<iiqiii", blk.tobytes(), 0)
    assert (ver, m, xz, yz, flags) == (2, M, xzp - 128, yzp - 128, 7)
    bfold = np.frombuffer(blk.tobytes(), np.int32, M, 32 + 8 * M)
    assert np.array_equal(np.frombuffer(blk.tobytes(), np.int32, M, 32 + 12 * M), wz)
    # the int8 view reproduces the oracle's uint8 accumulator with the
    # weight zero-point term: x' = u - 128, fold with x_zp - 128, then
    # - w_zp * sum (x' - x_zp')
    u = r.integers(0, 256, (4, K))
    acc, _ = oracle.qgemm(u, wq, bq, xzp, wz, xs, ws, ys, yzp, True)
    xv = u.astype(np.int64) - 128
    got = xv @ wq.astype(np.int64).T + bfold[None, :] - wz[None, :] * (xv - (xzp - 128)).sum(1)[:, None]
    assert np.array_equal(acc, got)
    # only x unsigned: flags 1; only weight zero points: flags 4
    b1 = ox.ox_int8_prepare(wq, ws, xs, 0, ys, 0, x_unsigned=True)
    assert struct.unpack_from("<iiqiii", b1.tobytes(), 0)[3:] == (-128, 0, 1)
    b4 = ox.ox_int8_prepare(wq, ws, xs, 0, ys, 0, w_zp=wz)
    assert struct.unpack_from("<iiqiii", b4.tobytes(), 0)[5] == 4


def test_int8_prepare_ex_errors(ox):
    wq = np.zeros((2, 3), np.int8)
    ws = [0.01, 0.01]
    with pytest.raises(ox.OxError):
        ox.ox_int8_prepare(wq, ws, 0.1, -1, 0.2, 0, x_unsigned=True)        # uint8 x_zp < 0
    with pytest.raises(ox.OxError):
        ox.ox_int8_prepare(wq, ws, 0.1, 0, 0.2, 256, y_unsigned=True)       # uint8 y_zp > 255
    with pytest.raises(ox.OxError):
        ox.ox_int8_prepare(wq, ws, 0.1, 0, 0.2, 0, w_zp=[0, 128])           # w_zp > 127
    with pytest.raises(TypeError):
        ox.ox_int8_prepare(wq.astype(np.uint8), ws, 0.1, 0, 0.2, 0)         # uint8 weights unconverted
    w8, z8 = ox.ox_int8_weights_from_uint8(np.array([[0, 255, 128]], np.uint8), 130)
    assert w8.tolist() == [[-128, 127, 0]] and z8.tolist() == [2]


def test_int8_prepare_refuses_exactly_the_channels_that_could_overflow(ox):
    # The int32 accumulator bound, exact per channel.  With x_zp = -128 an
    # activation byte can sit 255 above the zero point; K weights of -128
    # then reach -255*128*K, which fits int32 for K = 65793 and not for
    # K = 65794 (2^31 = 65793.1 * 32640).
    ok = np.full((1, 65793), -128, np.int8)
    bad = np.full((1, 65794), -128, np.int8)
    ox.ox_int8_prepare(ok, [0.01], 0.1, -128, 0.2, 0)
    with pytest.raises(ox.OxError) as e:
        ox.ox_int8_prepare(bad, [0.01], 0.1, -128, 0.2, 0)
    assert "channel 0" in str(e.value)
    # the K = 66000 case of a fixed K limit: refused at x_zp = -128 ...
    k66 = np.full((1, 66000), -128, np.int8)
    with pytest.raises(ox.OxError):
        ox.ox_int8_prepare(k66, [0.01], 0.1, -128, 0.2, 0)
    # ... and accepted at x_zp = 0, where |x - x_zp| <= 128 (128*128*66000 fits)
    ox.ox_int8_prepare(k66, [0.01], 0.1, 0, 0.2, 0)
    # the bias counts: -255*128*65793 = -2147483520, so bias_q = -128 reaches
    # INT32_MIN exactly (accepted) and -129 goes past it (refused)
    ox.ox_int8_prepare(ok, [0.01], 0.1, -128, 0.2, 0, bias_q=[-128])
    with pytest.raises(ox.OxError):
        ox.ox_int8_prepare(ok, [0.01], 0.1, -128, 0.2, 0, bias_q=[-129])
    # only the offending channel matters: a second channel of zeros is fine,
    # and the refusal names channel 1 when the long row is second
    two = np.zeros((2, 65794), np.int8)
    two[1, :] = -128
    with pytest.raises(ox.OxError) as e:
        ox.ox_int8_prepare(two, [0.01, 0.01], 0.1, -128, 0.2, 0)
    assert "channel 1" in str(e.value)
    # weight zero points: w - w_zp = -127 for w = 0, w_zp = 127; the bound is
    # 255*127*K, which fits for K = 66311 and not for K = 66312
    # (2^31 = 66311.06 * 32385)
    z = np.zeros((1, 66311), np.int8)
    ox.ox_int8_prepare(z, [0.01], 0.1, -128, 0.2, 0, w_zp=[127])
    with pytest.raises(ox.OxError):
        ox.ox_int8_prepare(np.zeros((1, 66312), np.int8), [0.01], 0.1, -128, 0.2, 0, w_zp=[127])
    # ... and a zero-point-free row of zeros of that length is fine
    ox.ox_int8_prepare(np.zeros((1, 66312), np.int8), [0.01], 0.1, -128, 0.2, 0)


def test_pack_weights_is_tap_major_channel_blocks(ox):
    # Wp[m][c/32][tap][c%32] = W[m][c][tap]: checked against a numpy
    # reshape/transpose of the same array
    r = np.random.default_rng(4)
    M, Cin = 5, 64
    W = r.integers(0, 60000, (M, Cin, 3, 3)).astype(np.uint16)
    assert ox.ox_conv2d_packed_weights_bytes("bf16", 2, Cin, 9, 9, M, 3, 3, (1, 1), (1, 1, 1, 1)) == W.nbytes
    Wp = ox.ox_conv2d_pack_weights(W, "bf16", 2, Cin, 9, 9, (1, 1), (1, 1, 1, 1))
    ref = W.reshape(M, Cin // 32, 32, 9).transpose(0, 1, 3, 2)
    assert np.array_equal(Wp.reshape(M, Cin // 32, 9, 32), ref)


def test_packed_layout_only_where_a_packed_kernel_exists(ox):
    b = ox.ox_conv2d_packed_weights_bytes
    assert b("bf16", 1, 48, 9, 9, 8, 3, 3) == 0            # C % 32 != 0
    assert b("bf16", 1, 64, 9, 9, 8, 5, 5) == 0            # not 3x3
    assert b("f32", 1, 64, 9, 9, 8, 3, 3) == 0             # bf16 only
    assert b("bf16", 1, 64, 9, 9, 8, 3, 3, (3, 3)) == 0    # stride 3
    assert b("bf16", 1, 64, 9, 9, 8, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 2) == 0   # grouped
    with pytest.raises(ox.OxError):
        ox.ox_conv2d_pack_weights(np.zeros((8, 48, 3, 3), np.uint16), "bf16", 1, 48, 9, 9)
    d = desc(ox, Cin=64, M=8)
    st = raw(ox).ox_conv2d_fused_packed(ox.OX_F32, C.byref(d), FAKE, FAKE, None, 0, FAKE, None)
    assert st == 3 and "packed" in ox.ox_last_error()


def test_static_scratch_entry_point_refuses_oversized_plans(ox, monkeypatch):
    # ox_conv2d_fused_static: a split-K plan needing more scratch than the
    # static array is refused as unsupported before any HIP call (forced
    # here with many slices on a long-K 1x1), and argument errors come first
    L = raw(ox)
    assert ox.ox_static_scratch_bytes() == 32 << 20
    monkeypatch.setenv("OX_FORCE_KERNEL", "pw")
    monkeypatch.setenv("OX_PW_SPLITS", "64")
    need = ox.ox_conv2d_workspace_bytes("bf16", 32, 2048, 7, 7, 512, 1, 1)
    assert need > ox.ox_static_scratch_bytes()
    d = ox.conv_desc(32, 2048, 7, 7, 512, 1, 1)
    st = L.ox_conv2d_fused_static(ox.OX_BF16, C.byref(d), FAKE, FAKE, 0, None, 0, FAKE, None)
    assert st == 3 and "static scratch" in ox.ox_last_error() and str(need) in ox.ox_last_error()
    st = L.ox_conv2d_fused_static(ox.OX_BF16, C.byref(d), None, FAKE, 0, None, 0, FAKE, None)
    assert st == 1 and "X is NULL" in ox.ox_last_error()
    st = L.ox_conv2d_fused_static(ox.OX_BF16, C.byref(d), FAKE, FAKE, 2, None, 0, FAKE, None)
    assert st == 1 and "w_packed" in ox.ox_last_error()
