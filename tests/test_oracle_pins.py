"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- a closed form, an invariant, brute force, or an independent library
routine (numpy integer matmul, torch.nn.functional.conv2d / batch_norm in
float64, scipy's normal CDF).  A dropped term, a wrong sign, a wrong index or a
transposed operand in the oracle fails at least one of these.  CPU only."""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ MatMul --

def read_golden(name):
    """key = value lines of a golden file (comments start with #)."""
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (t.strip() for t in line.split("=", 1))
                vals[k] = float(v) if "." in v else int(v)
    return vals


def test_all_ones_64_cube_gives_64():
    # The closed-form case of the OxiONNX 0.1.7 two-stream race report
    # ("Why OxiONNX 0.1.7 is a game changer"): an all-ones MatMul of the
    # sizes the golden file records, where every correct element equals K.
    g = read_golden("all_ones_64.txt")
    M, N, K = g["M"], g["N"], g["K"]
    assert M * N == g["elements"] and g["value"] == K
    A = np.ones((1, M, K))
    B = np.ones((1, K, N))
    C = oracle.matmul(A, B)
    assert C.shape == (1, M, N)
    assert np.all(C == g["value"])
    Y = oracle.gemm(A[0], B[0].T.copy(), transB=True)
    assert np.all(Y == g["value"])
    # the race's reported result (3456 elements reading 0.0) fails this pin
    bad = C.copy().ravel()
    bad[:g["race_wrong"]] = g["race_wrong_value"]
    assert np.count_nonzero(bad != g["value"]) == g["race_wrong"]


def test_matmul_integer_inputs_exact_against_int64():
    r = np.random.default_rng(7)
    A = r.integers(-3, 4, (5, 17, 33))
    B = r.integers(-3, 4, (5, 33, 11))
    C = oracle.matmul(A, B)
    ref = np.matmul(A.astype(np.int64), B.astype(np.int64))
    assert np.array_equal(C, ref.astype(np.float64))


def test_matmul_against_numpy_float64():
    A, B = synth.matmul_inputs(batch=3, M=9, K=31, N=7)
    C = oracle.matmul(A, B)
    ref = np.matmul(A.astype(np.float64), B.astype(np.float64))
    np.testing.assert_allclose(C, ref, rtol=1e-13, atol=1e-13)


def test_matmul_identity_zero_and_broadcast():
    r = np.random.default_rng(3)
    A = r.uniform(-1, 1, (4, 6, 8))
    eye = np.eye(8)[None].repeat(4, 0)
    assert np.array_equal(oracle.matmul(A, eye), A)
    assert np.all(oracle.matmul(A, np.zeros((4, 8, 5))) == 0.0)
    B1 = r.uniform(-1, 1, (8, 5))
    bc = oracle.matmul(A, B1)                       # batch stride 0
    rep = oracle.matmul(A, np.repeat(B1[None], 4, 0))
    assert np.array_equal(bc, rep)


# -------------------------------------------------------------------- Gemm --

@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_gemm_transposes_alpha_beta_against_numpy(ta, tb):
    r = np.random.default_rng(11 + 2 * ta + tb)
    M, N, K = 7, 9, 13
    A = r.uniform(-1, 1, (K, M) if ta else (M, K))
    B = r.uniform(-1, 1, (N, K) if tb else (K, N))
    bias = r.uniform(-1, 1, N)
    Y = oracle.gemm(A, B, bias, alpha=0.75, beta=-1.5, transA=ta, transB=tb)
    Am = A.T if ta else A
    Bm = B.T if tb else B
    ref = 0.75 * (Am @ Bm) - 1.5 * bias[None, :]
    np.testing.assert_allclose(Y, ref, rtol=1e-13, atol=1e-13)
    at = np.array([0, 5, M * N - 1, 17])
    np.testing.assert_array_equal(oracle.gemm(A, B, bias, 0.75, -1.5, ta, tb, at=at), Y.ravel()[at])


@pytest.mark.parametrize("act", ["none", "relu", "relu6", "gelu"])
def test_gemm_zero_weights_gives_activation_of_bias(act):
    r = np.random.default_rng(5)
    X = r.standard_normal((4, 8))
    bias = np.array([-7.0, -0.5, 0.0, 0.25, 3.0, 6.0, 6.5, 9.0])
    Y = oracle.gemm(X, np.zeros((8, 8)), bias, transB=True, act=act)
    expect = oracle.act(act, bias)
    assert np.array_equal(Y, np.broadcast_to(expect, Y.shape))


# ------------------------------------------------------------- activations --

def test_relu_and_relu6_at_the_kinks():
    v = np.array([-2.0, -1e-300, 0.0, 1e-300, 3.0, 6.0 - 1e-12, 6.0, 6.0 + 1e-12, 100.0])
    assert list(oracle.act("relu", v)) == [0.0, 0.0, 0.0, 1e-300, 3.0, 6.0 - 1e-12, 6.0,
                                           6.0 + 1e-12, 100.0]
    assert list(oracle.act("relu6", v)) == [0.0, 0.0, 0.0, 1e-300, 3.0, 6.0 - 1e-12, 6.0, 6.0, 6.0]


def test_gelu_against_normal_cdf_and_identities():
    v = np.linspace(-9, 9, 721)
    g = oracle.act("gelu", v)
    # GELU(v) = v * Phi(v): scipy's normal CDF is an independent routine.
    np.testing.assert_allclose(g, v * scipy.special.ndtr(v), rtol=1e-14, atol=1e-15)
    assert oracle.act("gelu", np.array([0.0]))[0] == 0.0
    # odd-part identity: GELU(v) - GELU(-v) = v * (Phi(v) + Phi(-v) - 1) + v = v
    np.testing.assert_allclose(g - oracle.act("gelu", -v), v, rtol=0, atol=1e-14)
    # saturation: for v >= 8, GELU(v) rounds to v in float32
    big = np.array([8.0, 10.0, 50.0])
    assert np.array_equal(oracle.act("gelu", big).astype(np.float32), big.astype(np.float32))


def test_gelu_against_arbitrary_precision():
    # GELU(v) = v * Phi(v), Phi evaluated by mpmath at 40 digits (an
    # independent arbitrary-precision routine).
    import mpmath
    mpmath.mp.dps = 40
    v = np.array([-6.0, -3.0, -2.0, -1.0, -0.5, -1e-3, 1e-3, 0.5, 1.0, 2.0, 3.0, 6.0])
    ref = np.array([float(mpmath.mpf(x) * mpmath.ncdf(mpmath.mpf(x))) for x in v])
    # the erf form loses relative (not absolute) precision where 1 + erf cancels
    np.testing.assert_allclose(oracle.act("gelu", v), ref, rtol=1e-15, atol=1e-15)


def test_residual_bn_relu6_chain_from_kyanite_example():
    # tests/golden/kyanite_residual_bn_relu6.txt restates the Kyanite README
    # "Cuda Executor" autokernel example: rank 4, dense strides
    # {648, 81, 9, 1} (C = 8, 9x9), four channel-broadcast operands, and the
    # chain y = max(min(((x0 + x1) - x2) / x3 * x4 + x5, 6), 0).  The oracle's
    # unfused BatchNorm (with x3 = sqrt(var + eps)) followed by its ReLU6 must
    # compute the same values.
    spec = {}
    for line in open(os.path.join(GOLDEN, "kyanite_residual_bn_relu6.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=", 1)
            spec[k.strip()] = v.strip()
    strides = [int(t) for t in spec["dense_strides"].split(",")]
    bstr = [int(t) for t in spec["broadcast_strides"].split(",")]
    ops = spec["ops"].split(",")
    C, H, W = strides[0] // strides[1], strides[1] // strides[2], strides[2]
    assert (C, H, W) == (8, 9, 9) and bstr == [0, 1, 0, 0]
    r = np.random.default_rng(31)
    N, eps = 2, 1e-5
    x0, x1 = r.standard_normal((N, C, H, W)), r.standard_normal((N, C, H, W))
    mean, var = r.standard_normal(C), r.uniform(0.5, 1.5, C)
    gamma, beta = r.uniform(0.5, 1.5, C), r.standard_normal(C)
    chan = {"x2": mean, "x3": np.sqrt(var + eps), "x4": gamma, "x5": beta}
    y = x0.copy()
    for op in ops:
        name, arg = op.split(":")
        if name == "add" and arg == "x1":
            y = y + x1
        elif name in ("sub", "div", "mul", "add"):
            c = chan[arg][None, :, None, None]
            y = {"sub": y - c, "div": y / c, "mul": y * c, "add": y + c}[name]
        elif name == "min":
            y = np.minimum(y, float(arg))
        elif name == "max":
            y = np.maximum(y, float(arg))
        else:
            raise AssertionError(op)
    got = oracle.act("relu6", oracle.batchnorm(x0 + x1, gamma, beta, mean, var, eps))
    np.testing.assert_allclose(got, y, rtol=1e-14, atol=1e-14)


# -------------------------------------------------------------------- Conv --

def torch_conv(X, W, b, stride, pads, dil, group):
    """torch.nn.functional.conv2d in float64 on the CPU, with ONNX (t,l,b,r)
    pads applied by F.pad: an independent library implementation."""
    t, l, bb, r = pads
    x = F.pad(torch.from_numpy(X), (l, r, t, bb))
    y = F.conv2d(x, torch.from_numpy(W), None if b is None else torch.from_numpy(b),
                 stride=stride, dilation=dil, groups=group)
    return y.numpy()


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


def sweep_cases(n, seed):
    r = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        N = int(r.integers(1, 3))
        Cin = int(r.integers(1, 9))
        M = int(r.integers(1, 9))
        H, W = int(r.integers(1, 10)), int(r.integers(1, 10))
        kH, kW = int(r.choice([1, 2, 3, 5, 7])), int(r.choice([1, 2, 3, 5, 7]))
        s = (int(r.integers(1, 4)), int(r.integers(1, 4)))
        d = (int(r.integers(1, 3)), int(r.integers(1, 3)))
        pads = tuple(int(v) for v in r.integers(0, 4, 4))
        g = int(r.choice(_divisors(math.gcd(Cin, M))))
        act = str(r.choice(["none", "relu", "relu6", "gelu"]))
        cases.append((N, Cin, H, W, M, kH, kW, s, pads, d, g, act))
    return cases


def test_conv_sweep_against_torch_float64():
    ran = shaped = 0
    for ci, (N, Cin, H, W, M, kH, kW, s, pads, d, g, act) in enumerate(sweep_cases(700, 2024)):
        r = np.random.default_rng(ci)
        X = r.standard_normal((N, Cin, H, W))
        Wt = r.standard_normal((M, Cin // g, kH, kW))
        b = r.standard_normal(M)
        desc = oracle.conv_desc(N, Cin, H, W, M, kH, kW, s, pads, d, g)
        rc, Ho, Wo = oracle.conv_out_dims(desc)
        if Ho < 1 or Wo < 1:
            assert rc == oracle.ESHAPE
            with pytest.raises(oracle.OracleError):
                oracle.conv2d(X, Wt, b, s, pads, d, g, act)
            shaped += 1
            continue
        Y = oracle.conv2d(X, Wt, b, s, pads, d, g, act)
        ref = oracle.act(act, torch_conv(X, Wt, b, s, pads, d, g))
        np.testing.assert_allclose(Y, ref.reshape(Y.shape), rtol=1e-12, atol=1e-12,
                                   err_msg=str((N, Cin, H, W, M, kH, kW, s, pads, d, g, act)))
        ran += 1
    assert ran > 300 and shaped > 10


def test_conv_residual_against_torch_float64():
    # the fused residual (Kyanite README, "Cuda Executor": a single
    # convolution + residual + bias + relu operation): act(conv + b + R),
    # against torch's float64 convolution plus the residual
    ran = 0
    for ci, (N, Cin, H, W, M, kH, kW, s, pads, d, g, act) in enumerate(sweep_cases(300, 77077)):
        desc = oracle.conv_desc(N, Cin, H, W, M, kH, kW, s, pads, d, g)
        rc, Ho, Wo = oracle.conv_out_dims(desc)
        if Ho < 1 or Wo < 1:
            continue
        r = np.random.default_rng(5000 + ci)
        X = r.standard_normal((N, Cin, H, W))
        Wt = r.standard_normal((M, Cin // g, kH, kW))
        b = r.standard_normal(M)
        R = r.standard_normal((N, M, Ho, Wo))
        Y = oracle.conv2d(X, Wt, b, s, pads, d, g, act, residual=R)
        ref = oracle.act(act, torch_conv(X, Wt, b, s, pads, d, g).reshape(Y.shape) + R)
        np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12,
                                   err_msg=str((N, Cin, H, W, M, kH, kW, s, pads, d, g, act)))
        ran += 1
    assert ran > 150


def test_conv_residual_special_cases():
    # a zero residual is the plain convolution, bit for bit; zero weights give
    # act(b + R) exactly; the sampled-point form agrees with the full one
    r = np.random.default_rng(88)
    X = r.standard_normal((2, 6, 7, 9))
    Wt = r.standard_normal((5, 6, 3, 3))
    b = r.standard_normal(5)
    R = r.standard_normal((2, 5, 7, 9))
    for act in ("none", "relu", "relu6", "gelu"):
        plain = oracle.conv2d(X, Wt, b, (1, 1), (1, 1, 1, 1), act=act)
        zero = oracle.conv2d(X, Wt, b, (1, 1), (1, 1, 1, 1), act=act, residual=np.zeros_like(R))
        assert np.array_equal(plain, zero)
        z = oracle.conv2d(X, np.zeros_like(Wt), b, (1, 1), (1, 1, 1, 1), act=act, residual=R)
        assert np.array_equal(z, oracle.act(act, b[None, :, None, None] + R))
        full = oracle.conv2d(X, Wt, b, (1, 1), (1, 1, 1, 1), act=act, residual=R)
        idx = r.integers(0, full.size, 50)
        at = oracle.conv2d(X, Wt, b, (1, 1), (1, 1, 1, 1), act=act, residual=R, at=idx)
        assert np.array_equal(at, full.ravel()[idx])


@pytest.mark.parametrize("k", [3, 7])
def test_conv_centre_tap_is_identity(k):
    r = np.random.default_rng(k)
    X = r.standard_normal((2, 3, 9, 8))
    Wt = np.zeros((3, 3, k, k))
    for c in range(3):
        Wt[c, c, k // 2, k // 2] = 1.0
    p = k // 2
    assert np.array_equal(oracle.conv2d(X, Wt, pads=(p, p, p, p)), X)
    # stride s picks X[..., ::s, ::s]
    Y2 = oracle.conv2d(X, Wt, stride=(2, 3), pads=(p, p, p, p))
    assert np.array_equal(Y2, X[:, :, ::2, ::3])
    # a dilated centre tap is still the identity
    Yd = oracle.conv2d(X, Wt, pads=(2 * p, 2 * p, 2 * p, 2 * p), dilation=(2, 2))
    assert np.array_equal(Yd, X)


def test_conv_off_centre_tap_shifts_with_zero_fill():
    r = np.random.default_rng(1)
    X = r.standard_normal((1, 1, 6, 7))
    Wt = np.zeros((1, 1, 3, 3))
    Wt[0, 0, 0, 2] = 1.0   # tap (kh=0, kw=2): Y[oh,ow] = X[oh-1, ow+1]
    Y = oracle.conv2d(X, Wt, pads=(1, 1, 1, 1))
    ref = np.zeros_like(X)
    ref[0, 0, 1:, :-1] = X[0, 0, :-1, 1:]
    assert np.array_equal(Y, ref)


def test_depthwise_scaled_delta():
    r = np.random.default_rng(2)
    X = r.standard_normal((2, 5, 7, 6))
    alpha = np.array([0.5, -2.0, 1.0, 0.25, 4.0])
    Wt = np.zeros((5, 1, 3, 3))
    Wt[:, 0, 1, 1] = alpha
    Y = oracle.conv2d(X, Wt, pads=(1, 1, 1, 1), group=5)
    assert np.array_equal(Y, X * alpha[None, :, None, None])


@pytest.mark.parametrize("act", ["none", "relu", "relu6", "gelu"])
def test_conv_zero_weights_give_activation_of_bias(act):
    X = np.random.default_rng(0).standard_normal((1, 4, 5, 5))
    b = np.array([-1.0, 0.5, 5.0, 7.0])
    Y = oracle.conv2d(X, np.zeros((4, 4, 3, 3)), b, pads=(1, 1, 1, 1), act=act)
    assert np.array_equal(Y, np.broadcast_to(oracle.act(act, b)[None, :, None, None], Y.shape))


def test_grouped_conv_is_concatenation_of_groups():
    r = np.random.default_rng(4)
    g, cpg, mpg = 3, 2, 4
    X = r.standard_normal((2, g * cpg, 6, 5))
    Wt = r.standard_normal((g * mpg, cpg, 3, 2))
    b = r.standard_normal(g * mpg)
    Y = oracle.conv2d(X, Wt, b, (2, 1), (1, 0, 2, 1), (1, 2), g)
    parts = [oracle.conv2d(X[:, i * cpg:(i + 1) * cpg], Wt[i * mpg:(i + 1) * mpg],
                           b[i * mpg:(i + 1) * mpg], (2, 1), (1, 0, 2, 1), (1, 2), 1)
             for i in range(g)]
    assert np.array_equal(Y, np.concatenate(parts, axis=1))


def test_1x1_conv_equals_per_image_matmul():
    # two independent oracle routines (direct conv and MatMul) agree
    r = np.random.default_rng(9)
    X = r.standard_normal((3, 12, 5, 7))
    Wt = r.standard_normal((10, 12, 1, 1))
    Y = oracle.conv2d(X, Wt)
    mm = oracle.matmul(X.reshape(3, 12, 35).transpose(0, 2, 1).copy(), Wt[:, :, 0, 0].T.copy())
    np.testing.assert_allclose(Y, mm.transpose(0, 2, 1).reshape(Y.shape), rtol=1e-13, atol=1e-13)


def test_conv_sampled_points_match_full():
    r = np.random.default_rng(6)
    X = r.standard_normal((2, 6, 11, 9))
    Wt = r.standard_normal((4, 3, 3, 3))
    b = r.standard_normal(4)
    Y = oracle.conv2d(X, Wt, b, (2, 1), (1, 2, 0, 1), (1, 1), 2, "gelu")
    at = r.integers(0, Y.size, 50)
    assert np.array_equal(oracle.conv2d(X, Wt, b, (2, 1), (1, 2, 0, 1), (1, 1), 2, "gelu", at=at),
                          Y.ravel()[at])


# --------------------------------------------------------------- BatchNorm --

def test_maxpool_against_torch_float64():
    # ONNX MaxPool: torch's max_pool2d on the input padded with -inf (ONNX
    # pads may be asymmetric), float64
    r = np.random.default_rng(606)
    ran = 0
    for ci in range(400):
        N, Cc = int(r.integers(1, 3)), int(r.integers(1, 5))
        H, W = int(r.integers(1, 12)), int(r.integers(1, 12))
        kH, kW = int(r.integers(1, 5)), int(r.integers(1, 5))
        s = (int(r.integers(1, 4)), int(r.integers(1, 4)))
        d = (int(r.integers(1, 3)), int(r.integers(1, 3)))
        pads = tuple(int(v) for v in r.integers(0, 3, 4))
        if pads[0] >= kH * d[0] or pads[2] >= kH * d[0] or pads[1] >= kW * d[1] or pads[3] >= kW * d[1]:
            continue                    # a window entirely in the padding: not a valid ONNX MaxPool
        desc = oracle.conv_desc(N, Cc, H, W, Cc, kH, kW, s, pads, d, 1)
        rc, Ho, Wo = oracle.conv_out_dims(desc)
        if Ho < 1 or Wo < 1:
            continue
        X = r.standard_normal((N, Cc, H, W))
        t, lft, b, rt = pads
        xp = F.pad(torch.from_numpy(X), (lft, rt, t, b), value=float("-inf"))
        ref = F.max_pool2d(xp, (kH, kW), stride=s, dilation=d).numpy()
        got = oracle.maxpool2d(X, (kH, kW), s, pads, d)
        assert got.shape == ref.shape and np.array_equal(got, ref), (ci, N, Cc, H, W, kH, kW, s, pads, d)
        ran += 1
    assert ran > 120
    # closed forms: a 1x1 window is the identity; a constant plane stays constant
    X = r.standard_normal((2, 3, 5, 6))
    assert np.array_equal(oracle.maxpool2d(X, (1, 1)), X)
    assert np.all(oracle.maxpool2d(np.full((1, 2, 7, 7), 2.5), (3, 3), (2, 2), (1, 1, 1, 1)) == 2.5)


def test_global_avgpool_against_torch_and_closed_forms():
    r = np.random.default_rng(707)
    X = r.standard_normal((3, 5, 7, 9))
    np.testing.assert_allclose(oracle.global_avgpool(X),
                               torch.from_numpy(X).mean(dim=(2, 3), keepdim=True).numpy(),
                               rtol=1e-14, atol=1e-14)
    assert np.all(oracle.global_avgpool(np.ones((2, 4, 7, 7))) == 1.0)
    # integer planes whose sums are exact: the mean is the exact quotient
    Xi = r.integers(-50, 50, (2, 3, 4, 4)).astype(np.float64)
    assert np.array_equal(oracle.global_avgpool(Xi)[..., 0, 0], Xi.sum(axis=(2, 3)) / 16.0)


def test_batchnorm_against_torch():
    r = np.random.default_rng(8)
    Y = r.standard_normal((2, 5, 4, 3))
    g, be, mu = r.uniform(0.5, 1.5, 5), r.standard_normal(5), r.standard_normal(5)
    var = r.uniform(0.5, 1.5, 5)
    out = oracle.batchnorm(Y, g, be, mu, var, 1e-5)
    ref = F.batch_norm(torch.from_numpy(Y), torch.from_numpy(mu), torch.from_numpy(var),
                       torch.from_numpy(g), torch.from_numpy(be), training=False, eps=1e-5).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("act", ["relu", "relu6", "none"])
def test_folded_conv_equals_unfused_conv_bn_act(act):
    # tensorforge "ResNet fusion": BN folded offline into the conv weights
    # (W' = scale*W, bias = shift) must equal Conv -> BN -> act.
    layer = synth.ConvLayer("t", 2, 6, 7, 7, 8, 3, 2, 1, 2, act)
    t = synth.conv_inputs(layer, 9, 0)
    b0 = np.random.default_rng(1).standard_normal(8)
    Wf, bf = oracle.fold_batchnorm(t["W"], t["gamma"], t["beta"], t["mean"], t["var"], 1e-5, b0)
    fused = oracle.conv2d(t["X"], Wf, bf, (2, 2), (1, 1, 1, 1), (1, 1), 2, act)
    chain = oracle.conv2d(t["X"], t["W"], b0, (2, 2), (1, 1, 1, 1), (1, 1), 2, "none")
    chain = oracle.act(act, oracle.batchnorm(chain, t["gamma"], t["beta"], t["mean"], t["var"], 1e-5))
    np.testing.assert_allclose(fused, chain, rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------------- int8 --

def test_int8_conv_acc_equals_float64_conv_of_shifted_inputs():
    r = np.random.default_rng(12)
    xq = r.integers(-128, 128, (2, 4, 6, 7)).astype(np.int8)
    wq = r.integers(-127, 128, (6, 2, 3, 3)).astype(np.int8)
    bias = r.integers(-1000, 1000, 6).astype(np.int32)
    zp = -13
    acc, _ = oracle.conv2d_int8(xq, wq, bias, zp, 0.05, np.full(6, 0.004, np.float32), 0.3, 3,
                                (1, 2), (1, 2, 0, 1), (2, 1), 2)
    # padding contributes (x_zp - x_zp) = 0: pad the shifted input with zeros
    ref = torch_conv(xq.astype(np.float64) - zp, wq.astype(np.float64), bias.astype(np.float64),
                     (1, 2), (1, 2, 0, 1), (2, 1), 2)
    assert np.array_equal(acc.astype(np.float64), ref)


def test_int8_k_term_identity():
    # onnx-vulkan-rs design notes: the zero-point correction
    # sum (a-az)(b-bz) = sum ab - az*sum b - bz*sum a + K*az*bz, here with
    # symmetric weights (bz = 0) over a Gemm.
    r = np.random.default_rng(13)
    xq = r.integers(-128, 128, (9, 40)).astype(np.int8)
    wq = r.integers(-127, 128, (5, 40)).astype(np.int8)
    zx = 17
    acc, _ = oracle.gemm_int8(xq, wq, None, zx, 0.1, np.full(5, 0.01, np.float32), 1.0, 0)
    x64, w64 = xq.astype(np.int64), wq.astype(np.int64)
    expanded = x64 @ w64.T - zx * w64.sum(1)[None, :]
    assert np.array_equal(acc, expanded)


def test_int8_requant_ties_round_half_to_even():
    # x_s = 2^-4, w_s = 2^-3, y_s = 2^-6: the multiplier is exactly 1/2, so
    # every odd accumulator is a tie.
    xs, ws, ys = 2.0 ** -4, 2.0 ** -3, 2.0 ** -6
    got = [oracle.requant1(a, xs, ws, ys, 0) for a in (1, 3, 5, -1, -3, -5)]
    assert got == [0, 2, 2, 0, -2, -2]       # half away from zero would give 1, 2, 3, -1, -2, -3
    assert [oracle.requant1(a, xs, ws, ys, 7) for a in (1, 3)] == [7, 9]


def test_int8_requant_saturates():
    xs, ws, ys = 2.0 ** -4, 2.0 ** -3, 2.0 ** -6     # multiplier 1/2
    # acc*M >= 127.5 - y_zp -> 127 ; <= -128.5 - y_zp -> -128
    assert oracle.requant1(2 * 127 - 2 * 5, xs, ws, ys, 5) == 127      # 122 + 5
    assert oracle.requant1(2 * 123, xs, ws, ys, 5) == 127              # 123 + 5 = 128 -> 127
    assert oracle.requant1(-2 * 133, xs, ws, ys, 5) == -128
    assert oracle.requant1(-2 * 133 + 2, xs, ws, ys, 5) == -127


def test_int8_padding_with_constant_zero_point_gives_bias():
    zp = 11
    xq = np.full((1, 3, 4, 5), zp, np.int8)
    wq = np.random.default_rng(0).integers(-127, 128, (4, 3, 5, 5)).astype(np.int8)
    bias = np.array([5, -7, 0, 123456], np.int32)
    acc, _ = oracle.conv2d_int8(xq, wq, bias, zp, 0.1, np.full(4, 0.01, np.float32), 1.0, 0,
                                (1, 1), (3, 3, 3, 3))
    assert np.array_equal(acc, np.broadcast_to(bias[None, :, None, None].astype(np.int64), acc.shape))


def test_int8_gemm_against_numpy_int64_and_requant_outputs():
    layer = synth.Int8Layer("t", "gemm", 37, 96, 24)
    t = synth.int8_inputs(layer, 4, 99)
    acc, y = oracle.gemm_int8(t["xq"], t["wq"], t["bias_q"], t["x_zp"], t["x_s"], t["w_s"],
                              t["y_s"], t["y_zp"])
    ref = (t["xq"].astype(np.int64) - t["x_zp"]) @ t["wq"].astype(np.int64).T + t["bias_q"][None, :]
    assert np.array_equal(acc, ref)
    # each output equals the single-accumulator requantisation of its acc
    for (i, j) in [(0, 0), (5, 7), (36, 23), (12, 3)]:
        assert y[i, j] == oracle.requant1(acc[i, j], t["x_s"], t["w_s"][j], t["y_s"], t["y_zp"])
    assert y.min() >= -128 and y.max() <= 127


def test_int8_accumulator_range_is_asserted():
    xq = np.full((1, 70000), -128, np.int8)
    wq = np.full((1, 70000), 127, np.int8)
    with pytest.raises(oracle.OracleError) as e:
        oracle.gemm_int8(xq, wq, None, 127, 0.1, np.ones(1, np.float32), 1.0, 0)
    assert e.value.code == oracle.ERANGE



def _np_requant(acc, x_s, w_s, y_s, y_zp, axis, lo=-128, hi=127):
    # The requantisation written out with numpy, independent of the oracle's C
    # code: multiplier (x_s * w_s[m]) / y_s in float64 in that order, the
    # accumulator times it, numpy's rint (half to even), + y_zp, saturate.
    mult = (np.float64(np.float32(x_s)) * np.asarray(w_s, np.float32).astype(np.float64)) \
        / np.float64(np.float32(y_s))
    shape = [1] * acc.ndim
    shape[axis] = -1
    v = acc.astype(np.float64) * mult.reshape(shape)
    return np.clip(np.rint(v) + y_zp, lo, hi).astype(np.int64)


def _distinct_scales(n, seed):
    # per-channel weight scales that differ from channel to channel, drawn as
    # the int8 workloads draw them (U[1e-3, 1e-2]), widened so that no two are
    # close: a requantisation that takes another channel's scale changes
    # many outputs
    ws = np.random.default_rng(seed).permutation(np.linspace(1e-3, 1e-2, n))
    return ws.astype(np.float32)


def test_int8_conv_requant_uses_each_output_channels_scale():
    # the requantised y of conv2d_int8, element by element, against the
    # numpy requantisation with w_s[m] of its own channel m (stride, pads and
    # a ragged channel count)
    layer = synth.Int8Layer("t", "conv", 1, 27, 11,
                            synth.ConvLayer("t", 2, 3, 9, 7, 11, 3, 2, 1, 1, "none"))
    t = synth.int8_inputs(layer, 4, 98)
    ws = _distinct_scales(11, 5)
    acc, y = oracle.conv2d_int8(t["xq"], t["wq"], t["bias_q"], t["x_zp"], t["x_s"], ws,
                                t["y_s"], t["y_zp"], (2, 2), (1, 1, 1, 1))
    ref = _np_requant(acc, t["x_s"], ws, t["y_s"], t["y_zp"], axis=1)
    assert np.array_equal(y.astype(np.int64), ref)
    # the channels' outputs really differ in scale: the same accumulator
    # requantised with a neighbour's scale gives other bytes somewhere
    assert not np.array_equal(ref, _np_requant(acc, t["x_s"], np.roll(ws, 1), t["y_s"],
                                               t["y_zp"], axis=1))


def test_qconv_requant_uses_each_output_channels_scale():
    # qconv2d with uint8 activations and outputs, per-channel weight zero
    # points and per-channel scales, in groups (each group's channels carry
    # their own scale)
    r = np.random.default_rng(36)
    x = r.integers(0, 256, (2, 4, 6, 7))
    w = r.integers(-128, 128, (6, 2, 3, 3))
    wz = r.integers(-128, 128, 6)
    bias = r.integers(-3000, 3000, 6).astype(np.int32)
    ws = _distinct_scales(6, 6)
    for unsigned, y_zp in ((False, -7), (True, 131)):
        acc, y = oracle.qconv2d(x, w, bias, 141, wz, 0.05, ws, 1.9, y_zp, unsigned,
                                (1, 2), (1, 2, 0, 1), (2, 1), 2)
        lo, hi = (0, 255) if unsigned else (-128, 127)
        ref = _np_requant(acc, 0.05, ws, 1.9, y_zp, axis=1, lo=lo, hi=hi)
        assert np.array_equal(y.astype(np.int64), ref)


def test_qgemm_requant_uses_each_output_columns_scale():
    # qgemm: column j of Y takes w_s[j]; int8 and uint8 outputs
    r = np.random.default_rng(37)
    x = r.integers(-128, 128, (13, 40))
    w = r.integers(-127, 128, (9, 40))
    wz = r.integers(-128, 128, 9)
    bias = r.integers(-2000, 2000, 9).astype(np.int32)
    ws = _distinct_scales(9, 7)
    for unsigned, y_zp in ((False, 3), (True, 120)):
        acc, y = oracle.qgemm(x, w, bias, -11, wz, 0.04, ws, 2.3, y_zp, unsigned)
        lo, hi = (0, 255) if unsigned else (-128, 127)
        ref = _np_requant(acc, 0.04, ws, 2.3, y_zp, axis=1, lo=lo, hi=hi)
        assert np.array_equal(y.astype(np.int64), ref)


def test_int8_gemm_requant_all_outputs_against_numpy():
    # every output of gemm_int8 (not only sampled ones) against the numpy
    # requantisation with its column's scale
    layer = synth.Int8Layer("t", "gemm", 37, 96, 24)
    t = synth.int8_inputs(layer, 4, 99)
    acc, y = oracle.gemm_int8(t["xq"], t["wq"], t["bias_q"], t["x_zp"], t["x_s"], t["w_s"],
                              t["y_s"], t["y_zp"])
    ref = _np_requant(acc, t["x_s"], t["w_s"], t["y_s"], t["y_zp"], axis=1)
    assert np.array_equal(y.astype(np.int64), ref)


# ---------------------------- uint8 activations, asymmetric weight zero points --

def test_qconv_acc_equals_float64_conv_of_both_shifted_operands():
    # uint8 activations, per-channel weight zero points: every product is
    # (x - x_zp)(w - w_zp[m]); the padding holds x_zp, i.e. zero after the shift
    r = np.random.default_rng(31)
    x = r.integers(0, 256, (2, 4, 6, 7))
    w = r.integers(-128, 128, (6, 2, 3, 3))
    wz = r.integers(-128, 128, 6)
    bias = r.integers(-1000, 1000, 6).astype(np.int32)
    zx = 141
    acc, _ = oracle.qconv2d(x, w, bias, zx, wz, 0.05, np.full(6, 0.004, np.float32), 0.3, 3,
                            False, (1, 2), (1, 2, 0, 1), (2, 1), 2)
    ref = torch_conv(x.astype(np.float64) - zx, w.astype(np.float64) - wz[:, None, None, None],
                     bias.astype(np.float64), (1, 2), (1, 2, 0, 1), (2, 1), 2)
    assert np.array_equal(acc.astype(np.float64), ref)


def test_qgemm_four_term_identity():
    # onnx-vulkan-rs design notes, the zero-point correction in full:
    # sum (a-az)(b-bz) = sum ab - az*sum b - bz*sum a + K*az*bz, with a
    # per-channel bz over a Gemm on uint8 activations
    r = np.random.default_rng(32)
    K = 72
    x = r.integers(0, 256, (11, K))
    w = r.integers(-128, 128, (7, K))
    wz = r.integers(-128, 128, 7)
    zx = 200
    acc, _ = oracle.qgemm(x, w, None, zx, wz, 0.1, np.full(7, 0.01, np.float32), 1.0, 0)
    x64, w64 = x.astype(np.int64), w.astype(np.int64)
    four = (x64 @ w64.T - zx * w64.sum(1)[None, :] - wz[None, :] * x64.sum(1)[:, None]
            + K * zx * wz[None, :])
    assert np.array_equal(acc, four)


def test_qconv_reduces_to_the_symmetric_int8_conv():
    # int8 activations with every weight zero point 0 is the symmetric case
    r = np.random.default_rng(33)
    x = r.integers(-128, 128, (1, 6, 5, 8)).astype(np.int8)
    w = r.integers(-127, 128, (4, 6, 3, 3)).astype(np.int8)
    bias = r.integers(-500, 500, 4).astype(np.int32)
    ws = np.full(4, 0.003, np.float32)
    acc0, y0 = oracle.conv2d_int8(x, w, bias, -9, 0.04, ws, 0.2, -3, (2, 1), (1, 1, 1, 1))
    acc1, y1 = oracle.qconv2d(x, w, bias, -9, np.zeros(4, np.int32), 0.04, ws, 0.2, -3, False,
                              (2, 1), (1, 1, 1, 1))
    assert np.array_equal(acc0, acc1) and np.array_equal(y0.astype(np.int32), y1)


def test_qconv_uint8_shift_by_128_is_exact():
    # u - zu = (u - 128) - (zu - 128): uint8 activations equal int8 ones
    # offset by 128, zero point included (the identity the GPU path uses)
    r = np.random.default_rng(34)
    u = r.integers(0, 256, (2, 3, 7, 7))
    w = r.integers(-128, 128, (5, 3, 3, 3))
    wz = r.integers(-128, 128, 5)
    ws = np.full(5, 0.002, np.float32)
    a0, _ = oracle.qconv2d(u, w, None, 77, wz, 0.05, ws, 0.5, 0, False, (1, 1), (2, 0, 1, 1))
    a1, _ = oracle.qconv2d(u - 128, w, None, 77 - 128, wz, 0.05, ws, 0.5, 0, False, (1, 1), (2, 0, 1, 1))
    assert np.array_equal(a0, a1)


def test_q_uint8_output_range_and_rounding():
    # multiplier 1/2: ties round half to even, then + y_zp, clamp to [0, 255]
    xs, ws, ys = 2.0 ** -4, 2.0 ** -3, 2.0 ** -6
    x = np.array([[1], [3], [5], [-1], [-3], [400], [-400]])
    w = np.array([[1]])
    _, y = oracle.qgemm(x, w, None, 0, None, xs, np.array([ws], np.float32), ys, 128, True)
    assert y[:, 0].tolist() == [128, 130, 130, 128, 126, 255, 0]
    _, y = oracle.qgemm(x, w, None, 0, None, xs, np.array([ws], np.float32), ys, 0, True)
    assert y[:, 0].tolist() == [0, 2, 2, 0, 0, 200, 0]
    with pytest.raises(oracle.OracleError):
        oracle.qgemm(x, w, None, 0, None, xs, np.array([ws], np.float32), ys, 256, True)


# ----------------------------------------------------------- MatMulNBits --

def test_matmul_nbits_against_unpacked_weights():
    # the oracle unpacks B itself; here W is built from the unpacked q, zero
    # points and scales the generator drew, and multiplied with numpy
    for (M, N, K, zp) in [(3, 5, 64, True), (2, 7, 200, False), (1, 4, 31, True)]:
        t = synth.nbits_inputs(M, N, K, 100 + K, with_zp=zp, pow2_scales=False)
        got = oracle.matmul_nbits(t["A"], t["B"], t["scales"], K, t["zero_points"], t["bias"])
        blk = np.arange(K) // 32
        W = (t["q"].astype(np.float64) - t["zp"][:, blk]) * t["scales"].astype(np.float64)[:, blk]
        ref = t["A"] @ W.T + t["bias"][None, :]
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_matmul_nbits_nibble_order_and_zero_point_cases():
    # one weight at k = 1 (the high nibble of byte 0) and one at k = 34
    # (block 1, byte 1, low nibble); A picks them out
    N, K = 1, 64
    B = np.zeros((N, 2, 16), np.uint8)
    B[0, 0, 0] = 0x5 | (0xC << 4)          # k=0 -> 5, k=1 -> 12
    B[0, 1, 1] = 0x3                       # k=34 -> 3
    scales = np.array([[0.5, 2.0]], np.float32)
    zps = np.array([[0x8 | (0x1 << 4)]], np.uint8)     # block 0: 8, block 1: 1
    A = np.zeros((3, K))
    A[0, 1] = 1.0
    A[1, 34] = 1.0
    A[2, 0] = 1.0
    Y = oracle.matmul_nbits(A, B, scales, K, zps)
    assert Y[:, 0].tolist() == [(12 - 8) * 0.5, (3 - 1) * 2.0, (5 - 8) * 0.5]
    # default zero point 8: an all-8 B contributes nothing, leaving the bias
    B8 = np.full((2, 1, 16), 0x88, np.uint8)
    Y = oracle.matmul_nbits(np.ones((4, 32)), B8, np.ones((2, 1), np.float32), 32, None, [1.5, -2.0])
    assert np.array_equal(Y, np.tile([1.5, -2.0], (4, 1)))


# ------------------------------------------------- DynamicQuantizeLinear --

def test_dynamic_quantize_closed_forms():
    # [0, 255]: scale 1, zero point 0, y = x
    y, sc, zp = oracle.dynamic_quantize_linear(np.arange(256, dtype=np.float32))
    assert sc == np.float32(1) and zp == 0 and np.array_equal(y, np.arange(256))
    # all positive: the range is widened to 0, so zp = 0 and the maximum maps to 255
    y, sc, zp = oracle.dynamic_quantize_linear(np.array([2.0, 4.0, 5.1], np.float32))
    assert zp == 0 and y[-1] == 255 and sc == np.float32(np.float32(5.1) / np.float32(255))
    # all negative: zp = 255, the minimum maps to 0
    y, sc, zp = oracle.dynamic_quantize_linear(np.array([-3.0, -1.0], np.float32))
    assert zp == 255 and y[0] == 0
    # symmetric [-1, 1]: in exact arithmetic -lo/scale = 127.5; in fp32 the
    # scale 2/255 rounds up (0.0078431377...), so 1/scale is just below 127.5:
    # zp = 127, x = 1 -> 127 + 127 = 254, x = -1 -> -127 + 127 = 0 (a
    # computation in double would give 128 and 255 here)
    y, sc, zp = oracle.dynamic_quantize_linear(np.array([-1.0, 0.0, 1.0], np.float32))
    assert float(sc) > 2 / 255
    assert zp == 127 and y.tolist() == [0, 127, 254]
    # all zero (and empty): scale 0, zero point 0, y = 0
    y, sc, zp = oracle.dynamic_quantize_linear(np.zeros(5, np.float32))
    assert sc == 0 and zp == 0 and not y.any()
    assert oracle.dynamic_quantize_linear(np.zeros(0, np.float32))[1] == 0


def test_dynamic_quantize_round_trip_error_is_half_a_step():
    # dequantising gives x back within scale/2 (all values lie in the range)
    r = np.random.default_rng(41)
    x = (r.standard_normal(5000) * 3 + 0.7).astype(np.float32)
    y, sc, zp = oracle.dynamic_quantize_linear(x)
    back = (y.astype(np.float64) - zp) * np.float64(sc)
    assert np.max(np.abs(back - x)) <= np.float64(sc) * 0.5 * (1 + 1e-5)
    assert y.min() == 0 or y.max() == 255
    # the extremes map to the ends of the range (up to the zero point's rounding)
    assert y[np.argmax(x)] >= 254 and y[np.argmin(x)] <= 1


# ------------------------------------------------------------- determinism --

def test_bit_identical_for_any_thread_count():
    r = np.random.default_rng(21)
    X = r.standard_normal((2, 16, 13, 11))
    Wt = r.standard_normal((24, 8, 3, 3))
    prev = oracle.set_threads(1)
    try:
        y1 = oracle.conv2d(X, Wt, None, (1, 1), (1, 1, 1, 1), (1, 1), 2, "gelu")
        g1 = oracle.gemm(X.reshape(32, -1)[:, :72], Wt.reshape(24, -1), transB=True)
        oracle.set_threads(max(2, os.cpu_count() or 2))
        y2 = oracle.conv2d(X, Wt, None, (1, 1), (1, 1, 1, 1), (1, 1), 2, "gelu")
        g2 = oracle.gemm(X.reshape(32, -1)[:, :72], Wt.reshape(24, -1), transB=True)
    finally:
        oracle.set_threads(prev)
    assert np.array_equal(y1, y2) and np.array_equal(g1, g2)
