"""CPU oracle for the fused GEMM / implicit-GEMM convolution path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark import this package.  The product library
(libox, package ``conv_implicit_gemm_amd``) never imports it, and the two share
no code: this is a ctypes wrapper over ``liboxref.so`` (plain C, fp64), which
``oracle/build.py`` compiles with gcc.

Every function takes and returns numpy arrays.  Floating inputs are widened to
float64 exactly (fp32 and bf16 values are representable in float64); the
oracle's sums run in float64 in a fixed order.  What each function computes,
and the passage of the pages it follows, is stated in ``oxref.h``.
"""
import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboxref.so")

ACT = {"none": 0, "relu": 1, "relu6": 2, "gelu": 3}

OK, EARG, ESHAPE, ERANGE = 0, -1, -2, -3


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__("oracle %s returned %d" % (what, code))
        self.code = code


class _Conv(C.Structure):
    _fields_ = [(n, C.c_int64) for n in
                ("N", "C", "H", "W", "M", "kH", "kW", "s_h", "s_w",
                 "p_t", "p_l", "p_b", "p_r", "d_h", "d_w", "group")]


_lib = None


def lib():
    """Load liboxref.so (building it first if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        P, I64, I32, D, F = C.c_void_p, C.c_int64, C.c_int32, C.c_double, C.c_float
        sig = {
            "oxref_set_threads": (C.c_int, [C.c_int]),
            "oxref_get_threads": (C.c_int, []),
            "oxref_act1": (D, [C.c_int, D]),
            "oxref_act": (C.c_int, [C.c_int, I64, P]),
            "oxref_matmul": (C.c_int, [I64, I64, I64, I64, P, I64, P, I64, P]),
            "oxref_gemm": (C.c_int, [I64, I64, I64, C.c_int, C.c_int, D, P, P, D, P, C.c_int, P]),
            "oxref_gemm_at": (C.c_int, [I64, I64, I64, C.c_int, C.c_int, D, P, P, D, P, C.c_int,
                                        I64, P, P]),
            "oxref_conv_out_dims": (C.c_int, [P, P, P]),
            "oxref_conv2d": (C.c_int, [P, P, P, P, C.c_int, P]),
            "oxref_conv2d_at": (C.c_int, [P, P, P, P, C.c_int, I64, P, P]),
            "oxref_conv2d_res": (C.c_int, [P, P, P, P, P, C.c_int, P]),
            "oxref_conv2d_res_at": (C.c_int, [P, P, P, P, P, C.c_int, I64, P, P]),
            "oxref_batchnorm": (C.c_int, [I64, I64, I64, P, P, P, P, P, D]),
            "oxref_maxpool2d": (C.c_int, [P, P, P]),
            "oxref_global_avgpool": (C.c_int, [I64, I64, I64, P, P]),
            "oxref_fold_batchnorm": (C.c_int, [I64, I64, P, P, P, P, P, P, D, P, P]),
            "oxref_conv2d_int8": (C.c_int, [P, P, P, P, I32, F, P, F, I32, P, P]),
            "oxref_gemm_int8": (C.c_int, [I64, I64, I64, P, P, P, I32, F, P, F, I32, P, P]),
            "oxref_requant1": (I32, [I64, F, F, F, I32]),
            "oxref_qconv2d": (C.c_int, [P, P, P, P, I32, P, F, P, F, I32, I32, I32, P, P]),
            "oxref_qgemm": (C.c_int, [I64, I64, I64, P, P, P, I32, P, F, P, F, I32, I32, I32, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _check(rc, what):
    if rc != OK:
        raise OracleError(rc, what)


def set_threads(n):
    """Set the OpenMP thread count; returns the previous maximum."""
    return lib().oxref_set_threads(int(n))


def get_threads():
    return lib().oxref_get_threads()


def act(name, v):
    """Apply an activation to an array (float64)."""
    v = _f64(v).copy()
    _check(lib().oxref_act(ACT[name], v.size, _p(v)), "act")
    return v


def matmul(A, B):
    """ONNX MatMul: A [batch,M,K] x B [batch,K,N] or [K,N] (broadcast) -> [batch,M,N]."""
    A = _f64(A)
    B = _f64(B)
    batch, M, K = A.shape
    if B.ndim == 2:
        sB = 0
        K2, N = B.shape
    else:
        assert B.shape[0] in (batch, 1)
        _, K2, N = B.shape
        sB = 0 if (B.shape[0] == 1 and batch != 1) else K2 * N
    assert K2 == K
    Cm = np.empty((batch, M, N), dtype=np.float64)
    _check(lib().oxref_matmul(batch, M, N, K, _p(A), M * K, _p(B), sB, _p(Cm)), "matmul")
    return Cm


def gemm(A, B, bias=None, alpha=1.0, beta=1.0, transA=False, transB=False,
         act="none", at=None):
    """ONNX Gemm + activation.  With ``at`` (flat output indices) only those
    outputs are computed and returned as a 1-D array."""
    A = _f64(A)
    B = _f64(B)
    bias = _f64(bias)
    M = A.shape[1] if transA else A.shape[0]
    K = A.shape[0] if transA else A.shape[1]
    N = B.shape[0] if transB else B.shape[1]
    assert (B.shape[1] if transB else B.shape[0]) == K, "A and B disagree on K"
    assert bias is None or bias.shape == (N,), "bias must have N elements"
    L = lib()
    if at is None:
        Y = np.empty((M, N), dtype=np.float64)
        _check(L.oxref_gemm(M, N, K, int(transA), int(transB), float(alpha), _p(A), _p(B),
                            float(beta), _p(bias), ACT[act], _p(Y)), "gemm")
        return Y
    idx = np.ascontiguousarray(np.asarray(at, dtype=np.int64))
    out = np.empty(idx.size, dtype=np.float64)
    _check(L.oxref_gemm_at(M, N, K, int(transA), int(transB), float(alpha), _p(A), _p(B),
                           float(beta), _p(bias), ACT[act], idx.size, _p(idx), _p(out)),
           "gemm_at")
    return out


def conv_desc(N, Cin, H, W, M, kH, kW, stride=(1, 1), pads=(0, 0, 0, 0),
              dilation=(1, 1), group=1):
    """Build the oracle's conv shape.  pads are ONNX order (top, left, bottom, right)."""
    d = _Conv()
    d.N, d.C, d.H, d.W, d.M, d.kH, d.kW = N, Cin, H, W, M, kH, kW
    d.s_h, d.s_w = stride
    d.p_t, d.p_l, d.p_b, d.p_r = pads
    d.d_h, d.d_w = dilation
    d.group = group
    return d


def conv_out_dims(d):
    ho, wo = C.c_int64(0), C.c_int64(0)
    rc = lib().oxref_conv_out_dims(C.byref(d), C.byref(ho), C.byref(wo))
    return rc, ho.value, wo.value


def conv2d(X, Wt, b=None, stride=(1, 1), pads=(0, 0, 0, 0), dilation=(1, 1),
           group=1, act="none", at=None, residual=None):
    """ONNX Conv (direct summation) + bias (+ residual) + activation.
    X [N,C,H,W], Wt [M,C/g,kH,kW]; residual, if given, has the output's
    shape [N,M,Ho,Wo] and is added after the bias, before the activation.
    With ``at`` only those flat output indices."""
    X = _f64(X)
    Wt = _f64(Wt)
    b = _f64(b)
    N, Cin, H, W = X.shape
    M, cpg, kH, kW = Wt.shape
    assert cpg * group == Cin, "weight channels do not match C/group"
    d = conv_desc(N, Cin, H, W, M, kH, kW, stride, pads, dilation, group)
    rc, Ho, Wo = conv_out_dims(d)
    _check(rc, "conv_out_dims")
    R = _f64(residual)
    if R is not None:
        assert R.shape == (N, M, Ho, Wo), "residual must have the output's shape"
    L = lib()
    if at is None:
        Y = np.empty((N, M, Ho, Wo), dtype=np.float64)
        _check(L.oxref_conv2d_res(C.byref(d), _p(X), _p(Wt), _p(b), _p(R), ACT[act], _p(Y)), "conv2d")
        return Y
    idx = np.ascontiguousarray(np.asarray(at, dtype=np.int64))
    out = np.empty(idx.size, dtype=np.float64)
    _check(L.oxref_conv2d_res_at(C.byref(d), _p(X), _p(Wt), _p(b), _p(R), ACT[act], idx.size,
                                 _p(idx), _p(out)), "conv2d_at")
    return out


def maxpool2d(X, kernel, stride=(1, 1), pads=(0, 0, 0, 0), dilation=(1, 1)):
    """ONNX MaxPool (ceil_mode 0) on X [N,C,H,W]; pads (top, left, bottom, right)."""
    X = _f64(X)
    N, Cc, H, W = X.shape
    d = conv_desc(N, Cc, H, W, Cc, kernel[0], kernel[1], stride, pads, dilation, 1)
    rc, Ho, Wo = conv_out_dims(d)
    _check(rc, "conv_out_dims")
    Y = np.empty((N, Cc, Ho, Wo), dtype=np.float64)
    _check(lib().oxref_maxpool2d(C.byref(d), _p(X), _p(Y)), "maxpool2d")
    return Y


def global_avgpool(X):
    """ONNX GlobalAveragePool: X [N,C,H,W] -> [N,C,1,1]."""
    X = _f64(X)
    N, Cc = X.shape[:2]
    HW = int(np.prod(X.shape[2:]))
    Y = np.empty((N, Cc, 1, 1), dtype=np.float64)
    _check(lib().oxref_global_avgpool(N, Cc, HW, _p(X), _p(Y)), "global_avgpool")
    return Y


def batchnorm_act(X, gamma, beta, mean, var, eps=1e-5, act="none"):
    """Unfused inference BatchNormalization followed by an activation."""
    return globals()["act"](act, batchnorm(X, gamma, beta, mean, var, eps))


def batchnorm(Y, gamma, beta, mean, var, eps=1e-5):
    """ONNX BatchNormalization (inference) on Y [N,M,...] (returns a new array)."""
    Y = _f64(Y).copy()
    N, M = Y.shape[0], Y.shape[1]
    HW = int(np.prod(Y.shape[2:])) if Y.ndim > 2 else 1
    g, bt, mu, v = (_f64(t) for t in (gamma, beta, mean, var))
    _check(lib().oxref_batchnorm(N, M, HW, _p(Y), _p(g), _p(bt), _p(mu), _p(v), float(eps)),
           "batchnorm")
    return Y


def fold_batchnorm(Wt, gamma, beta, mean, var, eps=1e-5, b0=None):
    """Offline BatchNorm fold in float64: returns (W', b') with W' shaped like Wt."""
    Wt = _f64(Wt)
    M = Wt.shape[0]
    Kper = int(Wt.size // M)
    g, bt, mu, v = (_f64(t) for t in (gamma, beta, mean, var))
    b0 = _f64(b0)
    Wo = np.empty_like(Wt)
    bo = np.empty(M, dtype=np.float64)
    _check(lib().oxref_fold_batchnorm(M, Kper, _p(Wt), _p(b0), _p(g), _p(bt), _p(mu), _p(v),
                                      float(eps), _p(Wo), _p(bo)), "fold_batchnorm")
    return Wo, bo


def _i8(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int8))


def conv2d_int8(Xq, Wq, bias_q, x_zp, x_s, w_s, y_s, y_zp, stride=(1, 1),
                pads=(0, 0, 0, 0), dilation=(1, 1), group=1):
    """Static int8 conv: returns (acc int64 [N,M,Ho,Wo], y int8 [N,M,Ho,Wo])."""
    Xq = _i8(Xq)
    Wq = _i8(Wq)
    N, Cin, H, W = Xq.shape
    M, cpg, kH, kW = Wq.shape
    d = conv_desc(N, Cin, H, W, M, kH, kW, stride, pads, dilation, group)
    rc, Ho, Wo = conv_out_dims(d)
    _check(rc, "conv_out_dims")
    bq = None if bias_q is None else np.ascontiguousarray(np.asarray(bias_q, dtype=np.int32))
    ws = np.ascontiguousarray(np.asarray(w_s, dtype=np.float32))
    acc = np.empty((N, M, Ho, Wo), dtype=np.int64)
    y = np.empty((N, M, Ho, Wo), dtype=np.int8)
    _check(lib().oxref_conv2d_int8(C.byref(d), _p(Xq), _p(Wq), _p(bq), int(x_zp),
                                   float(np.float32(x_s)), _p(ws), float(np.float32(y_s)),
                                   int(y_zp), _p(acc), _p(y)), "conv2d_int8")
    return acc, y


def gemm_int8(Xq, Wq, bias_q, x_zp, x_s, w_s, y_s, y_zp):
    """Static int8 Gemm, X [M,K], W [N,K]: returns (acc int64 [M,N], y int8 [M,N])."""
    Xq = _i8(Xq)
    Wq = _i8(Wq)
    M, K = Xq.shape
    N = Wq.shape[0]
    bq = None if bias_q is None else np.ascontiguousarray(np.asarray(bias_q, dtype=np.int32))
    ws = np.ascontiguousarray(np.asarray(w_s, dtype=np.float32))
    acc = np.empty((M, N), dtype=np.int64)
    y = np.empty((M, N), dtype=np.int8)
    _check(lib().oxref_gemm_int8(M, N, K, _p(Xq), _p(Wq), _p(bq), int(x_zp),
                                 float(np.float32(x_s)), _p(ws), float(np.float32(y_s)),
                                 int(y_zp), _p(acc), _p(y)), "gemm_int8")
    return acc, y


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _yrange(y_unsigned):
    return (0, 255) if y_unsigned else (-128, 127)


def qconv2d(X, Wq, bias_q, x_zp, w_zp, x_s, w_s, y_s, y_zp, y_unsigned=False, stride=(1, 1),
            pads=(0, 0, 0, 0), dilation=(1, 1), group=1):
    """Quantised conv with activation and per-channel weight zero points
    (int8 or uint8 stored integers): returns (acc int64, y int32 holding int8
    or uint8 values), both [N,M,Ho,Wo]."""
    X = _i32(X)
    Wq = _i32(Wq)
    N, Cin, H, W = X.shape
    M, _, kH, kW = Wq.shape
    d = conv_desc(N, Cin, H, W, M, kH, kW, stride, pads, dilation, group)
    rc, Ho, Wo = conv_out_dims(d)
    _check(rc, "conv_out_dims")
    bq = None if bias_q is None else _i32(bias_q)
    wz = None if w_zp is None else _i32(w_zp)
    ws = np.ascontiguousarray(np.asarray(w_s, dtype=np.float32))
    lo, hi = _yrange(y_unsigned)
    acc = np.empty((N, M, Ho, Wo), dtype=np.int64)
    y = np.empty((N, M, Ho, Wo), dtype=np.int32)
    _check(lib().oxref_qconv2d(C.byref(d), _p(X), _p(Wq), _p(bq), int(x_zp), _p(wz),
                               float(np.float32(x_s)), _p(ws), float(np.float32(y_s)), int(y_zp),
                               lo, hi, _p(acc), _p(y)), "qconv2d")
    return acc, y


def qgemm(X, Wq, bias_q, x_zp, w_zp, x_s, w_s, y_s, y_zp, y_unsigned=False):
    """Quantised Gemm X [M,K] x W [N,K] with both zero points: returns
    (acc int64 [M,N], y int32 [M,N] holding int8 or uint8 values)."""
    X = _i32(X)
    Wq = _i32(Wq)
    M, K = X.shape
    N = Wq.shape[0]
    bq = None if bias_q is None else _i32(bias_q)
    wz = None if w_zp is None else _i32(w_zp)
    ws = np.ascontiguousarray(np.asarray(w_s, dtype=np.float32))
    lo, hi = _yrange(y_unsigned)
    acc = np.empty((M, N), dtype=np.int64)
    y = np.empty((M, N), dtype=np.int32)
    _check(lib().oxref_qgemm(M, N, K, _p(X), _p(Wq), _p(bq), int(x_zp), _p(wz),
                             float(np.float32(x_s)), _p(ws), float(np.float32(y_s)), int(y_zp),
                             lo, hi, _p(acc), _p(y)), "qgemm")
    return acc, y


def matmul_nbits(A, B, scales, K, zero_points=None, bias=None):
    """Weight-only 4-bit MatMul (ONNX MatMulNBits, blocks of 32 along K; the
    Onyxia README's q4 weights): Y = A x W^T (+ bias) in float64 with
    W[n,k] = (q[n,k] - zp[n,k//32]) * scales[n,k//32], where q[n,k] is the low
    nibble of byte (k%32)//2 of block k//32 of row n for even k and the high
    nibble for odd k, and zp is block b's nibble of zero_points[n, b//2] (low
    for even b), or 8 when zero_points is None.  A: [M,K]; B: uint8
    [N, ceil(K/32), 16]; scales: [N, ceil(K/32)]."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.uint8)
    sc = np.asarray(scales, dtype=np.float64)
    N = B.shape[0]
    W = np.empty((N, K), dtype=np.float64)
    for k in range(K):
        b = k // 32
        byte = B[:, b, (k % 32) // 2].astype(np.int64)
        q = (byte & 15) if k % 2 == 0 else (byte >> 4)
        if zero_points is None:
            zp = 8
        else:
            zb = np.asarray(zero_points, dtype=np.uint8)[:, b // 2].astype(np.int64)
            zp = (zb & 15) if b % 2 == 0 else (zb >> 4)
        W[:, k] = (q - zp) * sc[:, b]
    Y = A @ W.T
    if bias is not None:
        Y = Y + np.asarray(bias, dtype=np.float64)[None, :]
    return Y


def dynamic_quantize_linear(x):
    """ONNX DynamicQuantizeLinear (the dynamically quantised graphs of the
    onnx-vulkan-rs notes), step by step in float32 as the operator defines it:
    the range [min(0, min x), max(0, max x)], y_scale = range / 255, the zero
    point -x_min / y_scale clamped to [0, 255] and rounded half to even, then
    y = clamp(rint(x / y_scale) + y_zp, 0, 255).  Reading: an all-zero (or
    empty) x gives y_scale = 0, y_zp = 0 and y = 0.  Returns (y uint8,
    y_scale float32, y_zp int)."""
    x = np.asarray(x, dtype=np.float32)
    f = np.float32
    x_min = f(min(f(0), x.min())) if x.size else f(0)
    x_max = f(max(f(0), x.max())) if x.size else f(0)
    y_scale = f(f(x_max - x_min) / f(255))
    if y_scale == 0:
        return np.zeros(x.shape, np.uint8), y_scale, 0
    zp = f(np.rint(np.clip(f(f(0) - f(x_min / y_scale)), f(0), f(255))))
    q = np.rint((x / y_scale).astype(np.float32)).astype(np.float32) + zp
    y = np.clip(q, f(0), f(255)).astype(np.uint8)
    return y, y_scale, int(zp)


def requant1(acc, x_s, w_s, y_s, y_zp):
    """The oracle's requantisation of a single accumulator."""
    return lib().oxref_requant1(int(acc), float(np.float32(x_s)), float(np.float32(w_s)),
                                float(np.float32(y_s)), int(y_zp))
