"""conv_implicit_gemm_amd -- Python binding of libox, the MI355X (gfx950) fused
GEMM / implicit-GEMM convolution library.

A thin ctypes layer over the C ABI declared in include/ox.h: each function
here has the name of the C entry point it calls and does argument marshalling
only (shapes from tensors, ``data_ptr()``, the current HIP stream).  Every
step of the computation runs in the library's own HIP kernels; PyTorch only
supplies device memory and the stream.  There is no CPU fallback: if libox.so
cannot be loaded, importing this package fails.
"""
import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libox.so")

OX_OK, OX_ERR_INVALID_ARG, OX_ERR_SHAPE, OX_ERR_UNSUPPORTED, OX_ERR_HIP = 0, 1, 2, 3, 4
OX_F32, OX_BF16, OX_I8, OX_I32 = 0, 1, 2, 3
ACT = {"none": 0, "relu": 1, "relu6": 2, "gelu": 3}
STATUS_NAMES = {0: "OX_OK", 1: "OX_ERR_INVALID_ARG", 2: "OX_ERR_SHAPE",
                3: "OX_ERR_UNSUPPORTED", 4: "OX_ERR_HIP"}

# every symbol include/ox.h declares
EXPORTS = ("ox_matmul_batched", "ox_gemm_fused", "ox_conv2d_fused", "ox_conv2d_int8",
           "ox_conv2d_variant", "ox_conv2d_fused_packed", "ox_conv2d_packed_weights_bytes",
           "ox_conv2d_pack_weights", "ox_fold_batchnorm", "ox_int8_params_bytes", "ox_int8_prepare",
           "ox_last_error", "ox_version", "ox_conv2d_workspace_bytes", "ox_conv2d_fused_ws",
           "ox_conv2d_fused_res", "ox_batchnorm_act", "ox_maxpool2d", "ox_global_avgpool",
           "ox_int8_prepare_ex", "ox_dynamic_quantize_workspace_bytes", "ox_dynamic_quantize_linear",
           "ox_matmul_nbits", "ox_gemm_workspace_bytes", "ox_gemm_fused_ws",
           "ox_static_scratch_bytes", "ox_conv2d_fused_static")


class OxError(RuntimeError):
    """A non-OX_OK status from libox, with the library's message."""

    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status
        self.message = message


class ConvDesc(C.Structure):
    """ox_conv_desc (pads in the ONNX order top, left, bottom, right)."""
    _fields_ = [(n, C.c_int64) for n in
                ("N", "C", "H", "W", "M", "kH", "kW", "s_h", "s_w",
                 "p_t", "p_l", "p_b", "p_r", "d_h", "d_w", "group")]


def _load():
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    L = C.CDLL(LIB_PATH)
    P, I64, I32, F, I = C.c_void_p, C.c_int64, C.c_int32, C.c_float, C.c_int
    sig = {
        "ox_matmul_batched": (I, [I, I64, I64, I64, I64, P, I64, P, I64, P, P]),
        "ox_gemm_fused": (I, [I, I64, I64, I64, I, I, F, P, P, F, P, I, P, P, P]),
        "ox_conv2d_fused": (I, [I, P, P, P, P, I, P, P]),
        "ox_conv2d_int8": (I, [P, P, P, P, I, P, P]),
        "ox_conv2d_variant": (I, [I, P, C.c_char_p, C.c_size_t]),
        "ox_conv2d_fused_packed": (I, [I, P, P, P, P, I, P, P]),
        "ox_conv2d_packed_weights_bytes": (C.c_size_t, [I, P]),
        "ox_conv2d_workspace_bytes": (C.c_size_t, [I, P]),
        "ox_conv2d_fused_ws": (I, [I, P, P, P, I, P, I, P, P, C.c_size_t, P]),
        "ox_conv2d_fused_static": (I, [I, P, P, P, I, P, I, P, P]),
        "ox_static_scratch_bytes": (C.c_size_t, []),
        "ox_conv2d_fused_res": (I, [I, P, P, P, P, P, I, P, P, C.c_size_t, P]),
        "ox_batchnorm_act": (I, [I, I64, I64, I64, P, P, P, P, P, F, I, P, P]),
        "ox_maxpool2d": (I, [I, P, P, P, P]),
        "ox_global_avgpool": (I, [I, I64, I64, I64, P, P, P]),
        "ox_conv2d_pack_weights": (I, [I, P, P, P]),
        "ox_fold_batchnorm": (I, [I64, I64, P, P, P, P, P, P, F, P, P]),
        "ox_int8_params_bytes": (C.c_size_t, [I64]),
        "ox_int8_prepare": (I, [I64, I64, P, P, F, I32, F, I32, P, P]),
        "ox_int8_prepare_ex": (I, [I64, I64, P, P, P, F, I32, I, F, I32, I, P, P]),
        "ox_dynamic_quantize_workspace_bytes": (C.c_size_t, []),
        "ox_matmul_nbits": (I, [I, I64, I64, I64, I, I, P, P, P, P, P, P, P]),
        "ox_gemm_workspace_bytes": (C.c_size_t, [I, I64, I64, I64]),
        "ox_gemm_fused_ws": (I, [I, I64, I64, I64, I, I, F, P, P, F, P, I, P, P, C.c_size_t, P]),
        "ox_dynamic_quantize_linear": (I, [I64, P, P, P, P, P, C.c_size_t, P]),
        "ox_last_error": (C.c_char_p, []),
        "ox_version": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def ox_last_error():
    return lib.ox_last_error().decode()


def ox_version():
    return lib.ox_version().decode()


def _check(status):
    if status != OX_OK:
        raise OxError(status, ox_last_error())


# ------------------------------------------------------------- marshalling --

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    # uint8 tensors travel as bytes through the int8 calls: the parameter
    # block (ox_int8_prepare(..., x_unsigned / y_unsigned)) says how to read them
    m = {torch.float32: OX_F32, torch.bfloat16: OX_BF16, torch.int8: OX_I8, torch.uint8: OX_I8,
         torch.int32: OX_I32}
    if t.dtype not in m:
        raise TypeError("unsupported tensor dtype %s" % t.dtype)
    return m[t.dtype]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _dense(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError("%s must be contiguous (dense row-major)" % name)


def conv_desc(N, Cin, H, W, M, kH, kW, stride=(1, 1), pads=(0, 0, 0, 0), dilation=(1, 1), group=1):
    d = ConvDesc()
    d.N, d.C, d.H, d.W, d.M, d.kH, d.kW = N, Cin, H, W, M, kH, kW
    d.s_h, d.s_w = stride
    d.p_t, d.p_l, d.p_b, d.p_r = pads
    d.d_h, d.d_w = dilation
    d.group = group
    return d


def conv_out_hw(H, W, kH, kW, stride=(1, 1), pads=(0, 0, 0, 0), dilation=(1, 1)):
    t, l, b, r = pads
    ho = (H + t + b - dilation[0] * (kH - 1) - 1) // stride[0] + 1
    wo = (W + l + r - dilation[1] * (kW - 1) - 1) // stride[1] + 1
    return ho, wo


# ----------------------------------------------------------------- hot path --

def ox_matmul_batched(A, B, C_out=None, stream=None):
    """ONNX MatMul: A [batch,M,K] x B [batch,K,N] (or [K,N] broadcast) -> [batch,M,N]."""
    torch = _torch()
    _dense(A, "A")
    _dense(B, "B")
    batch, M, K = A.shape
    if B.dim() == 2:
        K2, N = B.shape
        sB = 0
    else:
        bb, K2, N = B.shape
        sB = 0 if (bb == 1 and batch != 1) else K2 * N
    if C_out is None:
        C_out = torch.empty((batch, M, N), dtype=A.dtype, device=A.device)
    _dense(C_out, "C")
    _check(lib.ox_matmul_batched(_dtype_code(A), batch, M, N, K, _ptr(A), M * K, _ptr(B), sB,
                                 _ptr(C_out), _stream(stream)))
    return C_out


def ox_gemm_fused(A, B, bias=None, alpha=1.0, beta=1.0, transA=False, transB=False, act="none",
                  Y=None, int8_params=None, out_dtype=None, stream=None):
    """ONNX Gemm + activation.  Float: A, B, bias, Y of one dtype.  int8: A = x_q [M,K],
    B = w_q [N,K] (transB=True), int8_params = device block, out_dtype int8 or int32."""
    torch = _torch()
    for t, n in ((A, "A"), (B, "B"), (bias, "bias"), (Y, "Y")):
        _dense(t, n)
    M = A.shape[1] if transA else A.shape[0]
    K = A.shape[0] if transA else A.shape[1]
    N = B.shape[0] if transB else B.shape[1]
    code = _dtype_code(A)
    if code == OX_I8:
        out_dtype = out_dtype or torch.int8
        code = OX_I32 if out_dtype == torch.int32 else OX_I8
    else:
        out_dtype = A.dtype
    if Y is None:
        Y = torch.empty((M, N), dtype=out_dtype, device=A.device)
    _check(lib.ox_gemm_fused(code, M, N, K, int(transA), int(transB), float(alpha), _ptr(A), _ptr(B),
                             float(beta), _ptr(bias), ACT[act], _ptr(Y), _ptr(int8_params),
                             _stream(stream)))
    return Y


def ox_gemm_workspace_bytes(dtype, M, N, K):
    code = {"f32": OX_F32, "bf16": OX_BF16}[dtype]
    return int(lib.ox_gemm_workspace_bytes(code, M, N, K))


def ox_gemm_fused_ws(A, B, workspace, bias=None, alpha=1.0, beta=1.0, transA=False, transB=False,
                     act="none", Y=None, stream=None):
    """Float Gemm + activation with a split-K workspace (see ox_gemm_workspace_bytes)."""
    torch = _torch()
    for t, n in ((A, "A"), (B, "B"), (bias, "bias"), (Y, "Y"), (workspace, "workspace")):
        _dense(t, n)
    M = A.shape[1] if transA else A.shape[0]
    K = A.shape[0] if transA else A.shape[1]
    N = B.shape[0] if transB else B.shape[1]
    if Y is None:
        Y = torch.empty((M, N), dtype=A.dtype, device=A.device)
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.ox_gemm_fused_ws(_dtype_code(A), M, N, K, int(transA), int(transB), float(alpha),
                                _ptr(A), _ptr(B), float(beta), _ptr(bias), ACT[act], _ptr(Y),
                                _ptr(workspace), nb, _stream(stream)))
    return Y


def ox_conv2d_fused(X, W, bias=None, stride=(1, 1), pads=(0, 0, 0, 0), dilation=(1, 1), group=1,
                    act="none", Y=None, stream=None, workspace=None):
    """ONNX Conv + bias + activation (NCHW).  W is [M, C/group, kH, kW].
    workspace: optional device tensor of >= ox_conv2d_workspace_bytes bytes
    (enables split-K; goes through ox_conv2d_fused_ws)."""
    torch = _torch()
    for t, n in ((X, "X"), (W, "W"), (bias, "bias"), (Y, "Y")):
        _dense(t, n)
    N, Cin, H, Wd = X.shape
    M, _, kH, kW = W.shape
    d = conv_desc(N, Cin, H, Wd, M, kH, kW, stride, pads, dilation, group)
    if Y is None:
        ho, wo = conv_out_hw(H, Wd, kH, kW, stride, pads, dilation)
        Y = torch.empty((N, M, max(ho, 0), max(wo, 0)), dtype=X.dtype, device=X.device)
    if workspace is not None:
        _dense(workspace, "workspace")
        nbytes = workspace.numel() * workspace.element_size()
        _check(lib.ox_conv2d_fused_ws(_dtype_code(X), C.byref(d), _ptr(X), _ptr(W), 0, _ptr(bias),
                                      ACT[act], _ptr(Y), _ptr(workspace), nbytes, _stream(stream)))
    else:
        _check(lib.ox_conv2d_fused(_dtype_code(X), C.byref(d), _ptr(X), _ptr(W), _ptr(bias), ACT[act],
                                   _ptr(Y), _stream(stream)))
    return Y


def ox_conv2d_fused_res(X, W, R, bias=None, stride=(1, 1), pads=(0, 0, 0, 0), dilation=(1, 1),
                        group=1, act="none", Y=None, stream=None, workspace=None):
    """ONNX Conv + bias + residual R (the output's shape) + activation, fused:
    Y = act(conv(X, W) + bias + R).  Y may be R itself (in place)."""
    torch = _torch()
    for t, n in ((X, "X"), (W, "W"), (R, "R"), (bias, "bias"), (Y, "Y")):
        _dense(t, n)
    N, Cin, H, Wd = X.shape
    M, _, kH, kW = W.shape
    d = conv_desc(N, Cin, H, Wd, M, kH, kW, stride, pads, dilation, group)
    if Y is None:
        ho, wo = conv_out_hw(H, Wd, kH, kW, stride, pads, dilation)
        Y = torch.empty((N, M, max(ho, 0), max(wo, 0)), dtype=X.dtype, device=X.device)
    nbytes = 0
    if workspace is not None:
        _dense(workspace, "workspace")
        nbytes = workspace.numel() * workspace.element_size()
    _check(lib.ox_conv2d_fused_res(_dtype_code(X), C.byref(d), _ptr(X), _ptr(W), _ptr(bias), _ptr(R),
                                   ACT[act], _ptr(Y), _ptr(workspace), nbytes, _stream(stream)))
    return Y


def ox_matmul_nbits(A, B, scales, K, zero_points=None, bias=None, Y=None, stream=None):
    """MatMulNBits (4 bits, blocks of 32): A bf16 [M,K] x dequant(B)^T -> Y bf16 [M,N].
    B uint8 [N, ceil(K/32), 16], scales fp32 [N, ceil(K/32)], zero_points
    uint8 [N, ceil(ceil(K/32)/2)] or None (8)."""
    torch = _torch()
    for t, n in ((A, "A"), (B, "B"), (scales, "scales"), (zero_points, "zero_points"),
                 (bias, "bias"), (Y, "Y")):
        _dense(t, n)
    M = A.shape[0]
    N = B.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _check(lib.ox_matmul_nbits(OX_BF16, M, N, K, 4, 32, _ptr(A), _ptr(B), _ptr(scales),
                               _ptr(zero_points), _ptr(bias), _ptr(Y), _stream(stream)))
    return Y


def ox_dynamic_quantize_linear(X, Y=None, y_scale=None, y_zp=None, workspace=None, stream=None):
    """ONNX DynamicQuantizeLinear of a dense fp32 device tensor: returns
    (Y uint8 of X's shape, y_scale fp32 [1], y_zp uint8 [1]), all on the device."""
    torch = _torch()
    _dense(X, "X")
    if X.dtype != torch.float32:
        raise TypeError("X must be float32")
    if Y is None:
        Y = torch.empty(X.shape, dtype=torch.uint8, device=X.device)
    if y_scale is None:
        y_scale = torch.empty(1, dtype=torch.float32, device=X.device)
    if y_zp is None:
        y_zp = torch.empty(1, dtype=torch.uint8, device=X.device)
    if workspace is None:
        workspace = torch.empty(int(lib.ox_dynamic_quantize_workspace_bytes()), dtype=torch.uint8,
                                device=X.device)
    _check(lib.ox_dynamic_quantize_linear(X.numel(), _ptr(X), _ptr(Y), _ptr(y_scale), _ptr(y_zp),
                                          _ptr(workspace), workspace.numel(), _stream(stream)))
    return Y, y_scale, y_zp


def ox_batchnorm_act(X, gamma, beta, mean, var, eps=1e-5, act="none", Y=None, stream=None):
    """ONNX BatchNormalization (inference) + activation on NCHW X; the four
    parameters are fp32 device tensors [C].  Y may be X (in place)."""
    torch = _torch()
    for t, n in ((X, "X"), (gamma, "gamma"), (beta, "beta"), (mean, "mean"), (var, "var"), (Y, "Y")):
        _dense(t, n)
    N, Cc = X.shape[:2]
    HW = X.numel() // max(1, N * Cc)
    if Y is None:
        Y = torch.empty_like(X)
    _check(lib.ox_batchnorm_act(_dtype_code(X), N, Cc, HW, _ptr(X), _ptr(gamma), _ptr(beta), _ptr(mean),
                                _ptr(var), float(eps), ACT[act], _ptr(Y), _stream(stream)))
    return Y


def ox_maxpool2d(X, kernel, stride=(1, 1), pads=(0, 0, 0, 0), dilation=(1, 1), Y=None, stream=None):
    """ONNX MaxPool (NCHW, ceil_mode 0); pads (top, left, bottom, right)."""
    torch = _torch()
    _dense(X, "X")
    _dense(Y, "Y")
    N, Cc, H, W = X.shape
    d = conv_desc(N, Cc, H, W, Cc, kernel[0], kernel[1], stride, pads, dilation, 1)
    if Y is None:
        ho, wo = conv_out_hw(H, W, kernel[0], kernel[1], stride, pads, dilation)
        Y = torch.empty((N, Cc, max(ho, 0), max(wo, 0)), dtype=X.dtype, device=X.device)
    _check(lib.ox_maxpool2d(_dtype_code(X), C.byref(d), _ptr(X), _ptr(Y), _stream(stream)))
    return Y


def ox_global_avgpool(X, Y=None, stream=None):
    """ONNX GlobalAveragePool: [N, C, H, W] -> [N, C, 1, 1]."""
    torch = _torch()
    _dense(X, "X")
    _dense(Y, "Y")
    N, Cc = X.shape[:2]
    HW = X.numel() // max(1, N * Cc)
    if Y is None:
        Y = torch.empty((N, Cc, 1, 1), dtype=X.dtype, device=X.device)
    _check(lib.ox_global_avgpool(_dtype_code(X), N, Cc, HW, _ptr(X), _ptr(Y), _stream(stream)))
    return Y


def ox_conv2d_fused_packed(X, Wp, bias=None, stride=(1, 1), pads=(0, 0, 0, 0), dilation=(1, 1),
                           group=1, act="none", Y=None, M=None, kernel=(3, 3), stream=None,
                           workspace=None):
    """ox_conv2d_fused with weights packed by ox_conv2d_pack_weights (a device
    tensor of the packed bytes' dtype).  M: output channels; kernel: (kH, kW)."""
    torch = _torch()
    for t, n in ((X, "X"), (Wp, "Wp"), (bias, "bias"), (Y, "Y")):
        _dense(t, n)
    N, Cin, H, Wd = X.shape
    kH, kW = kernel
    if M is None:
        M = Wp.numel() // (Cin // group * kH * kW)
    d = conv_desc(N, Cin, H, Wd, M, kH, kW, stride, pads, dilation, group)
    if Y is None:
        ho, wo = conv_out_hw(H, Wd, kH, kW, stride, pads, dilation)
        Y = torch.empty((N, M, max(ho, 0), max(wo, 0)), dtype=X.dtype, device=X.device)
    if workspace is not None:
        _dense(workspace, "workspace")
        nbytes = workspace.numel() * workspace.element_size()
        _check(lib.ox_conv2d_fused_ws(_dtype_code(X), C.byref(d), _ptr(X), _ptr(Wp), 1, _ptr(bias),
                                      ACT[act], _ptr(Y), _ptr(workspace), nbytes, _stream(stream)))
    else:
        _check(lib.ox_conv2d_fused_packed(_dtype_code(X), C.byref(d), _ptr(X), _ptr(Wp), _ptr(bias),
                                          ACT[act], _ptr(Y), _stream(stream)))
    return Y


def ox_conv2d_fused_static(X, W, bias=None, stride=(1, 1), pads=(0, 0, 0, 0), dilation=(1, 1), group=1,
                           act="none", Y=None, stream=None, packed=False, M=None):
    """ox_conv2d_fused_ws with the library's static scratch array in place of a
    workspace (allocates nothing itself; Y must be given).  packed: W is
    packed by ox_conv2d_pack_weights (then M names the output channels)."""
    for t, n in ((X, "X"), (W, "W"), (bias, "bias"), (Y, "Y")):
        _dense(t, n)
    if Y is None:
        raise ValueError("ox_conv2d_fused_static: Y must be given")
    N, Cin, H, Wd = X.shape
    if packed:
        M = Y.shape[1] if M is None else M
        kH = kW = 3
    else:
        M, _, kH, kW = W.shape
    d = conv_desc(N, Cin, H, Wd, M, kH, kW, stride, pads, dilation, group)
    _check(lib.ox_conv2d_fused_static(_dtype_code(X), C.byref(d), _ptr(X), _ptr(W), int(bool(packed)),
                                      _ptr(bias), ACT[act], _ptr(Y), _stream(stream)))
    return Y


def ox_static_scratch_bytes():
    """Bytes of the static scratch array behind ox_conv2d_fused_static."""
    return int(lib.ox_static_scratch_bytes())


def ox_conv2d_workspace_bytes(dtype, N, Cin, H, W, M, kH, kW, stride=(1, 1), pads=(0, 0, 0, 0),
                              dilation=(1, 1), group=1):
    """Scratch bytes ox_conv2d_fused_ws may use for this geometry (0: none)."""
    d = conv_desc(N, Cin, H, W, M, kH, kW, stride, pads, dilation, group)
    return int(lib.ox_conv2d_workspace_bytes({"f32": OX_F32, "bf16": OX_BF16}[dtype], C.byref(d)))


def ox_conv2d_packed_weights_bytes(dtype, N, Cin, H, W, M, kH, kW, stride=(1, 1), pads=(0, 0, 0, 0),
                                   dilation=(1, 1), group=1):
    d = conv_desc(N, Cin, H, W, M, kH, kW, stride, pads, dilation, group)
    return int(lib.ox_conv2d_packed_weights_bytes({"f32": OX_F32, "bf16": OX_BF16}[dtype], C.byref(d)))


def ox_conv2d_pack_weights(W, dtype, N, Cin, H, Wd, stride=(1, 1), pads=(0, 0, 0, 0), dilation=(1, 1),
                           group=1):
    """Pack host weights W [M, C/g, kH, kW] (numpy array of the dtype's storage: float32, or
    uint16 bf16 bits) for ox_conv2d_fused_packed; returns a numpy array of the same dtype."""
    W = np.ascontiguousarray(W)
    M, _, kH, kW = W.shape
    d = conv_desc(N, Cin, H, Wd, M, kH, kW, stride, pads, dilation, group)
    code = {"f32": OX_F32, "bf16": OX_BF16}[dtype]
    out = np.empty_like(W)
    _check(lib.ox_conv2d_pack_weights(code, C.byref(d), W.ctypes.data, out.ctypes.data))
    return out


def ox_conv2d_int8(Xq, Wq, int8_params, y_type="i8", stride=(1, 1), pads=(0, 0, 0, 0),
                   dilation=(1, 1), group=1, Y=None, stream=None):
    """Static int8 Conv: Xq int8 (or uint8, as the parameter block says) [N,C,H,W],
    Wq int8 [M,C/g,kH,kW]; y_type 'i8', 'u8' (uint8 outputs, as the block
    says) or 'i32'."""
    torch = _torch()
    for t, n in ((Xq, "Xq"), (Wq, "Wq"), (Y, "Y")):
        _dense(t, n)
    N, Cin, H, Wd = Xq.shape
    M, _, kH, kW = Wq.shape
    d = conv_desc(N, Cin, H, Wd, M, kH, kW, stride, pads, dilation, group)
    yt = OX_I32 if y_type == "i32" else OX_I8
    if Y is None:
        ho, wo = conv_out_hw(H, Wd, kH, kW, stride, pads, dilation)
        Y = torch.empty((N, M, max(ho, 0), max(wo, 0)),
                        dtype=torch.int32 if yt == OX_I32 else
                        (torch.uint8 if y_type == "u8" else torch.int8), device=Xq.device)
    _check(lib.ox_conv2d_int8(C.byref(d), _ptr(Xq), _ptr(Wq), _ptr(int8_params), yt, _ptr(Y),
                              _stream(stream)))
    return Y


def ox_conv2d_variant(dtype, N, Cin, H, W, M, kH, kW, stride=(1, 1), pads=(0, 0, 0, 0),
                      dilation=(1, 1), group=1):
    """Name of the kernel variant a convolution of this geometry would launch
    (dtype: 'f32', 'bf16' or 'i8')."""
    d = conv_desc(N, Cin, H, W, M, kH, kW, stride, pads, dilation, group)
    buf = C.create_string_buffer(128)
    code = {"f32": OX_F32, "bf16": OX_BF16, "i8": OX_I8}[dtype]
    _check(lib.ox_conv2d_variant(code, C.byref(d), buf, 128))
    return buf.value.decode()


# ---------------------------------------------------------- offline (host) --

def _np(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def ox_fold_batchnorm(W, gamma, beta, mean, var, eps=1e-5, b0=None):
    """Fold an inference BatchNorm into conv / Gemm weights on the host.
    W: [M, ...] float32 (numpy or CPU tensor).  Returns (W', b') as float32 numpy."""
    W = _np(W, np.float32)
    M = W.shape[0]
    kper = int(W.size // M) if M else 0
    g, bt, mu, v = (_np(t, np.float32) for t in (gamma, beta, mean, var))
    b0 = None if b0 is None else _np(b0, np.float32)
    Wo = np.empty_like(W)
    bo = np.empty(M, np.float32)
    _check(lib.ox_fold_batchnorm(M, kper, W.ctypes.data, None if b0 is None else b0.ctypes.data,
                                 g.ctypes.data, bt.ctypes.data, mu.ctypes.data, v.ctypes.data,
                                 float(eps), Wo.ctypes.data, bo.ctypes.data))
    return Wo, bo


def ox_int8_params_bytes(M):
    return int(lib.ox_int8_params_bytes(int(M)))


def ox_int8_prepare(Wq, w_scale, x_scale, x_zp, y_scale, y_zp, bias_q=None, w_zp=None,
                    x_unsigned=False, y_unsigned=False):
    """Build the int8 parameter block on the host; returns it as a uint8 numpy array
    (copy it to the device, e.g. torch.from_numpy(block).cuda()).
    w_zp: per-channel weight zero points (or None); x_unsigned / y_unsigned:
    activations / requantised outputs are uint8.  Wq is int8 (uint8 weights:
    convert them with ox_int8_weights_from_uint8 first, and give the
    converted weights to the calls as well)."""
    if np.asarray(Wq).dtype != np.int8:
        raise TypeError("Wq must be int8 (convert uint8 weights with ox_int8_weights_from_uint8)")
    if w_zp is not None or x_unsigned or y_unsigned:
        Wq = _np(Wq, np.int8)
        M = Wq.shape[0]
        kper = int(Wq.size // M) if M else 0
        ws = _np(w_scale, np.float32)
        bq = None if bias_q is None else _np(bias_q, np.int32)
        wz = None if w_zp is None else _np(np.broadcast_to(np.asarray(w_zp, np.int32), (M,)), np.int32)
        out = np.zeros(ox_int8_params_bytes(M), np.uint8)
        _check(lib.ox_int8_prepare_ex(M, kper, Wq.ctypes.data, None if wz is None else wz.ctypes.data,
                                      ws.ctypes.data, float(np.float32(x_scale)), int(x_zp),
                                      int(bool(x_unsigned)), float(np.float32(y_scale)), int(y_zp),
                                      int(bool(y_unsigned)), None if bq is None else bq.ctypes.data,
                                      out.ctypes.data))
        return out
    Wq = _np(Wq, np.int8)
    M = Wq.shape[0]
    kper = int(Wq.size // M) if M else 0
    ws = _np(w_scale, np.float32)
    bq = None if bias_q is None else _np(bias_q, np.int32)
    out = np.zeros(ox_int8_params_bytes(M), np.uint8)
    _check(lib.ox_int8_prepare(M, kper, Wq.ctypes.data, ws.ctypes.data, float(np.float32(x_scale)),
                               int(x_zp), float(np.float32(y_scale)), int(y_zp),
                               None if bq is None else bq.ctypes.data, out.ctypes.data))
    return out


def ox_int8_weights_from_uint8(Wq_u8, w_zp_u8):
    """uint8 weights with (per-channel or scalar) uint8 zero points -> the
    int8 weights w - 128 and int32 zero points w_zp - 128 the int8 calls take;
    every product (w - w_zp) is unchanged."""
    Wq_u8 = np.asarray(Wq_u8)
    if Wq_u8.dtype != np.uint8:
        raise TypeError("Wq_u8 must be uint8")
    M = Wq_u8.shape[0]
    zp = np.broadcast_to(np.asarray(w_zp_u8, np.int32), (M,))
    if zp.min(initial=0) < 0 or zp.max(initial=0) > 255:
        raise ValueError("uint8 weight zero points must lie in [0, 255]")
    return (Wq_u8.astype(np.int16) - 128).astype(np.int8), (zp - 128).astype(np.int32)
