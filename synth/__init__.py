"""Seeded synthetic inputs and workload shapes.

This module serves both sides of every check -- the GPU library and the CPU
oracle -- and holds none of the method's arithmetic: it only lists layer
shapes and draws random tensors.  Every draw comes from
``numpy.random.default_rng([1234, cfg, layer, tensor])`` (PCG64), in float64,
then rounded to float32 (round to nearest even) and, for bf16 workloads, to
bfloat16 (round to nearest even).  Both sides receive identical bits.

The five workloads stand in for the pages' models, which are not available:
  cfg 0  batched MatMul fp32 [16,64,128] x [16,128,64] (OxiONNX 0.1.7,
         "True batched MatMul/Gemm dispatch"), plus the all-ones 64^3 case
         from its two-stream race report;
  cfg 1  MLP Gemm rows with a fused activation (tensorforge mlp.onnx scale-up);
  cfg 2  MobileNetV2 convolution layers (onnx-vulkan-rs validation model);
  cfg 3  ResNet-50-v2 convolution layers (tensorforge resnet50-v2);
  cfg 4  a static int8 conformer-encoder block (onnx-vulkan-rs Parakeet
         encoder), T = 1000 frames, d_model = 1024.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

SEED = 1234

# tensor ids inside one layer
T_X, T_W, T_BIAS, T_GAMMA, T_BETA, T_MEAN, T_VAR = 0, 1, 2, 3, 4, 5, 6
T_XS, T_XZP, T_WS, T_BF, T_YZP = 7, 8, 9, 10, 11


def rng(cfg: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([SEED, cfg, layer, tensor])


# ----------------------------------------------------------------- rounding --

def to_f32(a) -> np.ndarray:
    """float64 -> float32, round to nearest even (numpy's cast)."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))


def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs here are finite by construction."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32)


def round_to(a, dtype: str) -> np.ndarray:
    """Round float64 values to the storage type and return them as float64
    (the exact values both sides will read)."""
    f = to_f32(a)
    if dtype == "bf16":
        f = bf16_bits_to_f32(f32_to_bf16_bits(f))
    elif dtype != "f32":
        raise ValueError(dtype)
    return f.astype(np.float64)


# ------------------------------------------------------------------ shapes --

@dataclass
class ConvLayer:
    name: str
    N: int
    C: int
    H: int
    W: int
    M: int
    k: int
    stride: int = 1
    pad: int = 0
    group: int = 1
    act: str = "none"
    kW: Optional[int] = None          # defaults to k
    pads: Optional[Tuple[int, int, int, int]] = None   # ONNX (t, l, b, r); defaults to pad
    dilation: int = 1

    @property
    def kh(self):
        return self.k

    @property
    def kw(self):
        return self.k if self.kW is None else self.kW

    @property
    def onnx_pads(self):
        return self.pads if self.pads is not None else (self.pad,) * 4

    def out_hw(self):
        t, l, b, r = self.onnx_pads
        d = self.dilation
        ho = (self.H + t + b - d * (self.kh - 1) - 1) // self.stride + 1
        wo = (self.W + l + r - d * (self.kw - 1) - 1) // self.stride + 1
        return ho, wo

    def key(self):
        return (self.N, self.C, self.H, self.W, self.M, self.kh, self.kw, self.stride,
                self.onnx_pads, self.group, self.act, self.dilation)

    def flops(self):
        ho, wo = self.out_hw()
        return 2.0 * self.N * self.M * ho * wo * (self.C // self.group) * self.kh * self.kw

    def nbytes(self, esize: int):
        ho, wo = self.out_hw()
        x = self.N * self.C * self.H * self.W
        w = self.M * (self.C // self.group) * self.kh * self.kw
        y = self.N * self.M * ho * wo
        return (x + w + self.M + y) * esize


def mobilenetv2_layers(N: int) -> List[ConvLayer]:
    """MobileNetV2 convolutions: 3x3 s2 stem 3->32, then inverted-residual
    blocks (t, c, n, s); each block is 1x1 expand (x t, ReLU6; absent when
    t = 1), 3x3 depthwise (stride s on the first repeat, pad 1, ReLU6) and a
    1x1 linear projection.  51 convolutions."""
    L = [ConvLayer("stem3x3s2", N, 3, 224, 224, 32, 3, 2, 1, 1, "relu6")]
    cin, H = 32, 112
    for bi, (t, c, n, s) in enumerate([(1, 16, 1, 1), (6, 24, 2, 2), (6, 32, 3, 2), (6, 64, 4, 2),
                                        (6, 96, 3, 1), (6, 160, 3, 2), (6, 320, 1, 1)]):
        for r in range(n):
            stride = s if r == 0 else 1
            hid = cin * t
            tag = "b%d.%d" % (bi, r)
            if t != 1:
                L.append(ConvLayer(tag + ".expand", N, cin, H, H, hid, 1, 1, 0, 1, "relu6"))
            L.append(ConvLayer(tag + ".dw", N, hid, H, H, hid, 3, stride, 1, hid, "relu6"))
            Ho = (H + 2 - 3) // stride + 1
            L.append(ConvLayer(tag + ".project", N, hid, Ho, Ho, c, 1, 1, 0, 1, "none"))
            cin, H = c, Ho
    return L


def resnet50_layers(N: int) -> List[ConvLayer]:
    """ResNet-50-v2 convolution shapes: 7x7 s2 p3 stem 3->64, then per stage
    (C, H): 1x1 C->C/4, 3x3 C/4->C/4 at H, the stride-2 3x3 from 2H at the
    entry of stages 2-4, and 1x1 C/4->C.  Every conv has bias + ReLU."""
    L = [ConvLayer("stem7x7s2", N, 3, 224, 224, 64, 7, 2, 3, 1, "relu")]
    for si, (Cc, H) in enumerate([(256, 56), (512, 28), (1024, 14), (2048, 7)]):
        q = Cc // 4
        tag = "s%d" % (si + 1)
        L.append(ConvLayer(tag + ".1x1a", N, Cc, H, H, q, 1, 1, 0, 1, "relu"))
        L.append(ConvLayer(tag + ".3x3", N, q, H, H, q, 3, 1, 1, 1, "relu"))
        if si > 0:
            L.append(ConvLayer(tag + ".3x3s2", N, q, 2 * H, 2 * H, q, 3, 2, 1, 1, "relu"))
        L.append(ConvLayer(tag + ".1x1b", N, q, H, H, Cc, 1, 1, 0, 1, "relu"))
    return L


def unique_layers(layers: List[ConvLayer]) -> List[ConvLayer]:
    seen, out = set(), []
    for l in layers:
        if l.key() not in seen:
            seen.add(l.key())
            out.append(l)
    return out


@dataclass
class GemmRow:
    name: str
    M: int
    K: int
    N: int
    act: str


def mlp_rows() -> List[GemmRow]:
    rows = []
    for M in (1, 64, 256):
        for (K, N, a) in ((1024, 4096, "gelu"), (4096, 1024, "none"), (1024, 1024, "relu")):
            rows.append(GemmRow("mlp_M%d_%dx%d_%s" % (M, K, N, a), M, K, N, a))
    return rows


@dataclass
class Int8Layer:
    name: str
    kind: str                 # "gemm" or "conv"
    M: int                    # gemm rows (T) / conv batch is 1
    K: int
    N: int                    # output features / channels
    conv: Optional[ConvLayer] = None


def conformer_int8_layers(T: int = 1000, d: int = 1024) -> List[Int8Layer]:
    """The static int8 conformer block: FFN 1024->4096->1024 and QKV
    1024->3072 as Gemms on X [T, K]; a depthwise 1-D conv (kernel [1,9],
    pads [0,4,0,4], group 1024) and a pointwise 1024->2048 conv on
    [1, 1024, 1, T]."""
    return [
        Int8Layer("ffn1", "gemm", T, d, 4 * d),
        Int8Layer("ffn2", "gemm", T, 4 * d, d),
        Int8Layer("qkv", "gemm", T, d, 3 * d),
        Int8Layer("dw1d", "conv", 1, 9, d,
                  ConvLayer("dw1d", 1, d, 1, T, d, 1, 1, 0, d, "none", kW=9, pads=(0, 4, 0, 4))),
        Int8Layer("pw", "conv", 1, d, 2 * d,
                  ConvLayer("pw", 1, d, 1, T, 2 * d, 1, 1, 0, 1, "none")),
    ]


# ----------------------------------------------------------------- tensors --

def matmul_inputs(cfg: int = 0, layer: int = 0, batch=16, M=64, K=128, N=64):
    """A, B ~ U[-1, 1] in fp32 (returned as float32 arrays)."""
    A = to_f32(rng(cfg, layer, T_X).uniform(-1.0, 1.0, (batch, M, K)))
    B = to_f32(rng(cfg, layer, T_W).uniform(-1.0, 1.0, (batch, K, N)))
    return A, B


def gemm_inputs(row: GemmRow, cfg: int = 1, layer: int = 0):
    """X ~ N(0,1) [M,K]; W ~ N(0, 1/K) [N,K] (variance 1/K); b ~ U[-0.1, 0.1].
    Returned as float64 arrays holding float32 values."""
    X = rng(cfg, layer, T_X).standard_normal((row.M, row.K))
    W = rng(cfg, layer, T_W).standard_normal((row.N, row.K)) * np.sqrt(1.0 / row.K)
    b = rng(cfg, layer, T_BIAS).uniform(-0.1, 0.1, row.N)
    return X, W, b


def conv_inputs(layer: ConvLayer, cfg: int, li: int):
    """X ~ N(0,1); He-normal W ~ N(0, 2/fan_in) with fan_in = C/g*kH*kW;
    BatchNorm gamma ~ U[0.5,1.5], beta ~ N(0, 0.1), mean ~ N(0, 0.1),
    var ~ U[0.5,1.5] (the second argument of N read as the variance).
    Returned as float64 arrays (the caller rounds them to the storage type)."""
    cpg = layer.C // layer.group
    fan_in = cpg * layer.kh * layer.kw
    X = rng(cfg, li, T_X).standard_normal((layer.N, layer.C, layer.H, layer.W))
    W = rng(cfg, li, T_W).standard_normal((layer.M, cpg, layer.kh, layer.kw)) * np.sqrt(2.0 / fan_in)
    g = rng(cfg, li, T_GAMMA).uniform(0.5, 1.5, layer.M)
    be = rng(cfg, li, T_BETA).standard_normal(layer.M) * np.sqrt(0.1)
    mu = rng(cfg, li, T_MEAN).standard_normal(layer.M) * np.sqrt(0.1)
    var = rng(cfg, li, T_VAR).uniform(0.5, 1.5, layer.M)
    return dict(X=X, W=W, gamma=g, beta=be, mean=mu, var=var)


def int8_inputs(layer: Int8Layer, cfg: int = 4, li: int = 0):
    """Static int8 tensors: x_q ~ U{-128..127}, x_s ~ U[0.01,0.1],
    x_zp ~ U{-20..20}, w_q ~ U{-127..127} (symmetric), w_s[m] ~ U[1e-3,1e-2],
    bias_q[m] = rint(b_f / (x_s*w_s[m])) with b_f ~ U[-0.1,0.1],
    y_s = 3*x_s*mean(w_s)*sqrt(K)*73.9*73.6/127 (about a 3-sigma range),
    y_zp ~ U{-20..20}.  Scales are float32."""
    if layer.kind == "gemm":
        xshape = (layer.M, layer.K)
        wshape = (layer.N, layer.K)
        kred = layer.K
        nout = layer.N
    else:
        c = layer.conv
        xshape = (c.N, c.C, c.H, c.W)
        wshape = (c.M, c.C // c.group, c.kh, c.kw)
        kred = (c.C // c.group) * c.kh * c.kw
        nout = c.M
    xq = rng(cfg, li, T_X).integers(-128, 128, xshape).astype(np.int8)
    wq = rng(cfg, li, T_W).integers(-127, 128, wshape).astype(np.int8)
    x_s = np.float32(rng(cfg, li, T_XS).uniform(0.01, 0.1))
    x_zp = int(rng(cfg, li, T_XZP).integers(-20, 21))
    w_s = to_f32(rng(cfg, li, T_WS).uniform(1e-3, 1e-2, nout))
    b_f = rng(cfg, li, T_BF).uniform(-0.1, 0.1, nout)
    bias_q = np.rint(b_f / (np.float64(x_s) * w_s.astype(np.float64))).astype(np.int32)
    y_s = np.float32(3.0 * np.float64(x_s) * float(np.mean(w_s.astype(np.float64)))
                     * np.sqrt(kred) * 73.9 * 73.6 / 127.0)
    y_zp = int(rng(cfg, li, T_YZP).integers(-20, 21))
    return dict(xq=xq, wq=wq, x_s=x_s, x_zp=x_zp, w_s=w_s, bias_q=bias_q, y_s=y_s, y_zp=y_zp)


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """[rows, n] values in 0..15 -> [rows, ceil(n/2)] bytes, value 2i in the
    low nibble of byte i and value 2i+1 in its high nibble (the MatMulNBits
    storage order)."""
    q = np.asarray(q, dtype=np.uint8)
    if q.shape[1] % 2:
        q = np.concatenate([q, np.zeros((q.shape[0], 1), np.uint8)], axis=1)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def nbits_inputs(M: int, N: int, K: int, seed: int, with_zp: bool = True, pow2_scales: bool = True,
                 with_bias: bool = True):
    """Seeded MatMulNBits operands (4 bits, blocks of 32): A ~ N(0,1) in bf16,
    q ~ U{0..15}, zero points ~ U{0..15} (or the default 8), scales per block
    either powers of two around 1/(4*sqrt(K)) (every dequantised weight exact
    in bf16) or U[0.5,1.5]/(4*sqrt(K)); bias ~ N(0, 0.1) in bf16.  Returns a
    dict with the unpacked values (q, zp, scales) and the packed device forms
    (B [N, nblk, 16], zero_points [N, ceil(nblk/2)])."""
    r = np.random.default_rng(seed)
    nblk = (K + 31) // 32
    A = round_to(r.standard_normal((M, K)), "bf16")
    q = r.integers(0, 16, (N, nblk * 32)).astype(np.uint8)
    zp = r.integers(0, 16, (N, nblk)).astype(np.uint8) if with_zp else np.full((N, nblk), 8, np.uint8)
    base = 1.0 / (4.0 * np.sqrt(max(K, 1)))
    if pow2_scales:
        scales = (2.0 ** np.round(np.log2(base) + r.integers(-1, 2, (N, nblk)))).astype(np.float32)
    else:
        scales = (r.uniform(0.5, 1.5, (N, nblk)) * base).astype(np.float32)
    B = pack_nibbles(q).reshape(N, nblk, 16)
    zpk = pack_nibbles(zp) if with_zp else None
    bias = round_to(r.standard_normal(N) * 0.1, "bf16") if with_bias else None
    return {"A": A, "q": q[:, :K], "zp": zp, "scales": scales, "B": B, "zero_points": zpk,
            "bias": bias, "K": K}
