"""Throughput of the fused GEMM / implicit-GEMM convolution path on one MI355X.

A step is one pass over every layer of a workload with inputs resident in HBM:
by default the ResNet-50-v2 convolution layers (7x7 stem, 1x1 and 3x3
bottleneck convs of all four stages, stride-2 3x3 at stage entry) at batch 32
in bf16 with fp32 accumulation, BatchNorm folded into the weights and a
bias + ReLU epilogue.  Prints one JSON line: whole-job TFLOP/s (TOPS for
int8), the roofline object of the dominant kernel (measured with HIP events
on the launch stream inside the timed region) and the CPU oracle timed on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W]
                    [--workload resnet50|mobilenetv2|mlp|matmul|int8|resnet50-aux|dynq|nbits]
"""
import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2516.6, "f32": 157.3, "i8": 5033.0}   # dense MFMA TFLOP/s (TOPS int8)
HBM_PEAK = 8000.0                                      # GB/s
ESIZE = {"bf16": 2, "f32": 4, "i8": 1}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="resnet50",
                   choices=["resnet50", "mobilenetv2", "mlp", "matmul", "int8", "resnet50-aux",
                            "dynq", "nbits"])
    p.add_argument("--dtype", default=None, help="bf16 or f32 (float workloads)")
    p.add_argument("--batch", type=int, default=None)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample (0 = skip)")
    p.add_argument("--rows", default=None, help="write per-layer rows as JSON to this file")
    p.add_argument("--graph", action="store_true",
                   help="capture one step's launches in a HIP graph (torch.cuda.CUDAGraph) and time "
                        "K replays of it instead of K eager steps")
    p.add_argument("--quant", default="s8", choices=["s8", "u8", "s8-wzp", "u8-wzp"],
                   help="int8 workload: int8 ('s8') or uint8 ('u8') activations and outputs, "
                        "with ('-wzp') or without per-channel weight zero points")
    p.add_argument("--residual", action="store_true",
                   help="resnet50 / mobilenetv2: the block-closing convolutions add a residual "
                        "input before their activation (ox_conv2d_fused_res)")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="only run 10 plain device copies of this many bytes (the reference "
                        "reading for HBM byte counters), then exit")
    p.add_argument("--rotate-mb", type=float, default=512.0,
                   help="working set of the timed steps: identical copies of every layer's "
                        "tensors are cycled step by step until their total reaches this many MB, "
                        "so inputs come from HBM rather than the 256 MB last-level cache")
    p.add_argument("--ab", action="store_true",
                   help="only time every applicable kernel of each layer of the workload (forced "
                        "through OX_FORCE_KERNEL, on rotated tensors) next to the one the library "
                        "selects, print a markdown table, then exit")
    p.add_argument("--summarize-trace", default=None,
                   help="only print per-kernel medians of a rocprofv3 kernel-trace CSV as a "
                        "markdown table, then exit")
    return p.parse_args()


# ----------------------------------------------------------------- layers --

class Layer:
    """One launch of the hot path with its algorithmic work and host inputs."""

    def __init__(self, name, flops, nbytes, variant, launch, oracle_at, nout, kred):
        self.name, self.flops, self.nbytes, self.variant = name, flops, nbytes, variant
        self.launch = launch          # () -> status
        self.oracle_at = oracle_at    # (idx) -> values (CPU oracle on sampled outputs)
        self.nout, self.kred = nout, kred


def conv_layers(ox, synth, torch, cfg, layers, dtype, stream, residual=()):
    """residual: names of layers that add a residual input (the tensor of the
    output's shape) before their activation, through ox_conv2d_fused_res."""
    import oracle
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    out = []
    for li, l in enumerate(layers):
        t = synth.conv_inputs(l, cfg, li)
        # offline BatchNorm fold with the library's own host helper (untimed)
        W32 = t["W"].astype(np.float32)
        Wf, bf = ox.ox_fold_batchnorm(W32, *[t[k].astype(np.float32)
                                             for k in ("gamma", "beta", "mean", "var")], eps=1e-5)
        X64 = synth.round_to(t["X"], dtype)
        Xd = torch.from_numpy(X64.astype(np.float32)).cuda().to(tdt)
        Wd = torch.from_numpy(Wf).cuda().to(tdt)
        bd = torch.from_numpy(bf).cuda().to(tdt)
        ho, wo = l.out_hw()
        Yd = torch.empty((l.N, l.M, ho, wo), dtype=tdt, device="cuda")
        d = ox.conv_desc(l.N, l.C, l.H, l.W, l.M, l.kh, l.kw, (l.stride, l.stride), l.onnx_pads,
                         (1, 1), l.group)
        code = ox.OX_BF16 if dtype == "bf16" else ox.OX_F32
        act = ox.ACT[l.act]
        variant = ox.ox_conv2d_variant(dtype, l.N, l.C, l.H, l.W, l.M, l.kh, l.kw,
                                       (l.stride, l.stride), l.onnx_pads, (1, 1), l.group)
        Wlaunch = Wd
        fn = ox.lib.ox_conv2d_fused
        if ox.ox_conv2d_packed_weights_bytes(dtype, l.N, l.C, l.H, l.W, l.M, l.kh, l.kw,
                                             (l.stride, l.stride), l.onnx_pads, (1, 1), l.group):
            # offline weight packing (untimed, like the BatchNorm fold)
            bits = Wd.view(torch.int16).cpu().numpy().view(np.uint16)
            Wp = ox.ox_conv2d_pack_weights(bits, dtype, l.N, l.C, l.H, l.W, (l.stride, l.stride),
                                           l.onnx_pads, (1, 1), l.group)
            Wlaunch = torch.from_numpy(Wp.view(np.int16)).cuda().view(torch.bfloat16)
            fn = ox.lib.ox_conv2d_fused_packed
            variant += "+packed"
        args = (code, C.byref(d), Xd.data_ptr(), Wlaunch.data_ptr(), bd.data_ptr(), act,
                Yd.data_ptr(), stream)
        # split-K scratch for layers with few output tiles: allocated once,
        # outside the timed region, and handed to ox_conv2d_fused_ws
        wsb = ox.ox_conv2d_workspace_bytes(dtype, l.N, l.C, l.H, l.W, l.M, l.kh, l.kw,
                                           (l.stride, l.stride), l.onnx_pads, (1, 1), l.group)
        ws = None
        if wsb:
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            args = (code, C.byref(d), Xd.data_ptr(), Wlaunch.data_ptr(),
                    1 if fn is ox.lib.ox_conv2d_fused_packed else 0, bd.data_ptr(), act,
                    Yd.data_ptr(), ws.data_ptr(), wsb, stream)
            fn = ox.lib.ox_conv2d_fused_ws
        nbytes = l.nbytes(ESIZE[dtype])
        R64, Rd = None, None
        if l.name in residual:
            # a residual of the output's shape (seeded; the shortcut of a
            # bottleneck), read once more from HBM
            R64 = synth.round_to(synth.rng(cfg, li, 9).standard_normal((l.N, l.M, ho, wo)), dtype)
            Rd = torch.from_numpy(R64.astype(np.float32)).cuda().to(tdt)
            variant = ox.ox_conv2d_variant(dtype, l.N, l.C, l.H, l.W, l.M, l.kh, l.kw,
                                           (l.stride, l.stride), l.onnx_pads, (1, 1), l.group) + "+res"
            args = (code, C.byref(d), Xd.data_ptr(), Wd.data_ptr(), bd.data_ptr(), Rd.data_ptr(), act,
                    Yd.data_ptr(), ws.data_ptr() if ws is not None else None, wsb if ws is not None else 0,
                    stream)
            fn = ox.lib.ox_conv2d_fused_res
            nbytes += Rd.numel() * Rd.element_size()
        # the oracle reads the bits the GPU reads: X as rounded, W' and b' as
        # the device holds them
        Wh = Wd.float().cpu().numpy().astype(np.float64)
        bh = bd.float().cpu().numpy().astype(np.float64)
        keep = (Xd, Wd, Wlaunch, bd, Yd, d, ws, Rd)

        def launch(fn=fn, args=args, keep=keep):
            return fn(*args)

        def oracle_at(idx, X64=X64, Wh=Wh, bh=bh, l=l, R64=R64):
            return oracle.conv2d(X64, Wh, bh, (l.stride, l.stride), l.onnx_pads, (1, 1), l.group,
                                 l.act, at=idx, residual=R64)
        kred = (l.C // l.group) * l.kh * l.kw
        out.append(Layer(l.name, l.flops(), nbytes, variant, launch, oracle_at,
                         l.N * l.M * ho * wo, kred))
    return out


def aux_layers(ox, torch, dtype, batch, stream):
    """The memory-bound steps around ResNet-50's convolutions at the same
    batch: the stem MaxPool (3x3 s2 p1, 64 x 112^2), an unfoldable
    (pre-activation) BatchNorm + ReLU at each stage's input width and the
    head's GlobalAveragePool.  Seeded synthetic tensors."""
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    es = ESIZE[dtype]
    code = ox.OX_BF16 if dtype == "bf16" else ox.OX_F32
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    out = []

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32).to(tdt)

    X = rnd(batch, 64, 112, 112)
    Y = torch.empty((batch, 64, 56, 56), dtype=tdt, device="cuda")
    d = ox.conv_desc(batch, 64, 112, 112, 64, 3, 3, (2, 2), (1, 1, 1, 1))
    args = (code, C.byref(d), X.data_ptr(), Y.data_ptr(), stream)
    out.append(Layer("stem.maxpool3x3s2", 0.0, (X.numel() + Y.numel()) * es, "maxpool/" + dtype,
                     lambda a=args, k=(X, Y, d): ox.lib.ox_maxpool2d(*a), None, Y.numel(), 9))
    for cc, hw in ((256, 56), (512, 28), (1024, 14), (2048, 7)):
        X = rnd(batch, cc, hw, hw)
        Y = torch.empty_like(X)
        prm = [torch.rand(cc, generator=g, device="cuda") + 0.5 for _ in range(4)]
        args = (code, batch, cc, hw * hw, X.data_ptr(), prm[0].data_ptr(), prm[1].data_ptr(),
                prm[2].data_ptr(), prm[3].data_ptr(), 1e-5, ox.ACT["relu"], Y.data_ptr(), stream)
        out.append(Layer("bn_relu.%dx%d^2" % (cc, hw), 0.0, 2 * X.numel() * es + 16 * cc, "bn_act/" + dtype,
                         lambda a=args, k=(X, Y, prm): ox.lib.ox_batchnorm_act(*a), None, X.numel(), 1))
    X = rnd(batch, 2048, 7, 7)
    Y = torch.empty((batch, 2048, 1, 1), dtype=tdt, device="cuda")
    args = (code, batch, 2048, 49, X.data_ptr(), Y.data_ptr(), stream)
    out.append(Layer("head.gap", 0.0, (X.numel() + Y.numel()) * es, "gap/" + dtype,
                     lambda a=args, k=(X, Y): ox.lib.ox_global_avgpool(*a), None, Y.numel(), 49))
    return out


def nbits_layers(ox, synth, torch, stream):
    """MatMulNBits (4-bit weights in blocks of 32, zero points, bf16
    activations) on a 4096 x 4096 projection: decode (1 row) and prefill
    (64 rows, 256 rows).  Algorithmic bytes: A, packed B, scales, zero
    points and Y once each."""
    import oracle
    out = []
    N = K = 4096
    for M in (1, 64, 256):
        t = synth.nbits_inputs(M, N, K, 700 + M, pow2_scales=False, with_bias=False)
        A = torch.from_numpy(t["A"].astype(np.float32)).cuda().to(torch.bfloat16)
        B = torch.from_numpy(t["B"]).cuda()
        sc = torch.from_numpy(t["scales"]).cuda()
        zp = torch.from_numpy(t["zero_points"]).cuda()
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        args = (ox.OX_BF16, M, N, K, 4, 32, A.data_ptr(), B.data_ptr(), sc.data_ptr(), zp.data_ptr(),
                None, Y.data_ptr(), stream)
        nbytes = A.numel() * 2 + B.numel() + sc.numel() * 4 + zp.numel() + Y.numel() * 2

        def oracle_at(idx, t=t, M=M):
            rows = np.unique(np.asarray(idx) // N)
            full = oracle.matmul_nbits(t["A"][rows], t["B"], t["scales"], K, t["zero_points"])
            pos = {r: i for i, r in enumerate(rows)}
            return np.array([full[pos[i // N], i % N] for i in np.asarray(idx)])
        out.append(Layer("nbits.%dx%dx%d" % (M, N, K), 2.0 * M * N * K, nbytes,
                         "nbits/bf16" if M > 1 else "gemv-nbits/bf16",
                         lambda a=args, k=(A, B, sc, zp, Y): ox.lib.ox_matmul_nbits(*a),
                         oracle_at, M * N, K))
    return out


def dynq_layers(ox, torch, stream):
    """DynamicQuantizeLinear of the conformer block's fp32 activations
    (T = 1000 frames: the 1024-wide block input and the 4096-wide FFN hidden
    activation).  Algorithmic bytes: x read once (4 B) and y written (1 B)
    per element; the kernels read x twice (range, then quantise)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(4321)
    ws = torch.empty(int(ox.lib.ox_dynamic_quantize_workspace_bytes()), dtype=torch.uint8, device="cuda")
    out = []
    for width in (1024, 4096):
        X = torch.randn(1000, width, generator=g, device="cuda") * 1.7 + 0.2
        Y = torch.empty((1000, width), dtype=torch.uint8, device="cuda")
        sc = torch.empty(1, dtype=torch.float32, device="cuda")
        zp = torch.empty(1, dtype=torch.uint8, device="cuda")
        args = (X.numel(), X.data_ptr(), Y.data_ptr(), sc.data_ptr(), zp.data_ptr(), ws.data_ptr(),
                ws.numel(), stream)
        out.append(Layer("dynq.1000x%d" % width, 0.0, 5 * X.numel(), "dynq/f32",
                         lambda a=args, k=(X, Y, sc, zp, ws): ox.lib.ox_dynamic_quantize_linear(*a),
                         None, X.numel(), 1))
    return out


def gemm_layers(ox, synth, torch, rows, dtype, stream):
    import oracle
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    out = []
    for li, r in enumerate(rows):
        X, W, b = (synth.round_to(a, dtype) for a in synth.gemm_inputs(r, 1, li))
        Xd, Wd, bd = (torch.from_numpy(a.astype(np.float32)).cuda().to(tdt) for a in (X, W, b))
        Yd = torch.empty((r.M, r.N), dtype=tdt, device="cuda")
        code = ox.OX_BF16 if dtype == "bf16" else ox.OX_F32
        # the split-K workspace where one is planned (allocated once, untimed)
        nws = ox.ox_gemm_workspace_bytes(dtype, r.M, r.N, r.K)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        args = (code, r.M, r.N, r.K, 0, 1, 1.0, Xd.data_ptr(), Wd.data_ptr(), 1.0, bd.data_ptr(),
                ox.ACT[r.act], Yd.data_ptr(), ws.data_ptr() if nws else None, nws, stream)
        keep = (Xd, Wd, bd, Yd, ws)
        variant = ("gemv/%s" % dtype) if r.M == 1 else ("mfma/%s" % dtype)

        def launch(args=args, keep=keep):
            return ox.lib.ox_gemm_fused_ws(*args)

        def oracle_at(idx, X=X, W=W, b=b, r=r):
            return oracle.gemm(X, W, b, transB=True, act=r.act, at=idx)
        nbytes = (r.M * r.K + r.N * r.K + r.N + r.M * r.N) * ESIZE[dtype]
        out.append(Layer(r.name, 2.0 * r.M * r.N * r.K, nbytes, variant, launch, oracle_at,
                         r.M * r.N, r.K))
    return out


def matmul_layers(ox, synth, torch, stream):
    import oracle
    A, B = synth.matmul_inputs()
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    Cd = torch.empty((16, 64, 64), device="cuda")
    args = (ox.OX_F32, 16, 64, 64, 128, Ad.data_ptr(), 64 * 128, Bd.data_ptr(), 128 * 64,
            Cd.data_ptr(), stream)
    keep = (Ad, Bd, Cd)
    A64, B64 = A.astype(np.float64), B.astype(np.float64)

    def launch(args=args, keep=keep):
        return ox.lib.ox_matmul_batched(*args)

    def oracle_at(idx):
        return oracle.matmul(A64, B64).ravel()[idx]
    nbytes = (A.size + B.size + 16 * 64 * 64) * 4
    return [Layer("matmul_16x64x128x64", 2.0 * 16 * 64 * 64 * 128, nbytes, "mfma/f32", launch,
                  oracle_at, 16 * 64 * 64, 128)]


def int8_layers(ox, synth, torch, stream, quant="s8"):
    """quant 's8': int8 activations and outputs, symmetric weights; 'u8':
    uint8 activations and outputs (the same values shifted by 128, zero
    points too); '-wzp': per-channel weight zero points in [-8, 8]."""
    import oracle
    out = []
    u8 = quant.startswith("u8")
    wz = quant.endswith("-wzp")
    for li, l in enumerate(synth.conformer_int8_layers()):
        t = synth.int8_inputs(l, 4, li)
        wzp = None
        if u8:
            t = dict(t, xq=(t["xq"].astype(np.int16) + 128).astype(np.uint8), x_zp=t["x_zp"] + 128,
                     y_zp=t["y_zp"] + 128)
        if wz:
            wzp = np.random.default_rng(900 + li).integers(-8, 9, t["wq"].shape[0]).astype(np.int32)
        blk = torch.from_numpy(ox.ox_int8_prepare(t["wq"], t["w_s"], t["x_s"], t["x_zp"], t["y_s"],
                                                  t["y_zp"], t["bias_q"], w_zp=wzp, x_unsigned=u8,
                                                  y_unsigned=u8)).cuda()
        xq, wq = torch.from_numpy(t["xq"]).cuda(), torch.from_numpy(t["wq"]).cuda()
        ydt = torch.uint8 if u8 else torch.int8
        if l.kind == "gemm":
            Y = torch.empty((l.M, l.N), dtype=ydt, device="cuda")
            args = (ox.OX_I8, l.M, l.N, l.K, 0, 1, 1.0, xq.data_ptr(), wq.data_ptr(), 1.0, None, 0,
                    Y.data_ptr(), blk.data_ptr(), stream)
            fn = ox.lib.ox_gemm_fused
            flops = 2.0 * l.M * l.N * l.K
            nout = l.M * l.N
            variant = "mfma/i8"
            nbytes = l.M * l.K + l.N * l.K + l.M * l.N + 16 * l.N
        else:
            c = l.conv
            ho, wo = c.out_hw()
            Y = torch.empty((c.N, c.M, ho, wo), dtype=ydt, device="cuda")
            d = ox.conv_desc(c.N, c.C, c.H, c.W, c.M, c.kh, c.kw, (c.stride, c.stride), c.onnx_pads,
                             (1, 1), c.group)
            args = (C.byref(d), xq.data_ptr(), wq.data_ptr(), blk.data_ptr(), ox.OX_I8,
                    Y.data_ptr(), stream)
            fn = ox.lib.ox_conv2d_int8
            flops = c.flops()
            nout = c.N * c.M * ho * wo
            variant = ox.ox_conv2d_variant("i8", c.N, c.C, c.H, c.W, c.M, c.kh, c.kw,
                                           (c.stride, c.stride), c.onnx_pads, (1, 1), c.group)
            nbytes = c.nbytes(1) - c.M + 16 * c.M
        keep = (blk, xq, wq, Y, args)

        def launch(fn=fn, args=args, keep=keep):
            return fn(*args)

        def oracle_at(idx, l=l, t=t, wzp=wzp):
            if u8 or wz:
                if l.kind == "gemm":
                    _, y = oracle.qgemm(t["xq"], t["wq"], t["bias_q"], t["x_zp"], wzp, t["x_s"],
                                        t["w_s"], t["y_s"], t["y_zp"], u8)
                else:
                    c = l.conv
                    _, y = oracle.qconv2d(t["xq"], t["wq"], t["bias_q"], t["x_zp"], wzp, t["x_s"],
                                          t["w_s"], t["y_s"], t["y_zp"], u8, (c.stride, c.stride),
                                          c.onnx_pads, (1, 1), c.group)
                return y.ravel()[idx]
            if l.kind == "gemm":
                acc, y = oracle.gemm_int8(t["xq"], t["wq"], t["bias_q"], t["x_zp"], t["x_s"],
                                          t["w_s"], t["y_s"], t["y_zp"])
            else:
                c = l.conv
                acc, y = oracle.conv2d_int8(t["xq"], t["wq"], t["bias_q"], t["x_zp"], t["x_s"],
                                            t["w_s"], t["y_s"], t["y_zp"], (c.stride, c.stride),
                                            c.onnx_pads, (1, 1), c.group)
            return y.ravel()[idx]
        out.append(Layer(l.name, flops, nbytes, variant, launch, oracle_at, nout,
                         l.K if l.kind == "gemm" else (l.conv.C // l.conv.group) * l.conv.kh * l.conv.kw))
    return out


# ------------------------------------------------------------ CPU baseline --

def cpu_baseline(layers, seconds, int8):
    """Time the CPU oracle on a bounded sample of every layer's outputs and
    scale to the metric's unit (TFLOP/s or TOPS of the sampled outputs)."""
    import oracle
    threads = oracle.get_threads()
    if int8:
        # the int8 oracle has no point-sample entry: time whole small layers
        t0 = time.perf_counter()
        fl = 0.0
        for L in layers:
            if time.perf_counter() - t0 > seconds:
                break
            L.oracle_at(np.arange(1))
            fl += L.flops
        dt = time.perf_counter() - t0
        return {"value": fl / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
                "sample": "whole int8 layers in order until %.0f s of CPU time (%.1f s spent)"
                          % (seconds, dt)}
    macs_per_layer = 2e6
    rng = np.random.default_rng(0)
    for attempt in range(3):
        t0 = time.perf_counter()
        fl = 0.0
        npts = 0
        for L in layers:
            n = max(16, int(macs_per_layer / max(1, L.kred)))
            n = min(n, L.nout)
            idx = rng.integers(0, L.nout, n)
            L.oracle_at(idx)
            fl += 2.0 * n * L.kred
            npts += n
        dt = time.perf_counter() - t0
        if dt >= 0.5 * seconds or attempt == 2:
            break
        macs_per_layer *= min(50.0, seconds / max(dt, 1e-3))
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d sampled outputs (about %.2g MAC per layer) over all %d layers, %.1f s"
                      % (npts, macs_per_layer, len(layers), dt)}


# ------------------------------------------------------- measured traffic --

def _sources_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, dtype):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE per dispatch, scaled by a plain copy's
    reading), or None when there is none for this kernel and workload or the
    kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s_%s.txt" % (workload, dtype))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#") and "=" in line:
                k, v = line.split("=", 1)
                kv.setdefault(k.strip(), []).append(v.strip())
    for entry in kv.get("kernel", []):
        name, sources, digest, per_launch = entry.split("|")
        if name != kernel:
            continue
        if _sources_digest(sources.split(",")) != digest:
            return None
        return float(per_launch), os.path.relpath(path, ROOT)
    return None


# --------------------------------------------------------- machine facts --

def under_profiler():
    """True inside a rocprofv3 run: its preloaded library initialises the GPU
    in every child process, so a child must not go on to exec another
    program (rocm-smi starts through /usr/bin/env python3)."""
    return "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ)


def gpu_clocks():
    """Current shader and memory clock levels as rocm-smi reports them (a
    child process reading the driver's tables), or None (also under a
    profiler, where the child is not started)."""
    import subprocess
    if under_profiler():
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
    except Exception:
        return None
    card = next(iter(d.values())) if isinstance(d, dict) and d else {}
    keep = {}
    for k, v in card.items():
        kl = k.lower()
        if "sclk" in kl or "mclk" in kl or "fclk" in kl:
            keep[k] = v
    return keep or None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_ceiling(torch, stream, mb=64, sets=16, reps=48):
    """Plain device-to-device copies (torch's copy kernel) of `mb` MB each,
    cycling `sets` source/destination pairs (2 * sets * mb MB, far above the
    last-level cache): the HBM rate a streaming kernel can expect here."""
    n = int(mb * 1e6)
    pairs = [(torch.empty(n, dtype=torch.uint8, device="cuda"), torch.empty(n, dtype=torch.uint8, device="cuda"))
             for _ in range(sets)]
    for a, b in pairs:
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(reps):
        a, b = pairs[r % sets]
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del pairs
    return {"GB/s": 2 * n / (us * 1e-6) / 1e9, "bytes_moved_per_copy": 2 * n, "us_per_copy": us,
            "working_set_MB": 2 * sets * mb, "kernel": "torch copy_ (device to device)"}


def summarize_trace(path):
    """Per-kernel median / min / mean duration (us) of a rocprofv3
    kernel-trace CSV, grouped by kernel name and grid size, in order of first
    dispatch (the library's kernels)."""
    import csv
    groups = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name", "")
            if "ox::" not in name:      # the library's kernels only (not set-up copies)
                continue
            grid = row.get("Grid_Size", row.get("Grid_Size_X", ""))
            dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            groups.setdefault((name, grid), []).append(dur)
    print("| kernel | grid (threads) | dispatches | median us | min us | mean us |")
    print("|---|---:|---:|---:|---:|---:|")
    for (name, grid), d in groups.items():
        d = sorted(d)
        short = name.replace("(anonymous namespace)::", "").split("(")[0]
        print("| `%s` | %s | %d | %.2f | %.2f | %.2f |" % (short, grid, len(d), d[len(d) // 2], d[0],
                                                          sum(d) / len(d)))


# ------------------------------------------------------------- selection --

def _time_calls(torch, stream, calls, reps=None):
    """Per-call time (us) of `calls` (a list of closures, one per rotated
    tensor set) launched back to back, one event pair around them all."""
    reps = reps or max(24, 3 * len(calls))
    for c in calls:
        c()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(reps):
        calls[r % len(calls)]()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def ab_conv(ox, synth, torch, layers, dtype, stream, rotate_mb):
    """Every applicable conv kernel of each layer, timed on identical tensor
    sets cycled until they hold `rotate_mb` MB."""
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    cands = ["dwr", "dw", "pwd", "pw", "1x1", "patch", "patch+packed", "smallc", "igemm"]
    rows = []
    for l in layers:
        ho, wo = l.out_hw()
        st, pads = (l.stride, l.stride), l.onnx_pads
        geo = (l.N, l.C, l.H, l.W, l.M, l.kh, l.kw, st, pads, (1, 1), l.group)
        nb = l.nbytes(ESIZE[dtype])
        nsets = int(min(32, max(2, np.ceil(rotate_mb * 1e6 / nb))))
        K = (l.C // l.group) * l.kh * l.kw
        sets = []
        for k in range(nsets):
            X = torch.randn(l.N, l.C, l.H, l.W, device="cuda").to(tdt)
            W = (torch.randn(l.M, l.C // l.group, l.kh, l.kw) / np.sqrt(K)).to(tdt)
            b = (torch.randn(l.M, device="cuda") * 0.1).to(tdt)
            Y = torch.empty(l.N, l.M, ho, wo, device="cuda", dtype=tdt)
            Wp = None
            if dtype == "bf16" and ox.ox_conv2d_packed_weights_bytes(dtype, *geo):
                bits = W.view(torch.int16).numpy().view(np.uint16)
                Wp = torch.from_numpy(ox.ox_conv2d_pack_weights(bits, dtype, l.N, l.C, l.H, l.W, st, pads,
                                                                (1, 1), l.group).view(np.int16)).cuda().view(torch.bfloat16)
            sets.append((X, W.cuda(), b, Y, Wp))
        selected = ox.ox_conv2d_variant(dtype, *geo)
        times = {}
        for v in ["default"] + cands:
            packed = v.endswith("+packed") or (v == "default" and sets[0][4] is not None)
            if v == "default":
                os.environ.pop("OX_FORCE_KERNEL", None)
            else:
                os.environ["OX_FORCE_KERNEL"] = v.split("+")[0]
            try:
                if packed and sets[0][4] is None:
                    raise ox.OxError(3, "no packed weights")
                wsb = ox.ox_conv2d_workspace_bytes(dtype, *geo)
                ws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
                d = ox.conv_desc(*geo)
                code = ox.OX_BF16 if dtype == "bf16" else ox.OX_F32
                sp = stream.cuda_stream
                calls = []
                for (X, W, b, Y, Wp) in sets:
                    wt = Wp if packed else W
                    # the raw C-ABI call, as the benchmark step makes it
                    calls.append(lambda X=X, wt=wt, b=b, Y=Y: ox.lib.ox_conv2d_fused_ws(
                        code, C.byref(d), X.data_ptr(), wt.data_ptr(), 1 if packed else 0, b.data_ptr(),
                        ox.ACT[l.act], Y.data_ptr(), ws.data_ptr() if ws is not None else None, wsb, sp))
                if calls[0]() != 0:
                    raise ox.OxError(3, ox.ox_last_error())
                times[v] = _time_calls(torch, stream, calls)
            except ox.OxError:
                pass
        os.environ.pop("OX_FORCE_KERNEL", None)
        flops = l.flops()
        rows.append((l.name, "%d->%d %dx%d k%d s%d g%d" % (l.C, l.M, l.H, l.W, l.kh, l.stride, l.group),
                     flops / nb, selected, times))
    return rows


def ab_gemm(ox, synth, torch, grows, dtype, stream, rotate_mb):
    """GEMV against the tile engine at M = 1, split-K against a single pass
    where a split is planned."""
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    code = ox.OX_BF16 if dtype == "bf16" else ox.OX_F32
    rows = []
    for r in grows:
        nb = (r.M * r.K + r.N * r.K + r.N + r.M * r.N) * ESIZE[dtype]
        nsets = int(min(64, max(2, np.ceil(rotate_mb * 1e6 / nb))))
        sets = [(torch.randn(r.M, r.K, device="cuda").to(tdt), (torch.randn(r.N, r.K, device="cuda") / np.sqrt(r.K)).to(tdt),
                 (torch.randn(r.N, device="cuda") * 0.1).to(tdt), torch.empty(r.M, r.N, device="cuda", dtype=tdt))
                for _ in range(nsets)]
        nws = ox.ox_gemm_workspace_bytes(dtype, r.M, r.N, r.K)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        sp = stream.cuda_stream
        times = {}
        variants = [("default", None, nws)]
        if r.M == 1:
            variants += [("gemv", "gemv", 0), ("mfma", "mfma", 0)]
        if nws:
            variants += [("mfma split-K", "mfma", nws), ("mfma single pass", "mfma", 0)]
        for name, force, wsb in variants:
            if force:
                os.environ["OX_FORCE_KERNEL"] = force
            else:
                os.environ.pop("OX_FORCE_KERNEL", None)
            calls = [lambda X=X, W=W, b=b, Y=Y, wsb=wsb: ox.lib.ox_gemm_fused_ws(
                code, r.M, r.N, r.K, 0, 1, 1.0, X.data_ptr(), W.data_ptr(), 1.0, b.data_ptr(), ox.ACT[r.act],
                Y.data_ptr(), ws.data_ptr() if wsb else None, wsb, sp) for (X, W, b, Y) in sets]
            if calls[0]() == 0:
                times[name] = _time_calls(torch, stream, calls)
        os.environ.pop("OX_FORCE_KERNEL", None)
        m, n, k = r.M, r.N, r.K
        ai = 2.0 * m * n * k / ((m * k + k * n + m * n) * ESIZE[dtype])
        rows.append((r.name, "M%d N%d K%d" % (m, n, k), ai, "gemv" if m == 1 else
                     ("mfma split-K" if nws else "mfma"), times))
    return rows


def print_ab(rows, title):
    print("# %s" % title)
    print()
    print("| layer | shape | intensity (flop/B) | selected | fastest | selected / fastest | times (us per call) |")
    print("|---|---|---:|---|---|---:|---|")
    for name, shape, ai, sel, times in rows:
        if not times:
            continue
        # the selected kernel's time: its forced run where there is one (the
        # default run is the same kernel; the better of the two is kept, so
        # that run-to-run noise is not read as a wrong choice)
        key = sel.split("/")[0]
        if key == "patch" and "patch+packed" in times:
            key = "patch+packed"
        selt = min(t for k, t in times.items() if k in ("default", key))
        forced = {k: t for k, t in times.items() if k != "default"}
        best = min(forced, key=forced.get) if forced else "default"
        ratio = selt / min(selt, forced.get(best, selt))
        print("| %s | %s | %.0f | `%s` | `%s` | %.2f | %s |" % (
            name, shape, ai, sel, best, ratio, ", ".join("%s %.1f" % (k, v) for k, v in times.items())))


# -------------------------------------------------------------------- main --

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU; --gpus %d is not supported "
              "(the per-GPU path is the same kernel at one GPU's share)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    import torch
    import conv_implicit_gemm_amd as ox
    import synth

    torch.cuda.set_device(0)
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "copies": 10}))
        return
    stream = torch.cuda.current_stream()
    if args.ab:
        wl = args.workload
        dtype = args.dtype or ("f32" if wl == "mobilenetv2" else "bf16")
        if wl == "resnet50":
            rows = ab_conv(ox, synth, torch, synth.resnet50_layers(args.batch or 32), dtype, stream, args.rotate_mb)
        elif wl == "mobilenetv2":
            rows = ab_conv(ox, synth, torch, synth.mobilenetv2_layers(args.batch or 64), dtype, stream, args.rotate_mb)
        elif wl == "mlp":
            rows = ab_gemm(ox, synth, torch, synth.mlp_rows(), dtype, stream, args.rotate_mb)
        else:
            print("bench.py --ab: resnet50, mobilenetv2 or mlp", file=sys.stderr)
            sys.exit(2)
        print_ab(rows, "%s, %s%s: every applicable kernel per layer" % (
            wl, dtype, "" if wl == "mlp" else ", batch %d" % (args.batch or (32 if wl == "resnet50" else 64))))
        return
    if args.graph:
        # capture needs a stream of its own (default priority)
        stream = torch.cuda.Stream()
        torch.cuda.set_stream(stream)
    sp = stream.cuda_stream
    wl = args.workload
    if wl == "resnet50":
        dtype = args.dtype or "bf16"
        batch = args.batch or 32
        res = [l.name for l in synth.resnet50_layers(batch) if l.name.endswith("1x1b")] if args.residual else []
        builder = lambda: conv_layers(ox, synth, torch, 3, synth.resnet50_layers(batch), dtype, sp, res)
        cfg = {"workload": "resnet50-v2 convolutions (16 layers), NCHW", "batch": batch,
               "input": "3x224x224", "epilogue": "folded BN bias + ReLU"}
        if res:
            cfg["residual"] = "the last 1x1 of each stage adds a residual before its ReLU"
    elif wl == "resnet50-aux":
        dtype = args.dtype or "bf16"
        batch = args.batch or 32
        builder = lambda: aux_layers(ox, torch, dtype, batch, sp)
        cfg = {"workload": "resnet50 memory-bound steps: stem MaxPool, pre-activation BatchNorm + "
                           "ReLU at each stage width, head GlobalAveragePool", "batch": batch}
    elif wl == "mobilenetv2":
        dtype = args.dtype or "f32"
        batch = args.batch or 64
        mb = synth.mobilenetv2_layers(batch)
        # the stride-1 blocks whose input and output widths agree close with
        # a residual add after their (linear) projection
        res = [mb[i].name for i in range(len(mb)) if args.residual and mb[i].name.endswith("project")
               and not mb[i].name.endswith(".0.project")] if args.residual else []
        builder = lambda: conv_layers(ox, synth, torch, 2, mb, dtype, sp, res)
        cfg = {"workload": "mobilenetv2 convolutions (51 layers), NCHW", "batch": batch,
               "input": "3x224x224", "epilogue": "folded BN bias + ReLU6 / linear"}
        if res:
            cfg["residual"] = "the projection of each repeated block adds a residual"
    elif wl == "mlp":
        dtype = args.dtype or "bf16"
        builder = lambda: gemm_layers(ox, synth, torch, synth.mlp_rows(), dtype, sp)
        cfg = {"workload": "MLP Gemm rows M in {1,64,256} x (1024->4096 GELU, 4096->1024, "
                           "1024->1024 ReLU)"}
    elif wl == "nbits":
        dtype = "bf16"
        builder = lambda: nbits_layers(ox, synth, torch, sp)
        cfg = {"workload": "MatMulNBits 4-bit blocks of 32 with zero points, [M,4096] x "
                           "[4096->4096], M in {1, 64, 256}"}
    elif wl == "dynq":
        dtype = "f32"
        builder = lambda: dynq_layers(ox, torch, sp)
        cfg = {"workload": "DynamicQuantizeLinear fp32 -> uint8 of [1000,1024] and [1000,4096] "
                           "activations"}
    elif wl == "matmul":
        dtype = "f32"
        builder = lambda: matmul_layers(ox, synth, torch, sp)
        cfg = {"workload": "batched MatMul [16,64,128] x [16,128,64]"}
    else:
        dtype = "i8"
        builder = lambda: int8_layers(ox, synth, torch, sp, args.quant)
        cfg = {"workload": "static int8 conformer block, T=1000, d_model=1024 "
                           "(FFN, QKV, depthwise 1-D k9, pointwise)"}
        if args.quant != "s8":
            cfg["quant"] = {"u8": "uint8 activations and outputs",
                            "s8-wzp": "per-channel weight zero points",
                            "u8-wzp": "uint8 activations and outputs, per-channel weight zero "
                                      "points"}[args.quant]

    # Rotation: identical copies of every layer's tensors (same seeds), one
    # set per step in turn, until the sets hold --rotate-mb: each step then
    # finds its inputs in HBM, not in the 256 MB last-level cache.
    layers = builder()
    step_bytes = sum(L.nbytes for L in layers)
    nsets = int(min(64, max(1, np.ceil(args.rotate_mb * 1e6 / max(1.0, step_bytes)))))
    sets = [layers] + [builder() for _ in range(nsets - 1)]

    def step(s):
        for L in sets[s % nsets]:
            st = L.launch()
            if st != 0:
                raise RuntimeError("%s: %s" % (L.name, ox.ox_last_error()))

    # host cost of one C-ABI call (argument marshalling and the launch), on
    # the first set, without waiting for the GPU (whole steps, before the
    # warm-up: a profiler's last pass stays the per-kernel pass below)
    torch.cuda.synchronize()
    ncall = 0
    h0 = time.perf_counter()
    while ncall < 2000 and time.perf_counter() - h0 < 0.2:
        for L in layers:
            L.launch()
            ncall += 1
    t_call_us = (time.perf_counter() - h0) / max(1, ncall) * 1e6
    torch.cuda.synchronize()

    for w in range(max(args.warmup, nsets)):
        step(w)
    torch.cuda.synchronize()
    run_step = step
    if args.graph:
        graphs = []
        for k in range(nsets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(k)
            graphs.append(g)
        torch.cuda.synchronize()
        for w in range(max(args.warmup, nsets)):
            graphs[w % nsets].replay()
        torch.cuda.synchronize()
        run_step = lambda s: graphs[s % nsets].replay()
        cfg = dict(cfg, graph="one step per tensor set captured in a HIP graph, replayed in turn")

    clocks_before = gpu_clocks()
    # timed region: K steps back to back, one event pair around all of them
    # (same stream).  An event between two kernels is a stream marker that
    # itself costs a few microseconds of idle GPU, so the per-kernel events
    # are taken in a second pass of K steps, used only for the per-kernel
    # durations (the roofline), not for the step time.
    K = args.steps
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(K):
        run_step(s)
    t_end.record(stream)
    host_s = time.perf_counter() - wall0
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    clocks_after = gpu_clocks()

    # per-kernel pass: K more steps, an event pair around every launch;
    # the per-layer figure is the median over the K steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in layers] for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        for i, L in enumerate(sets[s % nsets]):
            ev[s][i][0].record(stream)
            st = L.launch()
            ev[s][i][1].record(stream)
            if st != 0:
                raise RuntimeError("%s: %s" % (L.name, ox.ox_last_error()))
    torch.cuda.synchronize()
    per_layer_ms = [float(np.median([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(K)]))
                    for i in range(len(layers))]

    step_flops = sum(L.flops for L in layers)
    ms_per_step = total_ms / K
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    if step_flops == 0:      # a workload of memory-bound steps only: report its bandwidth
        value = sum(L.nbytes for L in layers) / (ms_per_step * 1e-3) / 1e9

    # per-layer roofline (attainable time t_roof = max(FLOP / MFMA peak,
    # algorithmic bytes / HBM peak)) and the dominant kernel: the variant
    # with the largest share of the step
    pk = PEAK[dtype]
    groups = {}
    for L, t in zip(layers, per_layer_ms):
        g = groups.setdefault(L.variant, {"ms": 0.0, "flops": 0.0, "bytes": 0.0, "n": 0,
                                          "t_flop": 0.0, "t_byte": 0.0, "t_roof": 0.0})
        g["ms"] += t
        g["flops"] += L.flops
        g["bytes"] += L.nbytes
        g["n"] += 1
        tf, tb = L.flops / (pk * 1e12), L.nbytes / (HBM_PEAK * 1e9)
        if L.variant.startswith("dw") or L.variant.startswith("gemv"):
            tf = 0.0          # no MFMA: counted against HBM only
        g["t_flop"] += tf
        g["t_byte"] += tb
        g["t_roof"] += max(tf, tb)
    dom = max(groups, key=lambda k: groups[k]["ms"])
    g = groups[dom]
    avg_us = g["ms"] / g["n"] * 1e3
    if g["t_byte"] >= g["t_flop"]:
        ach = g["bytes"] / (g["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK, "unit": "GB/s",
                "frac": ach / HBM_PEAK, "traffic": None}
        algo_per_launch = g["bytes"] / g["n"]
    else:
        ach = g["flops"] / (g["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": pk,
                "unit": "TOPS" if dtype == "i8" else "TFLOP/s", "frac": ach / pk, "traffic": None}
        algo_per_launch = g["bytes"] / g["n"]
    mt = measured_traffic(dom, wl, dtype)
    roof["algorithmic_bytes_per_launch"] = algo_per_launch
    if mt:
        roof["traffic"] = mt[0]
        roof["traffic_vs_algorithmic"] = mt[0] / max(1.0, algo_per_launch)
        roof["traffic_source"] = mt[1]
    roof["kernel"] = dom
    roof["launches_per_step"] = g["n"]
    roof["avg_launch_us"] = avg_us
    roof["roofline_frac"] = g["t_roof"] / (g["ms"] * 1e-3)   # sum t_roof / sum t_meas

    # every variant family of the step (the dominant one is `roofline`)
    families = {}
    for name, gr in groups.items():
        mfma = gr["t_flop"] > gr["t_byte"]
        sec = gr["ms"] * 1e-3
        families[name] = {"launches_per_step": gr["n"], "us_per_step": gr["ms"] * 1e3,
                          "bound": "mfma" if mfma else "hbm",
                          "tflops": gr["flops"] / sec / 1e12, "gbs": gr["bytes"] / sec / 1e9,
                          "mfma_frac": gr["flops"] / sec / 1e12 / pk if gr["t_flop"] > 0 else None,
                          "hbm_frac": gr["bytes"] / sec / 1e9 / HBM_PEAK,
                          "roofline_frac": gr["t_roof"] / sec}

    cpu = None
    if args.cpu_seconds > 0 and step_flops > 0:
        cpu = cpu_baseline(layers, args.cpu_seconds, dtype == "i8")
        cpu["cpu_model"] = cpu_model()
    ceiling = copy_ceiling(torch, stream)

    unit = "TOPS" if dtype == "i8" else "TFLOP/s"
    if step_flops == 0:
        unit = "GB/s"
    out = {
        "metric": "TFLOP/s (TOPS int8) per fused GEMM/conv shape + % of MFMA or HBM roofline",
        "value": value, "unit": unit, "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype if dtype != "i8" else "int8",
        "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": cfg, "roofline": roof, "cpu_baseline": cpu,
        "families": families,
        "rotation": {"tensor_sets": nsets, "working_set_MB": nsets * step_bytes / 1e6,
                     "step_algorithmic_MB": step_bytes / 1e6},
        "timing": {"per_layer": "median over the K steps of an event pair around each launch "
                                "(a second pass; the step time has no events between kernels)",
                   "host_wall_s": wall, "host_enqueue_s_per_step": host_s / K,
                   "t_call_us": t_call_us},
        "machine": {"gpu_clocks_before": clocks_before, "gpu_clocks_after": clocks_after,
                    "cpu_model": cpu_model(), "copy_ceiling": ceiling},
    }
    if args.rows:
        rows = []
        for L, t in zip(layers, per_layer_ms):
            tf, tb = L.flops / (pk * 1e12), L.nbytes / (HBM_PEAK * 1e9)
            if L.variant.startswith("dw") or L.variant.startswith("gemv"):
                tf = 0.0
            rows.append({"layer": L.name, "variant": L.variant, "us": t * 1e3, "flop": L.flops,
                         "bytes": L.nbytes, "ai": L.flops / max(1.0, L.nbytes),
                         "bound": "mfma" if tf > tb else "hbm",
                         "tflops": L.flops / (t * 1e-3) / 1e12,
                         "gbs": L.nbytes / (t * 1e-3) / 1e9,
                         "mfma_frac": L.flops / (t * 1e-3) / 1e12 / PEAK[dtype],
                         "hbm_frac": L.nbytes / (t * 1e-3) / 1e9 / HBM_PEAK,
                         "roofline_frac": max(tf, tb) / (t * 1e-3)})
        with open(args.rows, "w") as f:
            json.dump({"workload": wl, "dtype": dtype, "rows": rows}, f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
