"""HIP graph capture of a chain of libox calls.

Every entry point launches kernels only (no allocation, no memset, no host
synchronisation), so a caller may record a whole layer chain into one HIP
graph and replay it.  The test captures such a chain (a split-K 3x3 conv with
its workspace, a depthwise conv, a residual pointwise conv, MaxPool,
BatchNorm + ReLU, GlobalAveragePool, a Gemm + GELU, a batched f32 MatMul, an
int8 Gemm and a split-K Gemm with its workspace), then replays it several
times with new inputs.  Each call reads its own input buffers, refilled with
new seeded values before every replay, so every replayed output is compared
with the oracle on those values; between replays the outputs are refilled
with NaN and the same chain runs eagerly on the same buffers, and each replay
must also equal the eager results bit for bit (the same kernels with the same
launch shapes and a fixed summation order)."""
import sys

import numpy as np
import pytest

import oracle
import synth
from parity import assert_close

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(dt)


def test_captured_chain_replays_match_eager_and_oracle():
    import conv_implicit_gemm_amd as ox
    bf = torch.bfloat16
    r = np.random.default_rng(4242)
    N, C, H = 2, 256, 7            # the 3x3 conv of this shape is planned split-K
    M = 128
    Hp = 4                         # MaxPool 3x3 s2 p1 of 7x7

    def wt(*shape, scale):
        h = synth.round_to(r.standard_normal(shape) * scale, "bf16")
        return h, to_dev(h, bf)

    # weights and parameters (fixed across replays): host float64 copies of
    # the exact bf16 values, and the device tensors
    (W1h, W1), (b1h, b1) = wt(M, C, 3, 3, scale=0.05), wt(M, scale=0.1)
    (Wdh, Wd), (bdh, bd) = wt(M, 1, 3, 3, scale=0.3), wt(M, scale=0.1)
    (Wph, Wp), (bph, bp) = wt(M, M, 1, 1, scale=0.08), wt(M, scale=0.1)
    gh = r.uniform(0.5, 1.5, M).astype(np.float32)
    beh = (r.standard_normal(M) * 0.3).astype(np.float32)
    muh = (r.standard_normal(M) * 0.3).astype(np.float32)
    varh = r.uniform(0.5, 1.5, M).astype(np.float32)
    gam, bet, mu, var = (torch.from_numpy(v).cuda() for v in (gh, beh, muh, varh))
    (Bgh, Bg), (bgh, bg) = wt(M, 300, scale=0.1), wt(300, scale=0.1)
    ws_bytes = ox.ox_conv2d_workspace_bytes("bf16", N, C, H, H, M, 3, 3, (1, 1), (1, 1, 1, 1))
    assert ws_bytes > 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    qlayer = synth.Int8Layer("g", "gemm", 77, 200, 45)
    qt = synth.int8_inputs(qlayer, 4, 61)
    qblk = torch.from_numpy(ox.ox_int8_prepare(qt["wq"], qt["w_s"], qt["x_s"], qt["x_zp"], qt["y_s"],
                                               qt["y_zp"], qt["bias_q"])).cuda()
    wq = torch.from_numpy(qt["wq"]).cuda()
    # a split-K Gemm with its workspace (64 rows, K = 2048)
    Bsh, Bs = wt(256, 2048, scale=0.02)
    gws_bytes = ox.ox_gemm_workspace_bytes("bf16", 64, 256, 2048)
    assert gws_bytes > 0
    gws = torch.empty(gws_bytes // 4, dtype=torch.float32, device="cuda")

    # inputs (refilled before every run, one buffer per call) and outputs
    # (fixed addresses)
    shapes_in = {"X0": (N, C, H, H), "X1": (N, M, H, H), "X2": (N, M, H, H), "R2": (N, M, H, H),
                 "X3": (N, M, H, H), "X4": (N, M, Hp, Hp), "X5": (N, M, Hp, Hp), "X6": (N, M),
                 "Ag": (64, 2048)}
    ins = {k: torch.empty(v, dtype=bf, device="cuda") for k, v in shapes_in.items()}
    A = torch.empty((4, 37, 53), dtype=torch.float32, device="cuda")
    B = torch.empty((4, 53, 29), dtype=torch.float32, device="cuda")
    xq = torch.empty((77, 200), dtype=torch.int8, device="cuda")
    Y1, Y2, Y3 = (torch.empty((N, M, H, H), dtype=bf, device="cuda") for _ in range(3))
    Y4, Y5 = (torch.empty((N, M, Hp, Hp), dtype=bf, device="cuda") for _ in range(2))
    Y6 = torch.empty((N, M, 1, 1), dtype=bf, device="cuda")
    Y7 = torch.empty((N, 300), dtype=bf, device="cuda")
    Cm = torch.empty((4, 37, 29), dtype=torch.float32, device="cuda")
    Yq = torch.empty((77, 45), dtype=torch.int8, device="cuda")
    Ys = torch.empty((64, 256), dtype=bf, device="cuda")
    outs = [Y1, Y2, Y3, Y4, Y5, Y6, Y7, Cm, Ys]

    s = torch.cuda.Stream()

    def chain():
        i = ins
        ox.ox_conv2d_fused(i["X0"], W1, b1, (1, 1), (1, 1, 1, 1), act="relu", Y=Y1, stream=s, workspace=ws)
        ox.ox_conv2d_fused(i["X1"], Wd, bd, (1, 1), (1, 1, 1, 1), group=M, act="relu6", Y=Y2, stream=s)
        ox.ox_conv2d_fused_res(i["X2"], Wp, i["R2"], bp, act="relu", Y=Y3, stream=s)
        ox.ox_maxpool2d(i["X3"], (3, 3), (2, 2), (1, 1, 1, 1), Y=Y4, stream=s)
        ox.ox_batchnorm_act(i["X4"], gam, bet, mu, var, 1e-5, "relu", Y=Y5, stream=s)
        ox.ox_global_avgpool(i["X5"], Y=Y6, stream=s)
        ox.ox_gemm_fused(i["X6"], Bg, bg, act="gelu", Y=Y7, stream=s)
        ox.ox_matmul_batched(A, B, Cm, stream=s)
        ox.ox_gemm_fused(xq, wq, transB=True, int8_params=qblk, out_dtype=torch.int8, Y=Yq, stream=s)
        ox.ox_gemm_fused_ws(i["Ag"], Bs, gws, transB=True, act="relu", Y=Ys, stream=s)

    def refill(rep):
        # new seeded inputs for every call; returns their host values
        rr = np.random.default_rng(5000 + rep)
        h = {}
        for k, shp in shapes_in.items():
            h[k] = synth.round_to(rr.standard_normal(shp), "bf16")
            ins[k].copy_(to_dev(h[k], bf))
        h["A"] = rr.standard_normal((4, 37, 53)).astype(np.float32).astype(np.float64)
        h["B"] = rr.standard_normal((4, 53, 29)).astype(np.float32).astype(np.float64)
        A.copy_(torch.from_numpy(h["A"].astype(np.float32)))
        B.copy_(torch.from_numpy(h["B"].astype(np.float32)))
        h["xq"] = rr.integers(-128, 128, (77, 200)).astype(np.int8)
        xq.copy_(torch.from_numpy(h["xq"]))
        for t in outs:
            t.fill_(float("nan"))
        Yq.fill_(0)
        torch.cuda.synchronize()
        return h

    def oracle_refs(h):
        # what each call computes, from the same inputs, by the oracle
        _, yq = oracle.gemm_int8(h["xq"], qt["wq"], qt["bias_q"], qt["x_zp"], qt["x_s"], qt["w_s"],
                                 qt["y_s"], qt["y_zp"])
        return [
            ("conv3x3", oracle.conv2d(h["X0"], W1h, b1h, (1, 1), (1, 1, 1, 1), act="relu"), "bf16"),
            ("depthwise", oracle.conv2d(h["X1"], Wdh, bdh, (1, 1), (1, 1, 1, 1), group=M, act="relu6"),
             "bf16"),
            ("1x1+residual", oracle.conv2d(h["X2"], Wph, bph, act="relu", residual=h["R2"]), "bf16"),
            ("maxpool", oracle.maxpool2d(h["X3"], (3, 3), (2, 2), (1, 1, 1, 1)), "bf16"),
            ("bn+relu", oracle.batchnorm_act(h["X4"], gh, beh, muh, varh, 1e-5, "relu"), "bf16"),
            ("gap", oracle.global_avgpool(h["X5"]), "bf16"),
            ("gemm+gelu", oracle.gemm(h["X6"], Bgh, bgh, act="gelu"), "bf16"),
            ("matmul", oracle.matmul(h["A"], h["B"]), "f32"),
            ("split-K gemm", oracle.gemm(h["Ag"], Bsh, None, transB=True, act="relu"), "bf16"),
            ("int8 gemm", yq, None),
        ]

    say("graph chain: warm-up and capture")
    refill(0)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        chain()                       # warm-up on the capture stream
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        chain()
    torch.cuda.synchronize()

    for rep in range(1, 5):
        say("graph chain replay", rep)
        h = refill(rep)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs + [Yq]]
        for (name, ref, dt), x in zip(oracle_refs(h), got):
            if dt is None:
                assert np.array_equal(x.cpu().numpy(), ref), "replay %d %s" % (rep, name)
            else:
                xh = x.double().cpu().numpy()
                assert not np.isnan(xh).any(), name
                assert_close(xh, ref.reshape(xh.shape), dt, "replay %d %s" % (rep, name))
        refill(rep)
        with torch.cuda.stream(s):
            chain()
        s.synchronize()
        eager = outs + [Yq]
        for i, (x, e) in enumerate(zip(got, eager)):
            assert not torch.isnan(e.float()).any().item(), i
            assert torch.equal(x, e), "replay %d output %d differs from eager" % (rep, i)
        assert Y7.float().abs().sum().item() > 0
