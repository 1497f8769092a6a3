"""HIP graph capture of a chain of libox calls.

Every entry point launches kernels only (no allocation, no memset, no host
synchronisation), so a caller may record a whole layer chain into one HIP
graph and replay it.  The test captures such a chain (a split-K 3x3 conv with
its workspace, a depthwise conv, a residual pointwise conv, MaxPool,
BatchNorm + ReLU, GlobalAveragePool, a Gemm + GELU, a batched f32 MatMul, an
int8 Gemm and a split-K Gemm with its workspace), then replays it several
times with new inputs; between replays the outputs are refilled with NaN and
the same chain runs eagerly on the same buffers.  Each replay must equal the eager results bit for bit (the same
kernels with the same launch shapes and a fixed summation order), and the
MatMul is also checked against the oracle."""
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


def test_captured_chain_replays_match_eager():
    import conv_implicit_gemm_amd as ox
    bf = torch.bfloat16
    r = np.random.default_rng(4242)
    N, C, H = 2, 256, 7            # the 3x3 conv of this shape is planned split-K
    M = 128
    Hp = 4                         # MaxPool 3x3 s2 p1 of 7x7

    def wt(*shape, scale):
        return to_dev(synth.round_to(r.standard_normal(shape) * scale, "bf16"), bf)

    # weights and parameters (fixed across replays)
    W1, b1 = wt(M, C, 3, 3, scale=0.05), wt(M, scale=0.1)
    Wd, bd = wt(M, 1, 3, 3, scale=0.3), wt(M, scale=0.1)
    Wp, bp = wt(M, M, 1, 1, scale=0.08), wt(M, scale=0.1)
    gam = torch.from_numpy(r.uniform(0.5, 1.5, M).astype(np.float32)).cuda()
    bet = torch.from_numpy((r.standard_normal(M) * 0.3).astype(np.float32)).cuda()
    mu = torch.from_numpy((r.standard_normal(M) * 0.3).astype(np.float32)).cuda()
    var = torch.from_numpy(r.uniform(0.5, 1.5, M).astype(np.float32)).cuda()
    Bg, bg = wt(M, 300, scale=0.1), wt(300, scale=0.1)
    ws_bytes = ox.ox_conv2d_workspace_bytes("bf16", N, C, H, H, M, 3, 3, (1, 1), (1, 1, 1, 1))
    assert ws_bytes > 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    qlayer = synth.Int8Layer("g", "gemm", 77, 200, 45)
    qt = synth.int8_inputs(qlayer, 4, 61)
    qblk = torch.from_numpy(ox.ox_int8_prepare(qt["wq"], qt["w_s"], qt["x_s"], qt["x_zp"], qt["y_s"],
                                               qt["y_zp"], qt["bias_q"])).cuda()
    wq = torch.from_numpy(qt["wq"]).cuda()
    # a split-K Gemm with its workspace (64 rows, K = 2048)
    Ag = wt(64, 2048, scale=1.0)
    Bs = wt(256, 2048, scale=0.02)
    gws_bytes = ox.ox_gemm_workspace_bytes("bf16", 64, 256, 2048)
    assert gws_bytes > 0
    gws = torch.empty(gws_bytes // 4, dtype=torch.float32, device="cuda")

    # inputs (refilled before every run) and outputs (fixed addresses)
    X0 = torch.empty((N, C, H, H), dtype=bf, device="cuda")
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
        ox.ox_conv2d_fused(X0, W1, b1, (1, 1), (1, 1, 1, 1), act="relu", Y=Y1, stream=s, workspace=ws)
        ox.ox_conv2d_fused(Y1, Wd, bd, (1, 1), (1, 1, 1, 1), group=M, act="relu6", Y=Y2, stream=s)
        ox.ox_conv2d_fused_res(Y2, Wp, Y1, bp, act="relu", Y=Y3, stream=s)
        ox.ox_maxpool2d(Y3, (3, 3), (2, 2), (1, 1, 1, 1), Y=Y4, stream=s)
        ox.ox_batchnorm_act(Y4, gam, bet, mu, var, 1e-5, "relu", Y=Y5, stream=s)
        ox.ox_global_avgpool(Y5, Y=Y6, stream=s)
        ox.ox_gemm_fused(Y6.view(N, M), Bg, bg, act="gelu", Y=Y7, stream=s)
        ox.ox_matmul_batched(A, B, Cm, stream=s)
        ox.ox_gemm_fused(xq, wq, transB=True, int8_params=qblk, out_dtype=torch.int8, Y=Yq, stream=s)
        ox.ox_gemm_fused_ws(Ag, Bs, gws, transB=True, act="relu", Y=Ys, stream=s)

    def refill(rep):
        rr = np.random.default_rng(5000 + rep)
        X0.copy_(to_dev(synth.round_to(rr.standard_normal((N, C, H, H)), "bf16"), bf))
        a64 = rr.standard_normal((4, 37, 53))
        b64 = rr.standard_normal((4, 53, 29))
        A.copy_(torch.from_numpy(a64.astype(np.float32)))
        B.copy_(torch.from_numpy(b64.astype(np.float32)))
        xq.copy_(torch.from_numpy(rr.integers(-128, 128, (77, 200)).astype(np.int8)))
        for t in outs:
            t.fill_(float("nan"))
        Yq.fill_(0)
        torch.cuda.synchronize()
        return a64.astype(np.float32).astype(np.float64), b64.astype(np.float32).astype(np.float64)

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
        a64, b64 = refill(rep)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs + [Yq]]
        assert_close(Cm.double().cpu().numpy(), oracle.matmul(a64, b64), "f32", "replay matmul")
        refill(rep)
        with torch.cuda.stream(s):
            chain()
        s.synchronize()
        eager = outs + [Yq]
        for i, (x, e) in enumerate(zip(got, eager)):
            assert not torch.isnan(e.float()).any().item(), i
            assert torch.equal(x, e), "replay %d output %d differs from eager" % (rep, i)
        assert Y7.float().abs().sum().item() > 0
