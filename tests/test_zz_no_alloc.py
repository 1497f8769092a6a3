"""The allocation-free convolution entry point (ox_conv2d_fused_static):
its scratch is the library's static device array, so a split-K plan runs
with no workspace argument.  Its results must equal those of the entry
point with a caller workspace (ox_conv2d_fused_ws), the same kernels and
plan, on two calls in a row -- the second on a smaller input -- and be
within the bf16 tolerance of the oracle."""
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


def dev(a64):
    return torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32)).cuda().to(torch.bfloat16)


def layer_tensors(layer, li):
    t = synth.conv_inputs(layer, 3, li)
    Wf, bf = oracle.fold_batchnorm(t["W"], t["gamma"], t["beta"], t["mean"], t["var"], 1e-5)
    return synth.round_to(t["X"], "bf16"), synth.round_to(Wf, "bf16"), synth.round_to(bf, "bf16")


# the ResNet-50 stage-4 layers whose plans split the channel range (3x3 on
# the LDS-patch kernel, the 2048 -> 512 1x1 on the pointwise kernel), each
# called at batch 32 and then at a smaller batch
CASES = [("s4.3x3", 512, 7, 512, 3, 1, 32, 8), ("s4.3x3s2", 512, 14, 512, 3, 2, 32, 4),
         ("s4.1x1a", 2048, 7, 512, 1, 1, 32, 12)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_static_scratch_matches_workspace_entry_point(case):
    import conv_implicit_gemm_amd as ox
    name, Cin, H, M, k, s, n_big, n_small = case
    assert ox.ox_static_scratch_bytes() == 32 << 20
    for N in (n_big, n_small):
        layer = synth.ConvLayer(name, N, Cin, H, H, M, k, s, k // 2, 1, "relu")
        X, Wt, b = layer_tensors(layer, 7 + N)
        pads = layer.onnx_pads
        need = ox.ox_conv2d_workspace_bytes("bf16", N, Cin, H, H, M, k, k, (s, s), pads)
        if N == n_big:
            assert 0 < need <= ox.ox_static_scratch_bytes(), (name, need)
        ho, wo = ox.conv_out_hw(H, H, k, k, (s, s), pads, (1, 1))
        Xd, Wd, bd = dev(X), dev(Wt), dev(b)
        say("static scratch", name, "N", N, "workspace bytes", need)
        Ys = torch.full((N, M, ho, wo), float("nan"), dtype=torch.bfloat16, device="cuda")
        ox.ox_conv2d_fused_static(Xd, Wd, bd, (s, s), pads, act="relu", Y=Ys)
        Yw = torch.full((N, M, ho, wo), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        ox.ox_conv2d_fused(Xd, Wd, bd, (s, s), pads, act="relu", Y=Yw, workspace=ws)
        torch.cuda.synchronize()
        assert not torch.isnan(Ys.float()).any().item()
        # the same kernels and plan: bit for bit
        assert torch.equal(Ys.view(torch.int16), Yw.view(torch.int16)), (name, N)
        ref = oracle.conv2d(X, Wt, b, (s, s), pads, (1, 1), 1, "relu")
        assert_close(Ys.float().cpu().numpy().astype(np.float64), ref, "bf16", "%s N=%d" % (name, N))


def test_static_scratch_packed_weights():
    # the packed-weight form of the 3x3 through the same entry point
    import conv_implicit_gemm_amd as ox
    N, Cin, H, M = 16, 512, 7, 512
    layer = synth.ConvLayer("p", N, Cin, H, H, M, 3, 1, 1, 1, "relu")
    X, Wt, b = layer_tensors(layer, 99)
    Wp = ox.ox_conv2d_pack_weights(synth.f32_to_bf16_bits(Wt.astype(np.float32)), "bf16", N, Cin, H, H, (1, 1), (1, 1, 1, 1))
    Wpd = torch.from_numpy(Wp.view(np.int16)).cuda().view(torch.bfloat16)
    say("static scratch packed")
    Y = torch.full((N, M, H, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ox.ox_conv2d_fused_static(dev(X), Wpd, dev(b), (1, 1), (1, 1, 1, 1), act="relu", Y=Y, packed=True)
    torch.cuda.synchronize()
    ref = oracle.conv2d(X, Wt, b, (1, 1), (1, 1, 1, 1), (1, 1), 1, "relu")
    assert_close(Y.float().cpu().numpy().astype(np.float64), ref, "bf16", "static packed")
