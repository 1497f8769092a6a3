"""GPU parity: libox's HIP kernels against the CPU oracle, element by element
on the same seeded inputs (the rule and tolerances are in tests/parity.py).

Every comparison covers every output element, the full-size workload
layers included (after checking that no output was left at its NaN
sentinel)."""
import math
import sys

import numpy as np
import pytest

import oracle
import synth
from kernel_rules import dwr_applies
from parity import assert_close

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ox():
    import conv_implicit_gemm_amd as ox
    return ox


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(a64, dtype):
    """float64 numpy holding values exact in `dtype` -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32)).to("cuda").to(TD[dtype])


def host64(t):
    return t.float().cpu().numpy().astype(np.float64)


def nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=TD[dtype], device="cuda")


# ------------------------------------------------------------------ MatMul --

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_ones_64_cube_every_element_is_64(ox, dtype):
    # "OxiONNX 0.1.7 Released": the 64x64x64 all-ones MatMul that its
    # two-stream race returned with 3456 of 4096 elements reading 0.0.  Here
    # the output starts as NaN, the call runs on a non-default stream, and only
    # that stream is synchronised.
    say("all-ones 64^3", dtype)
    A = torch.ones((1, 64, 64), dtype=TD[dtype], device="cuda")
    s = torch.cuda.Stream()
    Cm = nan_like((1, 64, 64), dtype)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ox.ox_matmul_batched(A, A, Cm, stream=s)
        Y = nan_like((64, 64), dtype)
        ox.ox_gemm_fused(A[0], A[0], transB=True, Y=Y, stream=s)
    s.synchronize()
    assert torch.all(Cm == 64).item() and torch.all(Y == 64).item()


def test_matmul_c0_seeded_against_oracle(ox):
    say("C0 batched matmul [16,64,128]x[16,128,64] f32")
    A, B = synth.matmul_inputs()
    Cg = ox.ox_matmul_batched(dev(A, "f32"), dev(B, "f32"))
    torch.cuda.synchronize()
    assert_close(host64(Cg), oracle.matmul(A, B), "f32", "C0")


@pytest.mark.parametrize("shape", [(3, 37, 53, 71), (1, 1, 1, 1), (2, 130, 5, 300), (5, 64, 129, 16)])
@pytest.mark.parametrize("bcast", [False, True])
def test_matmul_integer_inputs_are_exact(ox, shape, bcast):
    batch, M, N, K = shape
    say("matmul exact", shape, "bcast", bcast)
    r = np.random.default_rng(sum(shape) + bcast)
    A = r.integers(-3, 4, (batch, M, K)).astype(np.float64)
    B = r.integers(-3, 4, (1 if bcast else batch, K, N)).astype(np.float64)
    Cg = ox.ox_matmul_batched(dev(A, "f32"), dev(B, "f32"))
    torch.cuda.synchronize()
    assert np.array_equal(host64(Cg), oracle.matmul(A, B))
    Cb = ox.ox_matmul_batched(dev(A, "bf16"), dev(B, "bf16"))
    torch.cuda.synchronize()
    ref = oracle.matmul(A, B)
    # |sums| < 256 are exact in bf16
    exact = np.abs(ref) < 256
    assert np.array_equal(host64(Cb)[exact], ref[exact])


# -------------------------------------------------------------------- Gemm --

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("act", ["none", "relu", "gelu", "relu6"])
def test_gemm_layouts_and_scalars(ox, dtype, ta, tb, act):
    M, N, K = 77, 45, 133
    say("gemm", dtype, ta, tb, act)
    r = np.random.default_rng(100 + 8 * ta + 4 * tb + len(act))
    A = synth.round_to(r.standard_normal((K, M) if ta else (M, K)), dtype)
    B = synth.round_to(r.standard_normal((N, K) if tb else (K, N)) / math.sqrt(K), dtype)
    bias = synth.round_to(r.uniform(-1, 1, N), dtype)
    Y = nan_like((M, N), dtype)
    ox.ox_gemm_fused(dev(A, dtype), dev(B, dtype), dev(bias, dtype), alpha=0.5, beta=-2.0,
                     transA=bool(ta), transB=bool(tb), act=act, Y=Y)
    torch.cuda.synchronize()
    ref = oracle.gemm(A, B, bias, 0.5, -2.0, ta, tb, act)
    assert_close(host64(Y), ref, dtype, "gemm")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_gemm_long_k_few_tiles(ox, dtype, ta, tb):
    # few output tiles and a long, ragged K: the small tiles with four K
    # units per stage, in every operand layout
    M, N, K = 64, 200, 1500
    say("gemm long K", dtype, ta, tb)
    r = np.random.default_rng(150 + 2 * ta + tb)
    A = synth.round_to(r.standard_normal((K, M) if ta else (M, K)), dtype)
    B = synth.round_to(r.standard_normal((N, K) if tb else (K, N)) / math.sqrt(K), dtype)
    bias = synth.round_to(r.uniform(-1, 1, N), dtype)
    Y = nan_like((M, N), dtype)
    ox.ox_gemm_fused(dev(A, dtype), dev(B, dtype), dev(bias, dtype), transA=bool(ta),
                     transB=bool(tb), act="gelu", Y=Y)
    torch.cuda.synchronize()
    assert_close(host64(Y), oracle.gemm(A, B, bias, 1.0, 1.0, ta, tb, "gelu"), dtype, "gemm long K")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_gemm_split_k_workspace(ox, dtype, ta, tb):
    # few output tiles, long K: K slices with fp32 partials in the caller's
    # workspace, then the ordered sum with alpha, beta*bias and GELU; ragged K
    # (a short last slice) and the MLP's 4096-deep row shape (split-K is
    # planned from 64 K units on)
    for (M, N, K) in [(64, 200, 2600), (64, 1024, 4096), (37, 70, 2777)]:
        say("gemm split-K", dtype, ta, tb, (M, N, K))
        r = np.random.default_rng(170 + 2 * ta + tb + K)
        A = synth.round_to(r.standard_normal((K, M) if ta else (M, K)), dtype)
        B = synth.round_to(r.standard_normal((N, K) if tb else (K, N)) / math.sqrt(K), dtype)
        bias = synth.round_to(r.uniform(-1, 1, N), dtype)
        nb = ox.ox_gemm_workspace_bytes(dtype, M, N, K)
        assert nb > 0
        ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device="cuda")
        Y = nan_like((M, N), dtype)
        ox.ox_gemm_fused_ws(dev(A, dtype), dev(B, dtype), ws, dev(bias, dtype), alpha=0.75, beta=-1.5,
                            transA=bool(ta), transB=bool(tb), act="gelu", Y=Y)
        torch.cuda.synchronize()
        ref = oracle.gemm(A, B, bias, 0.75, -1.5, ta, tb, "gelu")
        assert_close(host64(Y), ref, dtype, "gemm split-K")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tb", [0, 1])
@pytest.mark.parametrize("force", [None, "mfma"])
def test_gemm_single_row(ox, dtype, tb, force, monkeypatch):
    if force:
        monkeypatch.setenv("OX_FORCE_KERNEL", force)
    M, N, K = 1, 1000, 777
    say("gemm M=1", dtype, tb, force)
    r = np.random.default_rng(7 + tb)
    A = synth.round_to(r.standard_normal((M, K)), dtype)
    B = synth.round_to(r.standard_normal((N, K) if tb else (K, N)) / math.sqrt(K), dtype)
    bias = synth.round_to(r.uniform(-0.1, 0.1, N), dtype)
    Y = nan_like((M, N), dtype)
    ox.ox_gemm_fused(dev(A, dtype), dev(B, dtype), dev(bias, dtype), transB=bool(tb), act="gelu", Y=Y)
    torch.cuda.synchronize()
    assert_close(host64(Y), oracle.gemm(A, B, bias, transB=tb, act="gelu"), dtype, "gemv")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemv_rows_per_block(ox, dtype):
    # the M = 1 kernel over [N, K] weights: 1, 2, 4 and 8 rows per block
    # (N = 1000, 1024, 2048, 4097: a partial last block), 16-byte rows whose
    # chunk count is or is not a multiple of the four K quarters, rows that
    # are not 16-byte aligned (element path), K below one chunk per lane
    r = np.random.default_rng(31)
    for N, K in ((1000, 1000), (1024, 4096), (2048, 1032), (4097, 1024), (1024, 1001), (64, 24), (3, 4100)):
        say("gemv", dtype, N, K)
        A = synth.round_to(r.standard_normal((1, K)), dtype)
        B = synth.round_to(r.standard_normal((N, K)) / math.sqrt(K), dtype)
        bias = synth.round_to(r.uniform(-0.1, 0.1, N), dtype)
        Y = nan_like((1, N), dtype)
        ox.ox_gemm_fused(dev(A, dtype), dev(B, dtype), dev(bias, dtype), transB=True, act="relu", Y=Y)
        torch.cuda.synchronize()
        assert_close(host64(Y), oracle.gemm(A, B, bias, transB=True, act="relu"), dtype, "gemv %d x %d" % (N, K))


def test_gemm_empty_reduction_writes_activation_of_bias(ox):
    say("gemm K=0")
    bias = np.array([-1.0, 0.5, 7.0], np.float64)
    Y = nan_like((4, 3), "f32")
    A = torch.empty((4, 0), device="cuda")
    B = torch.empty((3, 0), device="cuda")
    ox.ox_gemm_fused(A, B, dev(bias, "f32"), beta=1.0, transB=True, act="relu6", Y=Y)
    torch.cuda.synchronize()
    assert np.array_equal(host64(Y), np.broadcast_to(oracle.act("relu6", bias), (4, 3)))


GEMM_STAGES = ["1x1", "4x1", "2x2"]
GEMM_TILES = ["128x128", "64x128", "128x64", "64x64", "32x64"]


@pytest.mark.parametrize("stages", GEMM_STAGES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gemm_stage_shapes(ox, stages, dtype, monkeypatch):
    # every stage shape (K units per stage x stages in flight) on every tile
    # and operand layout: K of one stage, of fewer stages than are kept in
    # flight, and of many with a ragged tail; rows and columns past the
    # operands; one output row
    monkeypatch.setenv("OX_GEMM_STAGES", stages)
    r = np.random.default_rng(260 + GEMM_STAGES.index(stages) + (dtype == "bf16"))
    for tile in GEMM_TILES:
        monkeypatch.setenv("OX_FORCE_KERNEL", "mfma,tile=" + tile)
        for (M, N, K) in [(150, 140, 1000), (70, 130, 40), (33, 200, 392), (1, 70, 520)]:
            for ta, tb in [(0, 1), (0, 0), (1, 1), (1, 0)]:
                say("gemm stages", stages, tile, dtype, (M, N, K), ta, tb)
                A = synth.round_to(r.standard_normal((K, M) if ta else (M, K)), dtype)
                B = synth.round_to(r.standard_normal((N, K) if tb else (K, N)) / math.sqrt(K), dtype)
                bias = synth.round_to(r.uniform(-1, 1, N), dtype)
                Y = nan_like((M, N), dtype)
                ox.ox_gemm_fused(dev(A, dtype), dev(B, dtype), dev(bias, dtype), alpha=0.5, beta=-2.0,
                                 transA=bool(ta), transB=bool(tb), act="relu", Y=Y)
                torch.cuda.synchronize()
                ref = oracle.gemm(A, B, bias, 0.5, -2.0, ta, tb, "relu")
                assert_close(host64(Y), ref, dtype, "gemm %s %s %s" % (stages, tile, (M, N, K, ta, tb)))


@pytest.mark.parametrize("stages", GEMM_STAGES)
def test_qgemm_stage_shapes_bit_exact(ox, stages, monkeypatch):
    # the int8 Gemm under every stage shape and tile, with uint8 activations
    # (flipped on their way to LDS) and weight zero points (row sums taken
    # from the staged operand)
    monkeypatch.setenv("OX_GEMM_STAGES", stages)
    r = np.random.default_rng(280 + GEMM_STAGES.index(stages))
    for tile in GEMM_TILES:
        monkeypatch.setenv("OX_FORCE_KERNEL", "mfma,tile=" + tile)
        for (xu, yu, wz) in [(True, False, True), (False, True, False)]:
            for (M, K, N) in [(150, 1088, 140), (77, 64, 45), (40, 448, 70)]:
                say("qgemm stages", stages, tile, (xu, yu, wz), (M, K, N))
                x, w, wzp, xzp, bq, x_s, w_s = q_inputs(r, xu, wz, (M, K), (N, K))
                acc0, _ = oracle.qgemm(x, w, bq, xzp, wzp, x_s, w_s, 1.0, 0)
                y_s = q_out_scale(acc0, x_s, w_s)
                yzp = int(r.integers(0, 256)) if yu else int(r.integers(-128, 128))
                acc, y = oracle.qgemm(x, w, bq, xzp, wzp, x_s, w_s, y_s, yzp, yu)
                blk = ox.ox_int8_prepare(w, w_s, x_s, xzp, y_s, yzp, bq, w_zp=wzp, x_unsigned=xu,
                                         y_unsigned=yu)

                def call(xd, wd, bd, yt):
                    od = {"i32": torch.int32, "u8": torch.uint8, "i8": torch.int8}[yt]
                    return ox.ox_gemm_fused(xd, wd, transB=True, int8_params=bd, out_dtype=od)
                g32, g8 = q_run(ox, blk, x, xu, w, yu, call)
                assert np.array_equal(g32, acc), (stages, tile, M, K, N)
                assert np.array_equal(g8, y), (stages, tile, M, K, N)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_c1_mlp_rows(ox, dtype):
    # every row through the plain Gemm and through the split-K Gemm with a
    # NaN-filled workspace of the size the library asks for (the benchmark's
    # call), every output against the oracle
    for li, row in enumerate(synth.mlp_rows()):
        X, W, b = synth.gemm_inputs(row, 1, li)
        X, W, b = (synth.round_to(t, dtype) for t in (X, W, b))
        ref = oracle.gemm(X, W, b, transB=True, act=row.act)
        nb = ox.ox_gemm_workspace_bytes(dtype, row.M, row.N, row.K)
        for use_ws in (False, True):
            say("C1", row.name, dtype, "workspace %d B" % nb if use_ws else "no workspace")
            Y = nan_like((row.M, row.N), dtype)
            if use_ws:
                ws = torch.full((max(nb, 4) // 4,), float("nan"), dtype=torch.float32, device="cuda")
                ox.ox_gemm_fused_ws(dev(X, dtype), dev(W, dtype), ws, dev(b, dtype), transB=True,
                                    act=row.act, Y=Y)
            else:
                ox.ox_gemm_fused(dev(X, dtype), dev(W, dtype), dev(b, dtype), transB=True,
                                 act=row.act, Y=Y)
            torch.cuda.synchronize()
            assert not torch.isnan(Y).any().item()
            assert_close(host64(Y), ref, dtype, row.name)


# -------------------------------------------------------------------- Conv --

def conv_case_ok(N, Cin, H, W, M, kH, kW, s, pads, d, g):
    rc, Ho, Wo = oracle.conv_out_dims(oracle.conv_desc(N, Cin, H, W, M, kH, kW, s, pads, d, g))
    return rc == 0


def sweep(n, seed):
    from test_oracle_pins import sweep_cases
    return [c for c in sweep_cases(n, seed) if conv_case_ok(*c[:11])]


def workspace_for(ox, dtype, N, Cin, H, W, M, kH, kW, s, pads, d, g):
    """A device scratch buffer of the size ox_conv2d_fused_ws asks for (None if 0)."""
    n = ox.ox_conv2d_workspace_bytes(dtype, N, Cin, H, W, M, kH, kW, s, pads, d, g)
    return torch.empty(n, dtype=torch.uint8, device="cuda") if n else None


def run_conv(ox, X, Wt, b, dtype, s, pads, d, g, act, ws=False):
    ho, wo = ox.conv_out_hw(X.shape[2], X.shape[3], Wt.shape[2], Wt.shape[3], s, pads, d)
    Y = nan_like((X.shape[0], Wt.shape[0], ho, wo), dtype)
    wsb = workspace_for(ox, dtype, *X.shape, Wt.shape[0], Wt.shape[2], Wt.shape[3], s, pads, d, g) if ws else None
    ox.ox_conv2d_fused(dev(X, dtype), dev(Wt, dtype), None if b is None else dev(b, dtype),
                       s, pads, d, g, act, Y=Y, workspace=wsb)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("kind", ["1x1", "igemm"])
def test_conv_bf16_pair_stores(ox, kind, monkeypatch):
    # the tile engine's bf16 conv epilogue: with an even output plane and a
    # 4-byte aligned Y, neighbouring lanes exchange values and store pixel
    # pairs; an odd plane or a Y two bytes off alignment takes element
    # stores.  Every tile, ragged channel counts (M not a multiple of 4),
    # pixel ranges that end inside a tile and grouped convolutions; against
    # the oracle, and the pair and element paths bit-identical.
    r = np.random.default_rng(2024 + (kind == "igemm"))
    k = 1 if kind == "1x1" else 3
    pads = (0, 0, 0, 0) if k == 1 else (1, 1, 1, 1)
    for tile in GEMM_TILES:
        monkeypatch.setenv("OX_FORCE_KERNEL", "%s,tile=%s" % (kind, tile))
        for (N, Cin, H, W, M, g) in [(2, 32, 6, 6, 70, 1), (3, 16, 5, 5, 37, 1), (1, 64, 4, 10, 130, 2),
                                     (2, 24, 7, 8, 6, 3), (2, 48, 9, 8, 96, 1)]:
            if kind == "1x1" and g > 1:
                continue      # the 1x1 path takes ungrouped convolutions only
            X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
            Wt = synth.round_to(r.standard_normal((M, Cin // g, k, k)) / math.sqrt(Cin // g * k * k), "bf16")
            b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
            ref = oracle.conv2d(X, Wt, b, (1, 1), pads, (1, 1), g, "relu6")
            outs = []
            for yoff in (0, 1):
                say("bf16 pair stores", kind, tile, (N, Cin, H, W, M, g), "Y offset", yoff)
                Y = misaligned(nan_like((N, M, H, W), "bf16"), yoff)
                ox.ox_conv2d_fused(dev(X, "bf16"), dev(Wt, "bf16"), dev(b, "bf16"), (1, 1), pads, (1, 1), g,
                                   "relu6", Y=Y)
                torch.cuda.synchronize()
                assert_close(host64(Y), ref, "bf16", "%s %s case %s offset %d" % (kind, tile, (N, Cin, H, W, M, g), yoff))
                outs.append(Y.clone())
            assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_1x1_buffer_path(ox, dtype, monkeypatch):
    # 1x1 convolutions on the tile engine through the buffer loaders (fp32
    # columns one by one, bf16 in pixel pairs split into k-chunks as they
    # are written to LDS) with the Gemm's stage shapes: every tile, ragged
    # channels and pixel ranges, tiles straddling images, K tails and a K of
    # one partial unit; against the oracle, and bit-identical to the
    # gathering loader (OX_CONV_PIPE=0: the same sums in the same order)
    r = np.random.default_rng(880 + (dtype == "bf16"))
    for tile in GEMM_TILES:
        for (N, Cin, H, W, M) in [(3, 48, 4, 7, 40), (2, 16, 10, 10, 96), (2, 576, 2, 7, 130),
                                  (1, 1000, 1, 50, 72)]:
            say("conv 1x1 buffer", dtype, tile, (N, Cin, H, W, M))
            X = synth.round_to(r.standard_normal((N, Cin, H, W)), dtype)
            Wt = synth.round_to(r.standard_normal((M, Cin, 1, 1)) / math.sqrt(Cin), dtype)
            b = synth.round_to(r.uniform(-0.5, 0.5, M), dtype)
            monkeypatch.setenv("OX_FORCE_KERNEL", "1x1,tile=" + tile)
            out = {}
            for pipe in ("1", "0"):
                monkeypatch.setenv("OX_CONV_PIPE", pipe)
                out[pipe] = host64(run_conv(ox, X, Wt, b, dtype, (1, 1), (0, 0, 0, 0), (1, 1), 1, "relu"))
            assert_close(out["1"], oracle.conv2d(X, Wt, b, act="relu"), dtype, "1x1 buffer %s" % tile)
            assert np.array_equal(out["1"], out["0"]), (tile, (N, Cin, H, W, M))
            monkeypatch.delenv("OX_CONV_PIPE")
            monkeypatch.delenv("OX_FORCE_KERNEL")


def test_conv_igemm_f32_buffer_path(ox, monkeypatch):
    # fp32 implicit GEMM through the buffer loaders (each element's offset
    # from its (c, kh, kw), padding taps and k past K read as zeros) with the
    # Gemm's stage shapes: every tile, strides, pads, dilation, groups,
    # kernels of 1 to 7 taps a side; against the oracle and bit-identical to
    # the gathering loader (OX_CONV_PIPE=0: the same sums in the same order)
    r = np.random.default_rng(890)
    geoms = [(2, 16, 9, 11, 24, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1),
             (1, 12, 13, 10, 20, 3, 3, (2, 2), (2, 1, 0, 1), (1, 1), 2),
             (2, 8, 12, 12, 8, 3, 3, (1, 1), (2, 2, 2, 2), (2, 2), 1),
             (2, 64, 14, 14, 96, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1),
             (1, 3, 30, 30, 16, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1), 1),
             (1, 130, 7, 7, 70, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1),
             (2, 20, 8, 9, 30, 1, 3, (1, 2), (0, 1, 0, 1), (1, 1), 1)]
    for tile in GEMM_TILES:
        for (N, Cin, H, W, M, kh, kw, st, pads, dil, g) in geoms:
            say("igemm f32 buffer", tile, (N, Cin, H, W, M, kh, kw, st, pads, dil, g))
            X = synth.round_to(r.standard_normal((N, Cin, H, W)), "f32")
            Wt = synth.round_to(r.standard_normal((M, Cin // g, kh, kw)) / math.sqrt(Cin // g * kh * kw), "f32")
            b = synth.round_to(r.uniform(-0.5, 0.5, M), "f32")
            monkeypatch.setenv("OX_FORCE_KERNEL", "igemm,tile=" + tile)
            out = {}
            for pipe in ("1", "0"):
                monkeypatch.setenv("OX_CONV_PIPE", pipe)
                out[pipe] = host64(run_conv(ox, X, Wt, b, "f32", st, pads, dil, g, "relu"))
            assert_close(out["1"], oracle.conv2d(X, Wt, b, st, pads, dil, g, act="relu"), "f32",
                         "igemm buffer %s" % tile)
            assert np.array_equal(out["1"], out["0"]), (tile, (N, Cin, H, W, M, kh, kw))
            monkeypatch.delenv("OX_CONV_PIPE")
            monkeypatch.delenv("OX_FORCE_KERNEL")


def test_conv_sweep_integer_inputs_exact(ox):
    # fp32 with small integer inputs: every partial sum is exact, so any
    # indexing mistake (tap, pad, stride, dilation, group) shows as a mismatch.
    cases = sweep(400, 77)
    for ci, (N, Cin, H, W, M, kH, kW, s, pads, d, g, act) in enumerate(cases):
        act = "relu6" if act == "gelu" else act
        r = np.random.default_rng(ci)
        X = r.integers(-3, 4, (N, Cin, H, W)).astype(np.float64)
        Wt = r.integers(-2, 3, (M, Cin // g, kH, kW)).astype(np.float64)
        b = r.integers(-4, 5, M).astype(np.float64)
        say("conv sweep", ci, (N, Cin, H, W, M, kH, kW, s, pads, d, g, act))
        Y = run_conv(ox, X, Wt, b, "f32", s, pads, d, g, act)
        ref = oracle.conv2d(X, Wt, b, s, pads, d, g, act)
        assert np.array_equal(host64(Y), ref), (ci, N, Cin, H, W, M, kH, kW, s, pads, d, g, act)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_sweep_random_inputs(ox, dtype):
    cases = sweep(250, 4242)
    for ci, (N, Cin, H, W, M, kH, kW, s, pads, d, g, act) in enumerate(cases):
        r = np.random.default_rng(1000 + ci)
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), dtype)
        Wt = synth.round_to(r.standard_normal((M, Cin // g, kH, kW)) / math.sqrt(kH * kW * Cin // g), dtype)
        b = synth.round_to(r.uniform(-0.5, 0.5, M), dtype)
        say("conv sweep", dtype, ci, (N, Cin, H, W, M, kH, kW, s, pads, d, g, act))
        Y = run_conv(ox, X, Wt, b, dtype, s, pads, d, g, act)
        assert_close(host64(Y), oracle.conv2d(X, Wt, b, s, pads, d, g, act), dtype, str(ci))


@pytest.mark.parametrize("force", [None, "dw", "igemm"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("geom", [
    (2, 24, 19, 23, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)),
    (1, 40, 17, 18, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1)),
    (1, 16, 1, 50, 1, 9, (1, 1), (0, 4, 0, 4), (1, 1)),
    (3, 8, 13, 11, 5, 3, (2, 1), (2, 0, 1, 2), (2, 1)),
])
def test_depthwise_variants(ox, force, dtype, geom, monkeypatch):
    if force:
        monkeypatch.setenv("OX_FORCE_KERNEL", force)
    N, Cc, H, W, kH, kW, s, pads, d = geom
    say("depthwise", geom, dtype, force)
    r = np.random.default_rng(H * W + Cc)
    X = synth.round_to(r.standard_normal((N, Cc, H, W)), dtype)
    Wt = synth.round_to(r.standard_normal((Cc, 1, kH, kW)) / 3.0, dtype)
    b = synth.round_to(r.uniform(-0.5, 0.5, Cc), dtype)
    Y = run_conv(ox, X, Wt, b, dtype, s, pads, d, Cc, "relu6")
    assert_close(host64(Y), oracle.conv2d(X, Wt, b, s, pads, d, Cc, "relu6"), dtype, "dw")


@pytest.mark.parametrize("geom", [
    # N, C, H, W, kH, kW, stride, pads, Y offset (elements), OX_DW_TARGET
    (1, 3, 900, 4, 3, 3, 1, (1, 1, 1, 1), 0, 4096),     # runs of 4 rows, every strip full
    (2, 2, 600, 10, 3, 3, 1, (1, 1, 1, 1), 0, 4096),    # runs of 4 rows, partial last strips
    (1, 2, 64, 512, 3, 3, 2, (1, 1, 1, 1), 0, 2048),    # stride 2, runs of 2 rows
    (1, 2, 40, 256, 3, 3, 1, (1, 1, 1, 1), 0, 8192),    # strips of 8, runs of 3 rows
    (1, 2, 40, 256, 3, 3, 1, (1, 1, 1, 1), 1, 8192),    # the same, Y one element past alignment
    (2, 2, 40, 64, 1, 9, 1, (0, 4, 0, 4), 0, 2048),     # 1-D kernel, one window row
    (2, 5, 21, 40, 3, 3, 1, (1, 1, 1, 1), 0, 64),       # bands of one row
])
def test_depthwise_sliding_strips(ox, geom, monkeypatch):
    # one plane per block (block sizes pinned with OX_DW_TARGET): the
    # sliding-window strips over runs of rows (the window's rows rotating
    # through their register slots), runs that start inside a band, and the
    # store paths with and without the all-aligned fast path; bf16 and int8
    N, Cc, H, W, kH, kW, s, pads, yoff, target = geom
    monkeypatch.setenv("OX_DW_TARGET", str(target))
    say("depthwise sliding", geom)
    r = np.random.default_rng(H * 7 + W + target)
    X = synth.round_to(r.standard_normal((N, Cc, H, W)), "bf16")
    Wt = synth.round_to(r.standard_normal((Cc, 1, kH, kW)) / 3.0, "bf16")
    b = synth.round_to(r.uniform(-0.5, 0.5, Cc), "bf16")
    ho, wo = ox.conv_out_hw(H, W, kH, kW, (s, s), pads, (1, 1))
    Y = misaligned(nan_like((N, Cc, ho, wo), "bf16"), yoff)
    monkeypatch.setenv("OX_FORCE_KERNEL", "dw")
    ox.ox_conv2d_fused(dev(X, "bf16"), dev(Wt, "bf16"), dev(b, "bf16"), (s, s), pads, (1, 1), Cc, "relu6", Y=Y)
    torch.cuda.synchronize()
    monkeypatch.delenv("OX_FORCE_KERNEL")
    assert_close(host64(Y), oracle.conv2d(X, Wt, b, (s, s), pads, (1, 1), Cc, "relu6"), "bf16", "dw slide")
    conv = synth.ConvLayer("q", N, Cc, H, W, Cc, kH, s, 0, Cc, "none", kW=kW, pads=pads)
    layer = synth.Int8Layer("q", "conv", 1, kH * kW, Cc, conv)
    t = synth.int8_inputs(layer, 4, 80 + H + W)
    acc, y = int8_ref(layer, t)
    assert np.array_equal(int8_gpu(ox, layer, t, "i32").astype(np.int64), acc)
    assert np.array_equal(int8_gpu(ox, layer, t, "i8"), y)


@pytest.mark.parametrize("force", [None, "dw"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("geom", [
    (2, 20, 14, 14, (1, 1), 1),     # Wo = 14: rows alternate between aligned and unaligned strips
    (3, 12, 7, 7, (1, 1), 0),       # Wo = 7: one full strip and a tail per row
    (2, 16, 28, 28, (2, 2), 3),     # output pointer 3 elements past an aligned one
    (1, 8, 9, 16, (1, 1), 2),
])
def test_depthwise_output_alignment(ox, force, dtype, geom, monkeypatch):
    # the staged-band kernel (forced) stores strips of 4 outputs as one wide
    # store only where they are full and aligned, every other strip element
    # by element; the row kernel (chosen where it applies) stores a lane's
    # segment whole only where Y is aligned to it
    if force:
        monkeypatch.setenv("OX_FORCE_KERNEL", force)
    N, Cc, H, W, s, yoff = geom
    say("depthwise alignment", geom, dtype)
    r = np.random.default_rng(H * 31 + yoff)
    X = synth.round_to(r.standard_normal((N, Cc, H, W)), dtype)
    Wt = synth.round_to(r.standard_normal((Cc, 1, 3, 3)) / 3.0, dtype)
    b = synth.round_to(r.uniform(-0.5, 0.5, Cc), dtype)
    ho, wo = ox.conv_out_hw(H, W, 3, 3, s, (1, 1, 1, 1), (1, 1))
    Y = misaligned(nan_like((N, Cc, ho, wo), dtype), yoff)
    ox.ox_conv2d_fused(dev(X, dtype), dev(Wt, dtype), dev(b, dtype), s, (1, 1, 1, 1), (1, 1), Cc, "relu6", Y=Y)
    torch.cuda.synchronize()
    assert_close(host64(Y), oracle.conv2d(X, Wt, b, s, (1, 1, 1, 1), (1, 1), Cc, "relu6"), dtype, "dw align")


DWR_CASES = [
    # N, C, H, W, stride: one to nine bands per wave, ragged last bands (odd
    # heights), rows of 1 to 64 lanes, odd output widths (stride 2), tiny
    # planes, one band per wave at 64 lanes a row
    (2, 8, 112, 112, 1), (1, 6, 112, 112, 2), (3, 16, 56, 56, 1), (2, 24, 56, 56, 2),
    (4, 32, 28, 28, 1), (2, 48, 14, 14, 1), (3, 40, 14, 14, 2), (2, 64, 7, 8, 1),
    (1, 5, 9, 10, 1), (2, 3, 13, 6, 2), (1, 2, 1, 2, 1), (2, 7, 3, 2, 2), (1, 300, 4, 4, 1),
    (1, 2, 6, 512, 1), (1, 3, 900, 4, 1), (2, 5, 21, 40, 1),
]
# odd widths at stride 1 (lanes of one output each; bf16 2-byte loads),
# up to 63 lanes a row
DWR_ODD = [(2, 12, 7, 7, 1), (1, 3, 5, 9, 1), (2, 5, 11, 23, 1), (1, 4, 6, 63, 1)]


@pytest.mark.parametrize("tr,vmax", [(None, None), ("4", None), ("8", None), ("8", "2"), ("4", "1")])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dwr_cases(ox, dtype, tr, vmax, monkeypatch):
    # the row-segment depthwise kernel, forced, with each band height and
    # narrower segments; fp32 on integer values is exact, bf16 on random
    # values within tolerance; every activation.  Where no segment width
    # applies, the forced call is refused.
    monkeypatch.setenv("OX_FORCE_KERNEL", "dwr")
    if tr:
        monkeypatch.setenv("OX_DWR_TR", tr)
    if vmax:
        monkeypatch.setenv("OX_DWR_V", vmax)
    cases = DWR_CASES + DWR_ODD
    for ci, (N, Cc, H, W, st) in enumerate(cases):
        act = ["relu6", "none", "relu", "gelu"][ci % 4]
        r = np.random.default_rng(5100 + ci)
        if dtype == "f32":
            X = r.integers(-4, 5, (N, Cc, H, W)).astype(np.float64)
            Wt = r.integers(-3, 4, (Cc, 1, 3, 3)).astype(np.float64)
            b = r.integers(-5, 6, Cc).astype(np.float64)
            act = "relu" if act == "gelu" else act
        else:
            X = synth.round_to(r.standard_normal((N, Cc, H, W)), "bf16")
            Wt = synth.round_to(r.standard_normal((Cc, 1, 3, 3)) / 3.0, "bf16")
            b = synth.round_to(r.uniform(-0.5, 0.5, Cc), "bf16")
        bias = None if ci == 3 else b
        say("dwr", dtype, tr, vmax, (N, Cc, H, W, st, act))
        if not dwr_applies(dtype, W, st, int(vmax or 8)):
            with pytest.raises(ox.OxError):
                run_conv(ox, X, Wt, bias, dtype, (st, st), (1, 1, 1, 1), (1, 1), Cc, act)
            continue
        Y = run_conv(ox, X, Wt, bias, dtype, (st, st), (1, 1, 1, 1), (1, 1), Cc, act)
        ref = oracle.conv2d(X, Wt, bias, (st, st), (1, 1, 1, 1), (1, 1), Cc, act)
        if dtype == "f32":
            assert np.array_equal(host64(Y), ref), ("dwr", ci)
        else:
            assert_close(host64(Y), ref, dtype, "dwr %d" % ci)


def test_dwr_selection_and_misalignment(ox, monkeypatch):
    # the row kernel is chosen for 3x3 pads-1 depthwise convs it applies to;
    # rows wider than 64 lanes of one output (bf16, odd width), other pads,
    # or an X whose alignment admits no segment load take the staged-band
    # kernel; a Y off its store width is written element by element
    assert ox.ox_conv2d_variant("bf16", 2, 32, 56, 56, 32, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 32).startswith("dwr/")
    assert ox.ox_conv2d_variant("f32", 2, 32, 56, 56, 32, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), 32).startswith("dwr/")
    assert ox.ox_conv2d_variant("f32", 2, 32, 7, 7, 32, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 32).startswith("dwr/")
    assert ox.ox_conv2d_variant("bf16", 2, 32, 7, 7, 32, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 32).startswith("dwr/")
    assert ox.ox_conv2d_variant("bf16", 2, 32, 9, 65, 32, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 32).startswith("dw/")
    assert ox.ox_conv2d_variant("bf16", 2, 32, 8, 8, 32, 3, 3, (1, 1), (0, 0, 0, 0), (1, 1), 32).startswith("dw/")
    assert ox.ox_conv2d_variant("bf16", 1, 4, 8, 1040, 4, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 4).startswith("dw/")
    r = np.random.default_rng(5300)
    X = synth.round_to(r.standard_normal((2, 16, 20, 20)), "bf16")
    Wt = synth.round_to(r.standard_normal((16, 1, 3, 3)) / 3.0, "bf16")
    b = synth.round_to(r.uniform(-0.5, 0.5, 16), "bf16")
    ref = oracle.conv2d(X, Wt, b, (1, 1), (1, 1, 1, 1), (1, 1), 16, "relu6")
    for xoff, yoff in ((0, 1), (0, 2), (0, 4), (0, 8), (1, 0), (2, 3), (4, 0)):
        say("dwr misaligned X/Y", xoff, yoff)
        Xd = misaligned(dev(X, "bf16"), xoff) if xoff else dev(X, "bf16")
        Y = misaligned(nan_like((2, 16, 20, 20), "bf16"), yoff)
        ox.ox_conv2d_fused(Xd, dev(Wt, "bf16"), dev(b, "bf16"), (1, 1), (1, 1, 1, 1), (1, 1), 16,
                           "relu6", Y=Y)
        torch.cuda.synchronize()
        assert_close(host64(Y), ref, "bf16", "dwr xoff %d yoff %d" % (xoff, yoff))


@pytest.mark.parametrize("force", [None, "1x1", "igemm"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pointwise_variants(ox, force, dtype, monkeypatch):
    # C = 40 is not a multiple of 32: the generic 1x1 engine takes it
    if force:
        monkeypatch.setenv("OX_FORCE_KERNEL", force)
    say("1x1", dtype, force)
    r = np.random.default_rng(5)
    X = synth.round_to(r.standard_normal((3, 40, 9, 13)), dtype)
    Wt = synth.round_to(r.standard_normal((70, 40, 1, 1)) / 6.0, dtype)
    b = synth.round_to(r.uniform(-0.5, 0.5, 70), dtype)
    Y = run_conv(ox, X, Wt, b, dtype, (1, 1), (0, 0, 0, 0), (1, 1), 1, "relu")
    assert_close(host64(Y), oracle.conv2d(X, Wt, b, act="relu"), dtype, "1x1")


def misaligned(t, elems):
    """A copy of `t` whose data pointer sits `elems` elements past an aligned one."""
    flat = torch.empty(t.numel() + elems, dtype=t.dtype, device=t.device)
    v = flat[elems:].view(t.shape)
    v.copy_(t)
    return v


def test_pw_conv_sweep_bf16(ox, monkeypatch):
    # the pointwise kernel over ragged pixel counts (odd, even and multiple-of-4
    # planes, blocks spanning images), partial channel blocks and every chunk width
    monkeypatch.setenv("OX_FORCE_KERNEL", "pw")
    r = np.random.default_rng(909)
    for ci in range(40):
        N = int(r.integers(1, 5))
        Cin = int(r.choice([32, 64, 96, 128, 256, 384]))
        H, W = int(r.integers(1, 24)), int(r.integers(1, 24))
        M = int(r.integers(1, 300))
        act = str(r.choice(["none", "relu", "relu6", "gelu"]))
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, 1, 1)) / math.sqrt(Cin), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        say("pw sweep", ci, (N, Cin, H, W, M, act))
        Y = run_conv(ox, X, Wt, b, "bf16", (1, 1), (0, 0, 0, 0), (1, 1), 1, act)
        assert_close(host64(Y), oracle.conv2d(X, Wt, b, act=act), "bf16", "pw %d" % ci)


PWD_CFGS = ["128:64:64", "128:64:32", "64:64:64", "64:128:64", "64:128:32", "64:256:64", "64:256:32"]


@pytest.mark.parametrize("cfg", PWD_CFGS)
def test_pwd_each_config_integer_exact(ox, cfg, monkeypatch):
    # the DMA-staged pointwise kernel, each configuration pinned, on inputs
    # in {-1, 0, 1}: every sum is an integer of magnitude <= C <= 256, exact
    # in bf16, so a wrong swizzle, fragment row or pixel offset shows as a
    # mismatch.  Ragged pixel tails (N*H*W not a multiple of the tile),
    # partial channel blocks, tiles spanning images, every activation.
    monkeypatch.setenv("OX_FORCE_KERNEL", "pwd")
    monkeypatch.setenv("OX_PWD_CFG", cfg)
    kc = int(cfg.split(":")[2])
    r = np.random.default_rng(4100 + PWD_CFGS.index(cfg))
    # planes that are multiples of 8 pixels (16-byte pixel pieces) and even
    # planes that are not (4-byte pieces: 14x14, 6x7, 5x2, 3x6)
    cases = [(2, 128, 8, 8, 70), (3, 64, 4, 6, 150), (1, 256, 16, 16, 200), (5, 192, 2, 4, 33),
             (2, 96, 6, 12, 256), (1, 32, 8, 1, 300), (2, 128, 14, 14, 90), (3, 64, 6, 7, 130),
             (4, 192, 5, 2, 64), (2, 96, 3, 6, 200)]
    ran = 0
    for ci, (N, Cin, H, W, M) in enumerate(cases):
        if Cin % kc:
            continue
        act = ["none", "relu", "relu6", "gelu"][ci % 4]
        X = r.integers(-1, 2, (N, Cin, H, W)).astype(np.float64)
        Wt = r.integers(-1, 2, (M, Cin, 1, 1)).astype(np.float64)
        b = r.integers(-3, 4, M).astype(np.float64)
        say("pwd config", cfg, (N, Cin, H, W, M, act))
        Y = run_conv(ox, X, Wt, b, "bf16", (1, 1), (0, 0, 0, 0), (1, 1), 1, act)
        ref = oracle.conv2d(X, Wt, b, act=act)
        if act == "gelu":
            assert_close(host64(Y), ref, "bf16", "pwd %s case %d" % (cfg, ci))
        else:
            assert np.array_equal(host64(Y), ref), "pwd %s case %d" % (cfg, ci)
        ran += 1
    assert ran >= 5


@pytest.mark.parametrize("grid", ["1", "5", "37"])
def test_pwd_persistent_ranges(ox, grid, monkeypatch):
    # a small persistent grid: each block walks a pixel range of many tiles,
    # its ring running on from one tile into the next, and the ranges end
    # inside tiles; integer-valued inputs, compared exactly
    monkeypatch.setenv("OX_FORCE_KERNEL", "pwd")
    monkeypatch.setenv("OX_PWD_GRID", grid)
    r = np.random.default_rng(4150 + int(grid))
    for ci, (N, Cin, H, W, M) in enumerate([(3, 128, 12, 16, 64), (2, 64, 10, 24, 200),
                                            (4, 96, 8, 8, 130), (1, 256, 20, 8, 520)]):
        X = r.integers(-1, 2, (N, Cin, H, W)).astype(np.float64)
        Wt = r.integers(-1, 2, (M, Cin, 1, 1)).astype(np.float64)
        b = r.integers(-3, 4, M).astype(np.float64)
        say("pwd persistent", grid, (N, Cin, H, W, M))
        Y = run_conv(ox, X, Wt, b, "bf16", (1, 1), (0, 0, 0, 0), (1, 1), 1, "relu")
        assert np.array_equal(host64(Y), oracle.conv2d(X, Wt, b, act="relu")), \
            "pwd grid %s case %d" % (grid, ci)


def test_pwd_sweep_bf16(ox, monkeypatch):
    # default configuration choice over random shapes the DMA kernel takes
    # (H*W % 8 == 0, C % 32 == 0), random values
    monkeypatch.setenv("OX_FORCE_KERNEL", "pwd")
    r = np.random.default_rng(4200)
    for ci in range(30):
        N = int(r.integers(1, 5))
        Cin = int(r.choice([32, 64, 96, 128, 256, 384, 512]))
        H = int(r.integers(1, 20))
        W = 8 * int(r.integers(1, 4)) if ci % 2 else 2 * int(r.integers(1, 12))   # 16- or 4-byte pieces
        M = int(r.integers(1, 600))
        act = str(r.choice(["none", "relu", "relu6", "gelu"]))
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, 1, 1)) / math.sqrt(Cin), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        say("pwd sweep", ci, (N, Cin, H, W, M, act))
        Y = run_conv(ox, X, Wt, b, "bf16", (1, 1), (0, 0, 0, 0), (1, 1), 1, act)
        assert_close(host64(Y), oracle.conv2d(X, Wt, b, act=act), "bf16", "pwd sweep %d" % ci)


def test_pwd_not_taken_for_unaligned_or_odd_planes(ox, monkeypatch):
    # the DMA kernel needs 16-byte aligned tensors and H*W % 8 == 0: other
    # cases select another kernel (and a forced 'pwd' is refused), with the
    # same results
    r = np.random.default_rng(4300)
    X = synth.round_to(r.standard_normal((2, 64, 7, 7)), "bf16")
    Wt = synth.round_to(r.standard_normal((96, 64, 1, 1)) / 8.0, "bf16")
    b = synth.round_to(r.uniform(-0.5, 0.5, 96), "bf16")
    assert not ox.ox_conv2d_variant("bf16", 2, 64, 7, 7, 96, 1, 1).startswith("pwd/")
    assert ox.ox_conv2d_variant("bf16", 2, 64, 8, 8, 96, 1, 1).startswith("pwd/")
    monkeypatch.setenv("OX_FORCE_KERNEL", "pwd")
    with pytest.raises(ox.OxError):
        run_conv(ox, X, Wt, b, "bf16", (1, 1), (0, 0, 0, 0), (1, 1), 1, "relu")
    monkeypatch.delenv("OX_FORCE_KERNEL")
    X8 = synth.round_to(r.standard_normal((2, 64, 8, 8)), "bf16")
    ref = oracle.conv2d(X8, Wt, b, act="relu")
    # X one element off (no DMA piece fits: another kernel), two elements off
    # (4-byte pieces), Y off alignment (narrower stores), both 16-byte aligned
    for xoff, yoff in ((1, 0), (2, 0), (0, 4), (0, 1), (8, 8)):
        say("pwd alignment", xoff, yoff)
        Xd = misaligned(dev(X8, "bf16"), xoff)
        Y = misaligned(nan_like((2, 96, 8, 8), "bf16"), yoff)
        ox.ox_conv2d_fused(Xd, dev(Wt, "bf16"), dev(b, "bf16"), act="relu", Y=Y)
        torch.cuda.synchronize()
        assert_close(host64(Y), ref, "bf16", "pwd alignment %d %d" % (xoff, yoff))


@pytest.mark.parametrize("cfg", PWD_CFGS)
def test_pwd_residual_each_config(ox, cfg, monkeypatch):
    # Y = act(conv + b + R) on the DMA kernel: separate R, and R = Y in place
    monkeypatch.setenv("OX_FORCE_KERNEL", "pwd")
    monkeypatch.setenv("OX_PWD_CFG", cfg)
    kc = int(cfg.split(":")[2])
    r = np.random.default_rng(4400 + PWD_CFGS.index(cfg))
    N, Cin, H, W, M = 3, 64 if kc == 64 else 96, 6, 8, 140
    X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
    Wt = synth.round_to(r.standard_normal((M, Cin, 1, 1)) / math.sqrt(Cin), "bf16")
    b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
    Rr = synth.round_to(r.standard_normal((N, M, H, W)), "bf16")
    ref = oracle.conv2d(X, Wt, b, act="relu", residual=Rr)
    for in_place in (False, True):
        say("pwd residual", cfg, in_place)
        Y = run_conv_res(ox, X, Wt, b, Rr, "bf16", (1, 1), (0, 0, 0, 0), (1, 1), 1, "relu",
                         in_place=in_place)
        assert_close(host64(Y), ref, "bf16", "pwd residual %s %s" % (cfg, in_place))


@pytest.mark.parametrize("fp", ["1", "2"])
@pytest.mark.parametrize("plan", ["1:32", "1:64", "2:32", "2:64"])
def test_pw_each_config(ox, plan, fp, monkeypatch):
    # every block configuration (wave rows : channel chunk), pinned, with the
    # staging load width (1, 2, 4 pixels) and the store width (1 .. 8 pixels)
    # driven by the plane size and by X and Y pointers offset from alignment
    monkeypatch.setenv("OX_FORCE_KERNEL", "pw")
    monkeypatch.setenv("OX_PW_PLAN", plan)
    monkeypatch.setenv("OX_PW_FP", fp)      # 32-pixel fragments per wave
    r = np.random.default_rng(31 + int(plan[0]) * 1000 + int(plan[2:]))
    for ci, (N, Cin, H, W, M, xoff, yoff) in enumerate([
            (2, 128, 8, 8, 70, 0, 0), (3, 128, 6, 5, 150, 0, 0), (2, 256, 7, 7, 64, 0, 0),
            (2, 128, 4, 8, 96, 1, 1), (1, 256, 6, 6, 200, 2, 2), (5, 128, 3, 3, 33, 0, 3)]):
        HW = H * W
        P = 4 if HW % 4 == 0 and xoff % 4 == 0 else 2 if HW % 2 == 0 and xoff % 2 == 0 else 1
        if plan.endswith(":64") and P == 1 and fp == "2":
            continue      # those plans do not take single-pixel staging
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, 1, 1)) / math.sqrt(Cin), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        say("pw config", plan, (N, Cin, H, W, M, xoff, yoff))
        Xd = misaligned(dev(X, "bf16"), xoff)
        Y = misaligned(nan_like((N, M, H, W), "bf16"), yoff)
        ox.ox_conv2d_fused(Xd, dev(Wt, "bf16"), dev(b, "bf16"), (1, 1), (0, 0, 0, 0), (1, 1), 1,
                           "relu", Y=Y)
        torch.cuda.synchronize()
        assert_close(host64(Y), oracle.conv2d(X, Wt, b, act="relu"), "bf16",
                     "pw %s case %d" % (plan, ci))


@pytest.mark.parametrize("grid", ["1", "3", "8"])
def test_pw_persistent_blocks(ox, grid, monkeypatch):
    # a small persistent grid: every block runs many work units in a row, so
    # the loads of a unit's first chunks are issued while the previous unit
    # computes -- with odd and even chunk counts per unit, split-K slices and
    # partial tiles at the end of the pixel range
    monkeypatch.setenv("OX_FORCE_KERNEL", "pw")
    monkeypatch.setenv("OX_PW_GRID", grid)
    r = np.random.default_rng(700 + int(grid))
    for ci, (N, Cin, H, W, M, plan, splits) in enumerate([
            (3, 96, 9, 11, 200, "2:32", None), (2, 320, 8, 8, 70, "1:64", None),
            (4, 128, 6, 6, 260, "2:64", None), (2, 192, 7, 7, 130, "2:64", None),
            (2, 224, 5, 9, 96, "2:32", "3"), (3, 64, 12, 12, 300, "1:32", None)]):
        monkeypatch.setenv("OX_PW_PLAN", plan)
        if splits:
            monkeypatch.setenv("OX_PW_SPLITS", splits)
        else:
            monkeypatch.delenv("OX_PW_SPLITS", raising=False)
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, 1, 1)) / math.sqrt(Cin), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        say("pw persistent", grid, (N, Cin, H, W, M, plan, splits))
        Y = run_conv(ox, X, Wt, b, "bf16", (1, 1), (0, 0, 0, 0), (1, 1), 1, "relu",
                     ws=bool(splits))
        assert_close(host64(Y), oracle.conv2d(X, Wt, b, act="relu"), "bf16",
                     "pw persistent grid %s case %d" % (grid, ci))


@pytest.mark.parametrize("fp", ["1", "2"])
@pytest.mark.parametrize("splits", [2, 3, 5, 9])
def test_pw_split_k(ox, splits, fp, monkeypatch):
    # split-K: slices of the channel range write fp32 partials, a second
    # kernel adds them in slice order (its loads go out eight slices at a
    # time: 9 slices take two groups) -- same result as the oracle, and
    # bit-identical from run to run
    monkeypatch.setenv("OX_FORCE_KERNEL", "pw")
    monkeypatch.setenv("OX_PW_SPLITS", str(splits))
    monkeypatch.setenv("OX_PW_FP", fp)
    r = np.random.default_rng(600 + splits)
    for ci, (N, Cin, H, W, M) in enumerate([(2, 512, 7, 7, 200), (3, 320, 6, 6, 64), (1, 256, 9, 9, 130),
                                            (1, 1152, 5, 5, 72)]):
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, 1, 1)) / math.sqrt(Cin), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        say("pw split", splits, (N, Cin, H, W, M))
        assert ox.ox_conv2d_workspace_bytes("bf16", N, Cin, H, W, M, 1, 1) > 0
        Y1 = run_conv(ox, X, Wt, b, "bf16", (1, 1), (0, 0, 0, 0), (1, 1), 1, "relu6", ws=True)
        Y2 = run_conv(ox, X, Wt, b, "bf16", (1, 1), (0, 0, 0, 0), (1, 1), 1, "relu6", ws=True)
        assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
        assert_close(host64(Y1), oracle.conv2d(X, Wt, b, act="relu6"), "bf16",
                     "pw split %d case %d" % (splits, ci))


def test_smallc_conv_sweep_bf16(ox, monkeypatch):
    # the few-input-channel kernel (C <= 4): kernels up to 8 wide, both
    # strides, asymmetric pads, 16-byte and 2-byte input staging
    monkeypatch.setenv("OX_FORCE_KERNEL", "smallc")
    r = np.random.default_rng(4242)
    ran = 0
    for ci in range(40):
        N = int(r.integers(1, 4))
        Cin = int(r.integers(1, 5))
        kH, kW = int(r.integers(1, 9)), int(r.integers(1, 9))
        s = int(r.choice([1, 2]))
        H = int(r.integers(kH, 40))
        W = int(r.choice([r.integers(kW, 40), 8 * r.integers(1, 6)]))
        M = int(r.integers(1, 140))
        pads = tuple(int(v) for v in r.integers(0, 4, 4))
        if not conv_case_ok(N, Cin, H, W, M, kH, kW, (s, s), pads, (1, 1), 1):
            continue
        act = str(r.choice(["none", "relu", "relu6", "gelu"]))
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, kH, kW)) / math.sqrt(Cin * kH * kW), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        say("smallc sweep", ci, (N, Cin, H, W, M, kH, kW, s, pads, act))
        Y = run_conv(ox, X, Wt, b, "bf16", (s, s), pads, (1, 1), 1, act)
        assert_close(host64(Y), oracle.conv2d(X, Wt, b, (s, s), pads, (1, 1), 1, act), "bf16",
                     "smallc %d" % ci)
        ran += 1
    assert ran >= 25


def test_smallc_stem_misaligned_input(ox, monkeypatch):
    # an input pointer off 16-byte alignment takes the element-wise staging
    monkeypatch.setenv("OX_FORCE_KERNEL", "smallc")
    r = np.random.default_rng(77)
    X = synth.round_to(r.standard_normal((2, 3, 40, 48)), "bf16")
    Wt = synth.round_to(r.standard_normal((64, 3, 7, 7)) / math.sqrt(147), "bf16")
    b = synth.round_to(r.uniform(-0.5, 0.5, 64), "bf16")
    say("smallc misaligned")
    ref = oracle.conv2d(X, Wt, b, (2, 2), (3, 3, 3, 3), (1, 1), 1, "relu")
    for xoff, woff in ((1, 0), (0, 1), (3, 5)):
        Xd = misaligned(dev(X, "bf16"), xoff)
        Wd = misaligned(dev(Wt, "bf16"), woff)
        Y = nan_like((2, 64, 20, 24), "bf16")
        ox.ox_conv2d_fused(Xd, Wd, dev(b, "bf16"), (2, 2), (3, 3, 3, 3), (1, 1), 1, "relu", Y=Y)
        torch.cuda.synchronize()
        assert_close(host64(Y), ref, "bf16", "smallc misaligned %d %d" % (xoff, woff))


def conv_layer_tensors(layer, cfg, li, dtype):
    t = synth.conv_inputs(layer, cfg, li)
    Wf, bf = oracle.fold_batchnorm(t["W"], t["gamma"], t["beta"], t["mean"], t["var"], 1e-5)
    return (synth.round_to(t["X"], dtype), synth.round_to(Wf, dtype), synth.round_to(bf, dtype))


def check_layer(ox, layer, cfg, li, dtype, ws=False):
    # every output of the layer against the oracle
    X, Wt, b = conv_layer_tensors(layer, cfg, li, dtype)
    s = (layer.stride, layer.stride)
    Y = run_conv(ox, X, Wt, b, dtype, s, layer.onnx_pads, (1, 1), layer.group, layer.act, ws=ws)
    assert not torch.isnan(Y).any().item(), layer.name
    got = host64(Y)
    del Y
    ref = oracle.conv2d(X, Wt, b, s, layer.onnx_pads, (1, 1), layer.group, layer.act)
    assert_close(got, ref, dtype, layer.name)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 64])
def test_c2_mobilenetv2_layers(ox, dtype, N):
    for li, layer in enumerate(synth.unique_layers(synth.mobilenetv2_layers(N))):
        say("C2", N, dtype, layer.name, layer.key())
        check_layer(ox, layer, 2, li, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 32])
def test_c3_resnet50_layers(ox, dtype, N):
    # with a workspace, as the benchmark runs them (split-K where planned)
    for li, layer in enumerate(synth.resnet50_layers(N)):
        say("C3", N, dtype, layer.name, layer.key())
        check_layer(ox, layer, 3, li, dtype, ws=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gpu_fold_then_conv_equals_unfused_chain(ox, dtype):
    # tensorforge "ResNet fusion": the library's own offline fold feeding its
    # fused conv must match the oracle's Conv -> BatchNorm -> activation.
    layer = synth.ConvLayer("e2e", 2, 32, 14, 14, 48, 3, 2, 1, 1, "relu6")
    t = synth.conv_inputs(layer, 3, 99)
    X = synth.round_to(t["X"], dtype)
    W32 = t["W"].astype(np.float32)
    prm = [t[k].astype(np.float32) for k in ("gamma", "beta", "mean", "var")]
    Wf, bf = ox.ox_fold_batchnorm(W32, *prm, eps=1e-5)
    Y = nan_like((2, 48, 7, 7), dtype)
    ox.ox_conv2d_fused(dev(X, dtype), torch.from_numpy(Wf).cuda().to(TD[dtype]),
                       torch.from_numpy(bf).cuda().to(TD[dtype]), (2, 2), (1, 1, 1, 1), act="relu6", Y=Y)
    torch.cuda.synchronize()
    chain = oracle.conv2d(X, W32.astype(np.float64), None, (2, 2), (1, 1, 1, 1))
    chain = oracle.batchnorm(chain, *[p.astype(np.float64) for p in prm], eps=float(np.float32(1e-5)))
    chain = oracle.act("relu6", chain)
    assert_close(host64(Y), chain, dtype, "fold+conv")


def test_repeat_runs_are_bitwise_identical(ox):
    layer = synth.resnet50_layers(2)[5]   # stage-2 3x3
    X, Wt, b = conv_layer_tensors(layer, 3, 5, "bf16")
    outs = [host64(run_conv(ox, X, Wt, b, "bf16", (1, 1), (1, 1, 1, 1), (1, 1), 1, "relu"))
            for _ in range(3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


# -------------------------------------------------------------------- int8 --

def int8_gpu(ox, layer, t, y_type):
    blk = torch.from_numpy(ox.ox_int8_prepare(t["wq"], t["w_s"], t["x_s"], t["x_zp"], t["y_s"],
                                              t["y_zp"], t["bias_q"])).cuda()
    xq = torch.from_numpy(t["xq"]).cuda()
    wq = torch.from_numpy(t["wq"]).cuda()
    if layer.kind == "gemm":
        Y = ox.ox_gemm_fused(xq, wq, transB=True, int8_params=blk,
                             out_dtype=torch.int32 if y_type == "i32" else torch.int8)
    else:
        c = layer.conv
        Y = ox.ox_conv2d_int8(xq, wq, blk, y_type, (c.stride, c.stride), c.onnx_pads, (1, 1), c.group)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def int8_ref(layer, t):
    if layer.kind == "gemm":
        return oracle.gemm_int8(t["xq"], t["wq"], t["bias_q"], t["x_zp"], t["x_s"], t["w_s"],
                                t["y_s"], t["y_zp"])
    c = layer.conv
    return oracle.conv2d_int8(t["xq"], t["wq"], t["bias_q"], t["x_zp"], t["x_s"], t["w_s"], t["y_s"],
                              t["y_zp"], (c.stride, c.stride), c.onnx_pads, (1, 1), c.group)


def test_c4_int8_conformer_block_bit_exact(ox):
    for li, layer in enumerate(synth.conformer_int8_layers()):
        say("C4", layer.name)
        t = synth.int8_inputs(layer, 4, li)
        acc, y = int8_ref(layer, t)
        assert np.array_equal(int8_gpu(ox, layer, t, "i32").astype(np.int64), acc), layer.name
        assert np.array_equal(int8_gpu(ox, layer, t, "i8"), y), layer.name


@pytest.mark.parametrize("geom", [
    (2, 6, 9, 11, 10, 3, 3, 1, (1, 1, 1, 1), 1),
    (1, 12, 7, 8, 12, 3, 3, 2, (2, 1, 0, 3), 12),
    (1, 8, 5, 33, 8, 1, 9, 1, (0, 4, 0, 4), 8),
    (2, 32, 6, 6, 48, 1, 1, 1, (0, 0, 0, 0), 1),
    (1, 8, 10, 10, 16, 5, 5, 2, (3, 3, 3, 3), 4),
])
def test_int8_conv_small_shapes_bit_exact(ox, geom):
    N, Cin, H, W, M, kH, kW, s, pads, g = geom
    say("int8 conv", geom)
    conv = synth.ConvLayer("q", N, Cin, H, W, M, kH, s, 0, g, "none", kW=kW, pads=pads)
    layer = synth.Int8Layer("q", "conv", 1, (Cin // g) * kH * kW, M, conv)
    t = synth.int8_inputs(layer, 4, 50 + H + W)
    acc, y = int8_ref(layer, t)
    assert np.array_equal(int8_gpu(ox, layer, t, "i32").astype(np.int64), acc)
    assert np.array_equal(int8_gpu(ox, layer, t, "i8"), y)


def test_int8_gemm_ragged_bit_exact(ox):
    layer = synth.Int8Layer("g", "gemm", 77, 200, 45)
    say("int8 gemm ragged")
    t = synth.int8_inputs(layer, 4, 60)
    acc, y = int8_ref(layer, t)
    assert np.array_equal(int8_gpu(ox, layer, t, "i32").astype(np.int64), acc)
    assert np.array_equal(int8_gpu(ox, layer, t, "i8"), y)


def test_int8_requant_ties_on_gpu(ox):
    # x_s = 2^-4, w_s = 2^-3, y_s = 2^-6: multiplier 1/2, every odd accumulator
    # a tie; round half to even gives 0, 2, 0, -2 for 1, 3, -1, -3.
    say("int8 ties")
    K = 4
    accs = np.array([1, 3, -1, -3, 5, -5, 254, -258], np.int64)
    xq = np.zeros((1, K), np.int8)
    wq = np.zeros((len(accs), K), np.int8)
    blk = torch.from_numpy(ox.ox_int8_prepare(wq, np.full(len(accs), 2.0 ** -3, np.float32),
                                              2.0 ** -4, 0, 2.0 ** -6, 0, accs.astype(np.int32))).cuda()
    Y = ox.ox_gemm_fused(torch.from_numpy(xq).cuda(), torch.from_numpy(wq).cuda(), transB=True,
                         int8_params=blk, out_dtype=torch.int8)
    torch.cuda.synchronize()
    assert Y.cpu().numpy().ravel().tolist() == [0, 2, 0, -2, 2, -2, 127, -128]


# ---------------------- uint8 activations / outputs, weight zero points --

# (x uint8, y uint8, per-channel weight zero points)
QVARIANTS = [(False, False, False), (True, False, False), (False, False, True),
             (False, True, False), (True, True, True)]


def q_inputs(r, xu, wz, xshape, wshape):
    x = r.integers(0, 256, xshape) if xu else r.integers(-128, 128, xshape)
    w = r.integers(-128, 128, wshape).astype(np.int8)
    M = wshape[0]
    wzp = r.integers(-128, 128, M).astype(np.int32) if wz else None
    xzp = int(r.integers(0, 256)) if xu else int(r.integers(-128, 128))
    bq = r.integers(-20000, 20000, M).astype(np.int32)
    w_s = r.uniform(1e-3, 1e-2, M).astype(np.float32)
    return x, w, wzp, xzp, bq, np.float32(0.05), w_s


def q_out_scale(acc, x_s, w_s):
    # an output scale that spreads the requantised values over the 8-bit range
    spread = float(np.std(acc)) if acc.size > 1 else float(abs(acc).max() + 1)
    return np.float32(x_s * float(np.median(w_s)) * max(spread, 1.0) / 40.0)


def q_run(ox, blk, x, xu, w, yu, call):
    xd = torch.from_numpy(x.astype(np.uint8 if xu else np.int8)).cuda()
    wd = torch.from_numpy(w).cuda()
    bd = torch.from_numpy(blk).cuda()
    y32 = call(xd, wd, bd, "i32")
    y8 = call(xd, wd, bd, "u8" if yu else "i8")
    torch.cuda.synchronize()
    return y32.cpu().numpy().astype(np.int64), y8.cpu().numpy().astype(np.int32)


@pytest.mark.parametrize("xu,yu,wz", QVARIANTS)
def test_qgemm_variants_bit_exact(ox, xu, yu, wz):
    # QLinearMatMul / MatMulInteger with uint8 activations or outputs and
    # per-channel weight zero points, over ragged tiles and one row
    r = np.random.default_rng(700 + 4 * xu + 2 * yu + wz)
    for (M, K, N) in [(77, 200, 45), (130, 72, 33), (1, 64, 16), (64, 1000, 96), (40, 2500, 70)]:
        say("qgemm", (xu, yu, wz), (M, K, N))
        x, w, wzp, xzp, bq, x_s, w_s = q_inputs(r, xu, wz, (M, K), (N, K))
        acc0, _ = oracle.qgemm(x, w, bq, xzp, wzp, x_s, w_s, 1.0, 0)
        y_s = q_out_scale(acc0, x_s, w_s)
        yzp = int(r.integers(0, 256)) if yu else int(r.integers(-128, 128))
        acc, y = oracle.qgemm(x, w, bq, xzp, wzp, x_s, w_s, y_s, yzp, yu)
        blk = ox.ox_int8_prepare(w, w_s, x_s, xzp, y_s, yzp, bq, w_zp=wzp, x_unsigned=xu, y_unsigned=yu)

        def call(xd, wd, bd, yt):
            od = {"i32": torch.int32, "u8": torch.uint8, "i8": torch.int8}[yt]
            return ox.ox_gemm_fused(xd, wd, transB=True, int8_params=bd, out_dtype=od)
        g32, g8 = q_run(ox, blk, x, xu, w, yu, call)
        assert np.array_equal(g32, acc), (M, K, N)
        assert np.array_equal(g8, y), (M, K, N)
        assert len(np.unique(y)) > 8          # the outputs are spread, not saturated


@pytest.mark.parametrize("xu,yu,wz", QVARIANTS)
def test_qconv_variants_bit_exact(ox, xu, yu, wz):
    # QLinearConv / ConvInteger variants on every int8 conv kernel: the
    # implicit GEMM (padding at x_zp, strides, dilation, groups), the 1x1
    # kernel, and the depthwise kernel (2-D and the conformer's 1-D shape)
    r = np.random.default_rng(800 + 4 * xu + 2 * yu + wz)
    for (N, Cin, H, W, M, kH, kW, s, pads, d, g) in [
            (2, 16, 9, 11, 24, 3, 3, 1, (1, 1, 1, 1), 1, 1),
            (1, 12, 13, 10, 20, 3, 3, 2, (2, 1, 0, 1), 1, 2),
            (2, 8, 12, 12, 8, 3, 3, 1, (2, 2, 2, 2), 2, 1),
            (2, 64, 14, 14, 96, 3, 3, 1, (1, 1, 1, 1), 1, 1),
            (2, 48, 7, 9, 40, 1, 1, 1, (0, 0, 0, 0), 1, 1),
            (2, 24, 10, 13, 24, 3, 3, 1, (1, 1, 1, 1), 1, 24),
            (1, 16, 1, 50, 16, 1, 9, 1, (0, 4, 0, 4), 1, 16),
            (1, 128, 9, 9, 64, 3, 3, 1, (1, 1, 1, 1), 1, 1),      # long K: four K units per stage
            (1, 1024, 1, 50, 72, 1, 1, 1, (0, 0, 0, 0), 1, 1)]:
        geom = (N, Cin, H, W, M, kH, kW, s, pads, d, g)
        say("qconv", (xu, yu, wz), geom,
            ox.ox_conv2d_variant("i8", N, Cin, H, W, M, kH, kW, (s, s), pads, (d, d), g))
        x, w, wzp, xzp, bq, x_s, w_s = q_inputs(r, xu, wz, (N, Cin, H, W), (M, Cin // g, kH, kW))
        args = ((s, s), pads, (d, d), g)
        acc0, _ = oracle.qconv2d(x, w, bq, xzp, wzp, x_s, w_s, 1.0, 0, False, *args)
        y_s = q_out_scale(acc0, x_s, w_s)
        yzp = int(r.integers(0, 256)) if yu else int(r.integers(-128, 128))
        acc, y = oracle.qconv2d(x, w, bq, xzp, wzp, x_s, w_s, y_s, yzp, yu, *args)
        blk = ox.ox_int8_prepare(w, w_s, x_s, xzp, y_s, yzp, bq, w_zp=wzp, x_unsigned=xu, y_unsigned=yu)

        def call(xd, wd, bd, yt):
            return ox.ox_conv2d_int8(xd, wd, bd, yt, *args)
        g32, g8 = q_run(ox, blk, x, xu, w, yu, call)
        assert np.array_equal(g32, acc), geom
        assert np.array_equal(g8, y), geom


@pytest.mark.parametrize("xu,yu,wz", QVARIANTS)
def test_qconv_1x1_buffer_path_bit_exact(ox, xu, yu, wz, monkeypatch):
    # int8 1x1 convolutions on planes of whole 4-byte groups take the buffer
    # loaders (sixteen 4-column words per task, transposed into k-chunks in
    # LDS) with the Gemm's stage shapes: every tile, ragged channels and
    # pixel ranges, tiles straddling images, K tails, against the oracle and
    # against the gathering loader (OX_CONV_PIPE=0)
    r = np.random.default_rng(870 + 4 * xu + 2 * yu + wz)
    for tile in GEMM_TILES:
        for (N, Cin, H, W, M) in [(3, 48, 4, 7, 40), (1, 1024, 1, 1000, 72), (2, 64, 8, 8, 96),
                                  (2, 272, 2, 6, 130)]:
            geom = (N, Cin, H, W, M, 1, 1, 1, (0, 0, 0, 0), 1, 1)
            say("qconv 1x1 buffer", tile, (xu, yu, wz), geom)
            x, w, wzp, xzp, bq, x_s, w_s = q_inputs(r, xu, wz, (N, Cin, H, W), (M, Cin, 1, 1))
            args = ((1, 1), (0, 0, 0, 0), (1, 1), 1)
            acc0, _ = oracle.qconv2d(x, w, bq, xzp, wzp, x_s, w_s, 1.0, 0, False, *args)
            y_s = q_out_scale(acc0, x_s, w_s)
            yzp = int(r.integers(0, 256)) if yu else int(r.integers(-128, 128))
            acc, y = oracle.qconv2d(x, w, bq, xzp, wzp, x_s, w_s, y_s, yzp, yu, *args)
            blk = ox.ox_int8_prepare(w, w_s, x_s, xzp, y_s, yzp, bq, w_zp=wzp, x_unsigned=xu, y_unsigned=yu)

            def call(xd, wd, bd, yt):
                return ox.ox_conv2d_int8(xd, wd, bd, yt, *args)
            monkeypatch.setenv("OX_FORCE_KERNEL", "1x1,tile=" + tile)
            for pipe in ("1", "0"):
                monkeypatch.setenv("OX_CONV_PIPE", pipe)
                g32, g8 = q_run(ox, blk, x, xu, w, yu, call)
                assert np.array_equal(g32, acc), (tile, pipe, geom)
                assert np.array_equal(g8, y), (tile, pipe, geom)
            monkeypatch.delenv("OX_CONV_PIPE")
            monkeypatch.delenv("OX_FORCE_KERNEL")


# ----------------------------------------------------------- MatMulNBits --

def nbits_run(ox, t, a_offset=0):
    M, K = t["A"].shape
    buf = torch.zeros(M * K + a_offset, dtype=torch.bfloat16, device="cuda")
    Ad = buf[a_offset:].view(M, K)
    Ad.copy_(dev(t["A"], "bf16"))
    B = torch.from_numpy(t["B"]).cuda()
    sc = torch.from_numpy(t["scales"]).cuda()
    zp = None if t["zero_points"] is None else torch.from_numpy(t["zero_points"]).cuda()
    bias = None if t["bias"] is None else dev(t["bias"], "bf16")
    Y = nan_like((M, B.shape[0]), "bf16")
    ox.ox_matmul_nbits(Ad, B, sc, K, zp, bias, Y)
    torch.cuda.synchronize()
    return host64(Y)


@pytest.mark.parametrize("shape", [(1, 64, 64), (5, 45, 200), (33, 77, 512), (130, 96, 96),
                                   (64, 256, 4096), (1, 4096, 4096)])
@pytest.mark.parametrize("zp", [True, False])
def test_matmul_nbits_parity(ox, shape, zp):
    # decode (one row) and prefill rows, ragged N and K (a partial last
    # block), with and without zero points and bias; scales that are powers
    # of two keep every dequantised weight exact in bf16
    M, N, K = shape
    say("nbits", shape, zp)
    t = synth.nbits_inputs(M, N, K, 300 + M + N + K, with_zp=zp, with_bias=(M % 2 == 1))
    got = nbits_run(ox, t)
    ref = oracle.matmul_nbits(t["A"], t["B"], t["scales"], K, t["zero_points"], t["bias"])
    assert_close(got, ref, "bf16", "nbits %s" % (shape,))


def test_matmul_nbits_general_scales_and_unaligned_rows(ox):
    # arbitrary fp32 scales (each dequantised weight rounded to bf16 once)
    # and A one element off 16-byte alignment (the element-wise A loads)
    for (M, N, K, off) in [(7, 100, 320, 0), (3, 64, 96, 1), (40, 33, 72, 1)]:
        say("nbits general", (M, N, K, off))
        t = synth.nbits_inputs(M, N, K, 500 + K, pow2_scales=False)
        got = nbits_run(ox, t, off)
        ref = oracle.matmul_nbits(t["A"], t["B"], t["scales"], K, t["zero_points"], t["bias"])
        assert_close(got, ref, "bf16", "nbits general")


# ------------------------------------------------- DynamicQuantizeLinear --

def dq_check(ox, x, offset=0):
    n = x.size
    buf = torch.zeros(n + offset, dtype=torch.float32, device="cuda")
    Xd = buf[offset:]
    Xd.copy_(torch.from_numpy(np.ascontiguousarray(x.ravel())))
    Y = torch.full((n,), 77, dtype=torch.uint8, device="cuda")
    Yg, sc, zp = ox.ox_dynamic_quantize_linear(Xd, Y=Y)
    torch.cuda.synchronize()
    y_ref, sc_ref, zp_ref = oracle.dynamic_quantize_linear(x.ravel())
    assert sc.cpu().numpy()[0] == sc_ref and int(zp.cpu()[0]) == zp_ref
    assert np.array_equal(Yg.cpu().numpy(), y_ref)
    return y_ref, sc_ref, zp_ref


@pytest.mark.parametrize("n", [0, 1, 3, 17, 4096, 70001])
@pytest.mark.parametrize("offset", [0, 1])
def test_dynamic_quantize_bit_exact(ox, n, offset):
    # the vector path (aligned) and the element path (X one element off), a
    # ragged tail, several blocks; fp32 scale, zero point and bytes exact
    r = np.random.default_rng(n + 13 * offset)
    x = (r.standard_normal(n) * 2.5 + 0.3).astype(np.float32)
    say("dynq", n, offset)
    dq_check(ox, x, offset)


def test_dynamic_quantize_special_ranges(ox):
    say("dynq special")
    for x in [np.zeros(100, np.float32), np.linspace(0.5, 9.0, 333).astype(np.float32),
              -np.linspace(0.1, 4.0, 260).astype(np.float32), np.arange(256, dtype=np.float32),
              np.array([-1.0, 0.0, 1.0], np.float32), (np.ones(64) * 1e30).astype(np.float32)]:
        dq_check(ox, x)


def test_dynamic_quantize_then_matmul_integer(ox):
    # a dynamically quantised MatMulInteger: the conformer FFN's hidden
    # activation [1000, 4096] fp32 quantised on the device, then the int8
    # Gemm with int32 outputs against the oracle's acc on the oracle's bytes
    r = np.random.default_rng(77)
    x = (r.standard_normal((1000, 4096)) * 1.7).astype(np.float32)
    say("dynq + matmul integer")
    y_ref, sc, zp = dq_check(ox, x)
    w = r.integers(-128, 128, (256, 4096)).astype(np.int8)
    wz = r.integers(-5, 6, 256).astype(np.int32)
    w_s = np.full(256, 0.01, np.float32)
    blk = torch.from_numpy(ox.ox_int8_prepare(w, w_s, sc, zp, 1.0, 0, w_zp=wz, x_unsigned=True)).cuda()
    Xd = torch.from_numpy(x).cuda()
    Yq, _, _ = ox.ox_dynamic_quantize_linear(Xd)
    acc = ox.ox_gemm_fused(Yq.view(1000, 4096), torch.from_numpy(w).cuda(), transB=True,
                           int8_params=blk, out_dtype=torch.int32)
    torch.cuda.synchronize()
    rows = np.arange(0, 1000, 37)
    ref, _ = oracle.qgemm(y_ref.reshape(1000, 4096)[rows], w, None, zp, wz, sc, w_s, 1.0, 0)
    assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), ref)


def test_patch_conv_sweep_bf16(ox, monkeypatch):
    # the LDS-patch 3x3 kernel over strides, dilations, asymmetric pads,
    # ragged channel / pixel counts and several images per block
    monkeypatch.setenv("OX_FORCE_KERNEL", "patch")
    r = np.random.default_rng(321)
    ran = 0
    for ci in range(60):
        N = int(r.integers(1, 5))
        Cin = int(r.choice([32, 64, 96]))
        H, W = int(r.integers(1, 30)), int(r.integers(1, 30))
        M = int(r.integers(1, 150))
        s = int(r.choice([1, 2, 3]))
        d = int(r.choice([1, 2]))
        pads = tuple(int(v) for v in r.integers(0, 4, 4))
        if not conv_case_ok(N, Cin, H, W, M, 3, 3, (s, s), pads, (d, d), 1):
            continue
        try:
            ox.ox_conv2d_variant("bf16", N, Cin, H, W, M, 3, 3, (s, s), pads, (d, d), 1)
        except ox.OxError:
            continue      # no patch plan for this geometry
        act = str(r.choice(["none", "relu", "relu6", "gelu"]))
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, 3, 3)) / math.sqrt(9 * Cin), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        say("patch sweep", ci, (N, Cin, H, W, M, s, pads, d, act))
        Y = run_conv(ox, X, Wt, b, "bf16", (s, s), pads, (d, d), 1, act)
        assert_close(host64(Y), oracle.conv2d(X, Wt, b, (s, s), pads, (d, d), 1, act), "bf16",
                     "patch %d" % ci)
        ran += 1
    assert ran >= 30


def bf16_bits(a64):
    return synth.f32_to_bf16_bits(a64.astype(np.float32))


def run_conv_packed(ox, X, Wt, b, s, pads, d, act, ws=False):
    N, Cin, H, W = X.shape
    M = Wt.shape[0]
    Wp = ox.ox_conv2d_pack_weights(bf16_bits(Wt), "bf16", N, Cin, H, W, s, pads, d)
    Wp_dev = torch.from_numpy(Wp.view(np.int16)).cuda().view(torch.bfloat16)
    ho, wo = ox.conv_out_hw(H, W, 3, 3, s, pads, d)
    Y = nan_like((N, M, ho, wo), "bf16")
    wsb = workspace_for(ox, "bf16", N, Cin, H, W, M, 3, 3, s, pads, d, 1) if ws else None
    ox.ox_conv2d_fused_packed(dev(X, "bf16"), Wp_dev, dev(b, "bf16"), s, pads, d, act=act, Y=Y, M=M,
                              workspace=wsb)
    torch.cuda.synchronize()
    return Y


def test_packed_patch_conv_sweep_bf16(ox):
    r = np.random.default_rng(654)
    ran = 0
    for ci in range(50):
        N = int(r.integers(1, 5))
        Cin = int(r.choice([32, 64, 96]))
        H, W = int(r.integers(1, 30)), int(r.integers(1, 30))
        M = int(r.integers(1, 150))
        s = int(r.choice([1, 2]))
        d = int(r.choice([1, 2]))
        pads = tuple(int(v) for v in r.integers(0, 4, 4))
        if not conv_case_ok(N, Cin, H, W, M, 3, 3, (s, s), pads, (d, d), 1):
            continue
        act = str(r.choice(["none", "relu", "relu6", "gelu"]))
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, 3, 3)) / math.sqrt(9 * Cin), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        say("packed sweep", ci, (N, Cin, H, W, M, s, pads, d, act))
        Y = run_conv_packed(ox, X, Wt, b, (s, s), pads, (d, d), act)
        assert_close(host64(Y), oracle.conv2d(X, Wt, b, (s, s), pads, (d, d), 1, act), "bf16",
                     "packed %d" % ci)
        ran += 1
    assert ran >= 30


@pytest.mark.parametrize("cfg", ["1:2", "1:1", "2:2", "2:1"])
def test_patch_each_config(ox, cfg, monkeypatch):
    # every block configuration of the 3x3 kernel (wave grid : pixel tiles
    # per wave), pinned, over both strides, both staging widths (even and odd
    # plane sizes), ONNX-layout and packed weights, and partial channel blocks
    r = np.random.default_rng(77 + int(cfg[0]) * 10 + int(cfg[2]))
    monkeypatch.setenv("OX_FORCE_KERNEL", "patch")
    ran = 0
    for ci, (N, Cin, H, W, M, s, pads) in enumerate([
            (2, 64, 14, 14, 64, 1, (1, 1, 1, 1)), (3, 32, 9, 7, 96, 1, (1, 1, 1, 1)),
            (2, 96, 16, 12, 130, 2, (1, 1, 1, 1)), (1, 32, 13, 11, 40, 2, (0, 1, 2, 1))]):
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, 3, 3)) / math.sqrt(9 * Cin), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        ho, wo = ox.conv_out_hw(H, W, 3, 3, (s, s), pads, (1, 1))
        ref = oracle.conv2d(X, Wt, b, (s, s), pads, (1, 1), 1, "relu")
        for tr in range(ho, 0, -1):
            monkeypatch.setenv("OX_PATCH_PLAN", "%s:%d:1" % (cfg, tr))
            try:
                ox.ox_conv2d_variant("bf16", N, Cin, H, W, M, 3, 3, (s, s), pads, (1, 1), 1)
            except ox.OxError:
                continue
            say("patch config", cfg, "TR", tr, (N, Cin, H, W, M, s, pads))
            Y = run_conv(ox, X, Wt, b, "bf16", (s, s), pads, (1, 1), 1, "relu")
            assert_close(host64(Y), ref, "bf16", "config %s case %d" % (cfg, ci))
            Y = run_conv_packed(ox, X, Wt, b, (s, s), pads, (1, 1), "relu")
            assert_close(host64(Y), ref, "bf16", "packed config %s case %d" % (cfg, ci))
            ran += 1
            break
    assert ran == 4


@pytest.mark.parametrize("cfg", ["1:2", "1:1", "2:2", "2:1"])
def test_patch_split_k(ox, cfg, monkeypatch):
    # split-K on the 3x3 kernel: fp32 partials of channel slices, added in
    # slice order by a second kernel per wave sub-tile; parity with the
    # oracle and bit-identical repeats
    monkeypatch.setenv("OX_FORCE_KERNEL", "patch")
    r = np.random.default_rng(5150 + int(cfg[0]) * 10 + int(cfg[2]))
    ran = 0
    for ci, (N, Cin, H, W, M, s, splits) in enumerate([
            (3, 128, 7, 7, 96, 1, 2), (2, 160, 10, 9, 70, 2, 3), (4, 96, 5, 6, 130, 1, 3),
            (1, 288, 6, 6, 40, 1, 9)]):
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, 3, 3)) / math.sqrt(9 * Cin), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        pads = (1, 1, 1, 1)
        ho, wo = ox.conv_out_hw(H, W, 3, 3, (s, s), pads, (1, 1))
        ref = oracle.conv2d(X, Wt, b, (s, s), pads, (1, 1), 1, "relu")
        for tr, imb in [(ho, 2), (ho, 1), (max(1, ho // 2), 1)]:
            monkeypatch.setenv("OX_PATCH_PLAN", "%s:%d:%d:%d" % (cfg, tr, imb, splits))
            try:
                ox.ox_conv2d_variant("bf16", N, Cin, H, W, M, 3, 3, (s, s), pads, (1, 1), 1)
            except ox.OxError:
                continue
            say("patch split", cfg, "TR", tr, "IMB", imb, "S", splits, (N, Cin, H, W, M, s))
            assert ox.ox_conv2d_workspace_bytes("bf16", N, Cin, H, W, M, 3, 3, (s, s), pads) > 0
            Y1 = run_conv(ox, X, Wt, b, "bf16", (s, s), pads, (1, 1), 1, "relu", ws=True)
            Y2 = run_conv_packed(ox, X, Wt, b, (s, s), pads, (1, 1), "relu", ws=True)
            assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
            assert_close(host64(Y1), ref, "bf16", "split %s case %d tr %d" % (cfg, ci, tr))
            ran += 1
    assert ran >= 3


@pytest.mark.parametrize("xcd", ["8:1", "4:2", "2:4", "1:8"])
def test_patch_xcd_orders(ox, xcd, monkeypatch):
    # every split of the tile grid into XCD rectangles covers each output once
    monkeypatch.setenv("OX_PATCH_XCD", xcd)
    r = np.random.default_rng(8080 + int(xcd[0]))
    N, Cin, H, W, M = 16, 64, 8, 8, 512
    X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
    Wt = synth.round_to(r.standard_normal((M, Cin, 3, 3)) / math.sqrt(9 * Cin), "bf16")
    b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
    say("patch xcd", xcd)
    Y = run_conv_packed(ox, X, Wt, b, (1, 1), (1, 1, 1, 1), (1, 1), "relu")
    assert_close(host64(Y), oracle.conv2d(X, Wt, b, (1, 1), (1, 1, 1, 1), (1, 1), 1, "relu"), "bf16",
                 "xcd %s" % xcd)


@pytest.mark.parametrize("N", [1, 32])
def test_c3_resnet50_3x3_packed(ox, N):
    for li, layer in enumerate(synth.resnet50_layers(N)):
        if layer.k != 3:
            continue
        say("C3 packed", N, layer.name)
        X, Wt, b = conv_layer_tensors(layer, 3, li, "bf16")
        s = (layer.stride, layer.stride)
        Y = run_conv_packed(ox, X, Wt, b, s, layer.onnx_pads, (1, 1), layer.act, ws=True)
        assert not torch.isnan(Y).any().item()
        got = host64(Y)
        del Y
        ref = oracle.conv2d(X, Wt, b, s, layer.onnx_pads, (1, 1), 1, layer.act)
        assert_close(got, ref, "bf16", layer.name)


# ------------------------------------------------------------- residual --

def run_conv_res(ox, X, Wt, b, Rr, dtype, s, pads, d, g, act, ws=False, in_place=False, roff=0):
    """ox_conv2d_fused_res on device copies; Rr is the residual (float64 of
    values exact in dtype).  in_place: Y is the residual tensor itself;
    roff: R (and Y) sit roff elements past an aligned pointer."""
    Rd = misaligned(dev(Rr, dtype), roff) if roff else dev(Rr, dtype)
    Y = Rd if in_place else misaligned(nan_like(Rr.shape, dtype), roff)
    wsb = workspace_for(ox, dtype, *X.shape, Wt.shape[0], Wt.shape[2], Wt.shape[3], s, pads, d, g) if ws else None
    ox.ox_conv2d_fused_res(dev(X, dtype), dev(Wt, dtype), Rd, None if b is None else dev(b, dtype),
                           s, pads, d, g, act, Y=Y, workspace=wsb)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("grid", [None, "3"])
def test_residual_pointwise(ox, grid, monkeypatch):
    # the pointwise kernel's residual epilogue (fp32 staging, R read in runs
    # of V pixels): every activation, ragged tiles, split-K (the residual is
    # added in the second pass), a persistent grid, R one element off
    # alignment (V = 1), and R = Y in place (the kernel is asked for: on odd
    # planes with few channels the selection takes the tile engine)
    monkeypatch.setenv("OX_FORCE_KERNEL", "pw")
    if grid:
        monkeypatch.setenv("OX_PW_GRID", grid)
    r = np.random.default_rng(4040 + (3 if grid else 0))
    cases = [(2, 64, 8, 8, 96, "relu", False, 0, False), (3, 128, 7, 7, 130, "relu6", False, 0, False),
             (1, 256, 6, 10, 64, "gelu", True, 0, False), (2, 96, 9, 9, 70, "none", False, 1, False),
             (2, 128, 8, 8, 128, "relu", False, 0, True), (1, 512, 7, 7, 200, "relu", True, 0, True)]
    for ci, (N, Cin, H, W, M, act, ws, roff, in_place) in enumerate(cases):
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), "bf16")
        Wt = synth.round_to(r.standard_normal((M, Cin, 1, 1)) / math.sqrt(Cin), "bf16")
        b = synth.round_to(r.uniform(-0.5, 0.5, M), "bf16")
        Rr = synth.round_to(r.standard_normal((N, M, H, W)), "bf16")
        assert ox.ox_conv2d_variant("bf16", N, Cin, H, W, M, 1, 1).startswith("pw")
        say("residual pw", grid, (N, Cin, H, W, M, act, ws, roff, in_place))
        Y = run_conv_res(ox, X, Wt, b, Rr, "bf16", (1, 1), (0, 0, 0, 0), (1, 1), 1, act, ws=ws,
                         in_place=in_place, roff=roff)
        assert_close(host64(Y), oracle.conv2d(X, Wt, b, act=act, residual=Rr), "bf16",
                     "residual pw case %d" % ci)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_residual_tile_engine(ox, dtype):
    # every other geometry takes the tile engine's epilogue: 3x3, strided,
    # dilated, grouped, depthwise, a C that is not a multiple of 32, fp32 1x1
    r = np.random.default_rng(5151)
    cases = [(2, 32, 9, 11, 40, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1, "relu"),
             (1, 24, 13, 13, 24, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), 24, "relu6"),
             (2, 16, 10, 8, 32, 3, 3, (1, 1), (2, 2, 2, 2), (2, 2), 4, "gelu"),
             (3, 40, 6, 7, 70, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1), 1, "none"),
             (1, 3, 20, 20, 16, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1), 1, "relu")]
    for ci, (N, Cin, H, W, M, kH, kW, s, pads, d, g, act) in enumerate(cases):
        X = synth.round_to(r.standard_normal((N, Cin, H, W)), dtype)
        Wt = synth.round_to(r.standard_normal((M, Cin // g, kH, kW)) / math.sqrt(kH * kW * Cin // g), dtype)
        b = synth.round_to(r.uniform(-0.5, 0.5, M), dtype)
        ho, wo = ox.conv_out_hw(H, W, kH, kW, s, pads, d)
        Rr = synth.round_to(r.standard_normal((N, M, ho, wo)), dtype)
        say("residual engine", dtype, (N, Cin, H, W, M, kH, kW, s, pads, d, g, act))
        Y = run_conv_res(ox, X, Wt, b, Rr, dtype, s, pads, d, g, act, in_place=(ci == 1))
        assert_close(host64(Y), oracle.conv2d(X, Wt, b, s, pads, d, g, act, residual=Rr), dtype,
                     "residual engine case %d" % ci)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_c3_resnet50_bottleneck_residual(ox, dtype):
    # the bottleneck's last 1x1 (C/4 -> C) with the block input as residual
    # and ReLU, at batch 32, every output
    for li, layer in enumerate(synth.resnet50_layers(32)):
        if not layer.name.endswith("1x1b"):
            continue
        X, Wt, b = conv_layer_tensors(layer, 3, li, dtype)
        Rr = synth.round_to(np.random.default_rng([7, li]).standard_normal((layer.N, layer.M, layer.H, layer.W)),
                            dtype)
        say("C3 residual", dtype, layer.name)
        Y = run_conv_res(ox, X, Wt, b, Rr, dtype, (1, 1), (0, 0, 0, 0), (1, 1), 1, "relu", ws=True)
        assert not torch.isnan(Y).any().item(), layer.name
        got = host64(Y)
        del Y
        ref = oracle.conv2d(X, Wt, b, act="relu", residual=Rr)
        assert_close(got, ref, dtype, layer.name)


# --------------------------------------- BatchNorm + act, MaxPool, GAP --

def bn_params(r, Cc):
    g = r.uniform(0.5, 1.5, Cc).astype(np.float32)
    be = (r.standard_normal(Cc) * 0.3).astype(np.float32)
    mu = (r.standard_normal(Cc) * 0.3).astype(np.float32)
    var = r.uniform(0.5, 1.5, Cc).astype(np.float32)
    return g, be, mu, var


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batchnorm_act(ox, dtype):
    # vector path (plane length a multiple of the vector), element path (odd
    # planes, a misaligned X), in place, every activation
    r = np.random.default_rng(8080)
    for ci, (N, Cc, H, W, act, xoff, in_place) in enumerate([
            (3, 16, 8, 8, "relu", 0, False), (2, 7, 5, 9, "relu6", 0, False), (1, 33, 7, 7, "gelu", 1, False),
            (2, 64, 28, 28, "none", 0, True), (4, 5, 1, 1, "relu", 0, False)]):
        X = synth.round_to(r.standard_normal((N, Cc, H, W)) * 2, dtype)
        g, be, mu, var = bn_params(r, Cc)
        say("bn act", dtype, (N, Cc, H, W, act, xoff, in_place))
        Xd = misaligned(dev(X, dtype), xoff) if xoff else dev(X, dtype)
        prm = [torch.from_numpy(v).cuda() for v in (g, be, mu, var)]
        Y = ox.ox_batchnorm_act(Xd, *prm, eps=1e-5, act=act, Y=Xd if in_place else None)
        torch.cuda.synchronize()
        ref = oracle.batchnorm_act(X, g, be, mu, var, 1e-5, act)
        assert_close(host64(Y), ref, dtype, "bn case %d" % ci)


@pytest.mark.parametrize("simple", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_maxpool(ox, dtype, simple, monkeypatch):
    # a maximum of values exact in the dtype is one of them: bit-exact; the
    # staged-band (depthwise) kernel and the one-thread-per-output kernel
    if simple:
        monkeypatch.setenv("OX_POOL_SIMPLE", "1")
    r = np.random.default_rng(9090)
    ran = 0
    while ran < 40:
        N, Cc = int(r.integers(1, 3)), int(r.integers(1, 6))
        H, W = int(r.integers(1, 15)), int(r.integers(1, 15))
        kH, kW = int(r.integers(1, 4)), int(r.integers(1, 4))
        s = (int(r.integers(1, 3)), int(r.integers(1, 3)))
        d = (int(r.integers(1, 3)), int(r.integers(1, 3)))
        pads = tuple(int(v) for v in r.integers(0, 2, 4))
        if pads[0] >= (kH - 1) * d[0] + 1 or pads[2] >= (kH - 1) * d[0] + 1 or \
           pads[1] >= (kW - 1) * d[1] + 1 or pads[3] >= (kW - 1) * d[1] + 1:
            continue
        ho, wo = ox.conv_out_hw(H, W, kH, kW, s, pads, d)
        if ho < 1 or wo < 1:
            continue
        X = synth.round_to(r.standard_normal((N, Cc, H, W)), dtype)
        say("maxpool", dtype, (N, Cc, H, W, kH, kW, s, pads, d))
        Y = ox.ox_maxpool2d(dev(X, dtype), (kH, kW), s, pads, d, Y=nan_like((N, Cc, ho, wo), dtype))
        torch.cuda.synchronize()
        assert np.array_equal(host64(Y), oracle.maxpool2d(X, (kH, kW), s, pads, d)), ran
        ran += 1


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_global_avgpool(ox, dtype):
    r = np.random.default_rng(1010)
    for N, Cc, H, W in [(2, 7, 7, 7), (1, 5, 1, 1), (3, 4, 15, 20), (2, 3, 9, 1)]:
        X = synth.round_to(r.standard_normal((N, Cc, H, W)), dtype)
        say("gap", dtype, (N, Cc, H, W))
        Y = ox.ox_global_avgpool(dev(X, dtype), Y=nan_like((N, Cc, 1, 1), dtype))
        torch.cuda.synchronize()
        assert_close(host64(Y), oracle.global_avgpool(X), dtype, "gap")
        Y2 = ox.ox_global_avgpool(dev(X, dtype))
        torch.cuda.synchronize()
        assert torch.equal(Y.view(-1), Y2.view(-1))     # fixed summation order


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_resnet50_pool_and_bn_full_size(ox, dtype):
    # the ResNet-50 stem MaxPool (3x3 s2 p1, 64 x 112^2 -> 56^2), a
    # pre-activation BN + ReLU at stage 1 and the head's GlobalAveragePool,
    # batch 32, every output
    r = np.random.default_rng(2020)
    X = synth.round_to(r.standard_normal((32, 64, 112, 112)), dtype)
    Y = ox.ox_maxpool2d(dev(X, dtype), (3, 3), (2, 2), (1, 1, 1, 1))
    torch.cuda.synchronize()
    assert not torch.isnan(Y).any().item()
    got = host64(Y)
    ref = oracle.maxpool2d(X, (3, 3), (2, 2), (1, 1, 1, 1))
    assert np.array_equal(got, ref)
    X = synth.round_to(r.standard_normal((32, 256, 56, 56)), dtype)
    g, be, mu, var = bn_params(r, 256)
    Y = ox.ox_batchnorm_act(dev(X, dtype), *[torch.from_numpy(v).cuda() for v in (g, be, mu, var)],
                            act="relu")
    torch.cuda.synchronize()
    assert not torch.isnan(Y).any().item()
    got = host64(Y)
    del Y
    assert_close(got, oracle.batchnorm_act(X, g, be, mu, var, 1e-5, "relu"), dtype, "bn full size")
    X = synth.round_to(r.standard_normal((32, 2048, 7, 7)), dtype)
    Y = ox.ox_global_avgpool(dev(X, dtype))
    torch.cuda.synchronize()
    assert_close(host64(Y), oracle.global_avgpool(X), dtype, "gap full size")
