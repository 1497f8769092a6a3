"""Parity rule and helpers shared by the GPU tests.

The rule is the one the onnx-vulkan-rs validation uses: an element passes
when |got - ref| <= atol + rtol*|ref|, and the report gives the worst element
as a fraction of its allowance (max_tolerance_ratio) and where it is.  A NaN
anywhere fails.  Tolerances: fp32 1e-4 / 1e-4; bf16 inputs with fp32
accumulation 1e-2 / 1e-2; int8 / int32 results must be bit-exact.
"""
import numpy as np

TOL = {"f32": (1e-4, 1e-4), "bf16": (1e-2, 1e-2)}


def tolerance_report(got, ref, atol, rtol):
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return {"ok": True, "max_tolerance_ratio": 0.0, "argmax": -1, "nan": False}
    nan = bool(np.isnan(got).any() or np.isnan(ref).any())
    allow = atol + rtol * np.abs(ref)
    ratio = np.abs(got - ref) / allow
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    i = int(np.argmax(ratio))
    return {"ok": (not nan) and bool(ratio[i] <= 1.0), "max_tolerance_ratio": float(ratio[i]),
            "argmax": i, "got": float(got[i]), "ref": float(ref[i]), "nan": nan}


def assert_close(got, ref, dtype, what=""):
    atol, rtol = TOL[dtype]
    r = tolerance_report(got, ref, atol, rtol)
    assert r["ok"], "%s: parity failed (%s): %r" % (what, dtype, r)
    return r


def sample_indices(total, n, seed, extra_tail=64):
    """Seeded sample of flat output indices: n random ones, plus the first and
    the last `extra_tail` (the ragged tail of every tiling)."""
    r = np.random.default_rng(seed)
    idx = r.integers(0, total, min(n, total)) if total > 0 else np.zeros(0, np.int64)
    head = np.arange(min(extra_tail, total))
    tail = np.arange(max(0, total - extra_tail), total)
    return np.unique(np.concatenate([idx, head, tail])).astype(np.int64)
