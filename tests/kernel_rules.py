"""Host-side applicability rules of kernels whose choice the tests check
(restated from the library's planning, for the tests' expectations)."""


def dwr_applies(dtype, W, s, vmax=8, xoff_bytes=0):
    """The row-segment depthwise 3x3 kernel (pads 1, stride s): some segment
    width V (outputs per lane) with a 4-, 8- or 16-byte input load, V | Wo,
    Wo / V <= 64, X aligned to the load; for bf16 at stride 1 whole pairs (V
    even) on even widths and one output per lane (a 2-byte load) on odd
    ones."""
    E = 4 if dtype == "f32" else 2
    Wo = (W - 1) // s + 1
    if W != Wo * s:
        return False
    odd1 = dtype == "bf16" and s == 1 and W % 2 == 1
    for V in ((1,) if odd1 else (8, 4, 2, 1)):
        lb = V * s * E
        if V > vmax or lb > 16 or (lb < 4 and not odd1) or (dtype == "bf16" and s == 1 and V % 2 and not odd1):
            continue
        if Wo % V or Wo // V > 64 or xoff_bytes % lb:
            continue
        return True
    return False
