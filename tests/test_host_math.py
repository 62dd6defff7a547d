"""Host-side checks of numeric facts the GPU kernels rely on (no GPU)."""
from fractions import Fraction

import numpy as np


def _rn32(q: Fraction) -> np.float32:
    """Exact round-to-nearest-even of a rational to fp32."""
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.array(c).view(np.uint32)) & 1))


def test_div6_fma_correction_exact_for_all_bf16():
    """The quantizer computes f32(b / 6) as q0 = b*c, r = fma(-q0, 6, b),
    q = fma(r, c, q0) with c = RN(1/6).  For every non-negative finite bf16 b
    this equals the correctly rounded quotient."""
    c = np.float32(1.0) / np.float32(6.0)
    assert float(c) == 0.16666667163372039794921875
    Fc = Fraction(float(c))
    bad = []
    for u in range(0, 0x7F80, 1):
        b = np.array(u << 16, np.uint32).view(np.float32)[()]
        Fb = Fraction(float(b))
        want = _rn32(Fb / 6)
        q0 = _rn32(Fb * Fc)
        r = _rn32(Fb - Fraction(float(q0)) * 6)
        q = _rn32(Fraction(float(r)) * Fc + Fraction(float(q0)))
        if q != want:
            bad.append(float(b))
    assert not bad, bad[:10]


def test_two_stage_e2m1_equals_rne_of_half_steps():
    """The pages' half-step table equals round-to-nearest-even onto the E2M1
    grid of the half step value (what the GPU's FP4 conversion computes):
    for each half step hs, the nearest magnitude to hs/2, ties to the even
    index."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    table = [0, 1, 2, 3, 4, 4, 5, 6, 6, 6, 6, 7, 7]  # reading of the pages' step_to_idx
    for hs in range(13):
        v = hs / 2
        d = [abs(g - v) for g in grid]
        m = min(d)
        cands = [i for i, x in enumerate(d) if x == m]
        idx = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        assert idx == table[hs], hs
