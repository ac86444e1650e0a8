"""The quantizer kernel's candidate search forms w * rcp(s) instead of the FP32
division w / s (the stored codes still use the division).  Its claim: with w
a BF16 value and s an FP16 scale, the error |w - s q| of every candidate is the
same either way, for any reciprocal within one ulp of 1/s, because a quotient
that is not exactly a half-integer lies far from one, and at an exact
half-integer both neighbouring codes leave the same error.  Checked here on the
CPU in IEEE float32 (numpy), over a million sampled (w, s) pairs and the
reciprocal perturbed by one ulp either way."""
import numpy as np
import pytest


def bf16_round(a):
    b = np.asarray(a, np.float32).view(np.uint32)
    lsb = (b >> 16) & 1
    return ((b + 0x7FFF + lsb) & 0xFFFF0000).view(np.float32)


@pytest.mark.parametrize("bits", [2, 4])
def test_reciprocal_search_gives_the_division_errors(bits):
    rng = np.random.default_rng(bits)
    n = 1 << 20
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    # FP16 scales over a wide range, including subnormal halves
    s = rng.uniform(-24, 15, n)
    s = np.float16(np.exp2(s)).astype(np.float32)
    s = s[(s > 0) & np.isfinite(s)]
    m = s.size
    # weights within and beyond the code span, plus exact half-integer quotients
    w = bf16_round(s * rng.uniform(-1.5, 1.5, m) * (1 << bits))
    half = (rng.integers(lo, hi + 1, m) + np.float32(0.5)).astype(np.float32)
    exact = bf16_round(half * s)
    use = rng.random(m) < 0.25
    w = np.where(use & (exact == half * s), exact, w).astype(np.float32)

    q_div = np.clip(np.rint(w / s), lo, hi)
    e_div = np.abs(w.astype(np.float64) - s.astype(np.float64) * q_div)
    r0 = (np.float32(1.0) / s).astype(np.float32)
    for r in (r0, np.nextafter(r0, np.float32(np.inf)), np.nextafter(r0, np.float32(0))):
        q_rcp = np.clip(np.rint((w * r).astype(np.float32)), lo, hi)
        e_rcp = np.abs(w.astype(np.float64) - s.astype(np.float64) * q_rcp)
        bad = e_rcp != e_div
        assert not bad.any(), (w[bad][:5], s[bad][:5], q_div[bad][:5], q_rcp[bad][:5])
    # the exact half-integer cases were exercised
    assert np.sum(use & (w == exact)) > m // 50
