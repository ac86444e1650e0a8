"""Pins of the oracle's quantizer (model card "hampsonw/DeepSeek-V4-Flash-0731-WNA16",
"How it was created" steps 2-5: symmetric b-bit weights per K group, an
importance-weighted scale search, packed signed codes, weighted and unweighted
reconstruction error).  The readings Q1-Q6 are stated in oracle/moe_oracle.c.

None of these re-types the oracle's arithmetic: the FP16 rounding is checked
against numpy's own float16 conversion, the search against matrices built from
known codes and power-of-two scales (which it must recover exactly),
invariances, nesting of the candidate grids, and the error sums against the
reconstruction decoded with the already-pinned format functions.
"""
import numpy as np
import pytest

from oracle import oracle as O


def bf16_bits(x):
    """float64 values exactly representable in BF16 -> BF16 bit patterns."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in BF16"
    return (b >> 16).astype(np.uint16)


def decoded(res, K, bits, group):
    """Codes (via the pinned field decoder) and per-element scales."""
    rows = res["codes"].shape[0]
    q = np.stack([O.codes(res["codes"][n], K, bits) for n in range(rows)])
    s = np.array([[O.f16_to_f64(int(h)) for h in r] for r in res["scales"]])
    return q, np.repeat(s, group, axis=1)


def test_f16_rounding_matches_numpy_on_every_half_and_midpoint():
    # every finite non-negative half, and the midpoints between neighbours
    h = np.arange(0x7C00, dtype=np.uint16)              # +0 .. 65504
    v = h.view(np.float16).astype(np.float64)
    for x in v[::7]:
        assert O.f64_to_f16_rne(x) == int(np.float16(x).view(np.uint16))
    mids = (v[:-1] + v[1:]) / 2
    for x in mids[::5]:
        assert O.f64_to_f16_rne(x) == int(np.float16(x).view(np.uint16))   # ties to even
    for x in [1e-8, 3e-8, 6e-5, 0.1, 1.0 / 3.0, 1000.1, 65503.9]:
        assert O.f64_to_f16_rne(x) == int(np.float16(x).view(np.uint16))


@pytest.mark.parametrize("bits,group,ncand,cstar", [(2, 32, 4, 2), (2, 128, 8, 4), (4, 64, 16, 2),
                                                    (4, 128, 8, 1)])
def test_recovers_known_codes_and_power_of_two_scales(bits, group, ncand, cstar):
    """W = q * s with s = 2^j and the most negative code in every group: the
    span factor (2^b - 1)/2 and the candidate grid 1 - c/(2C) make candidate
    c* land exactly on s, the only zero-error candidate."""
    rng = np.random.default_rng(bits * 1000 + group)
    rows, K = 5, 2 * group
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    q = rng.integers(lo, hi + 1, size=(rows, K))
    q[:, ::group] = lo                                  # amax = 2^(b-1) * s in every group
    j = rng.integers(-12, 0, size=(rows, K // group))
    s = np.repeat(np.ldexp(1.0, j), group, axis=1)
    res = O.quantize(bf16_bits(q * s), bits, group, ncand)
    qd, sd = decoded(res, K, bits, group)
    assert np.array_equal(qd, q)
    assert np.array_equal(sd, s)
    assert np.all(res["choice"] == cstar)
    assert res["sums"][0] == 0.0 and res["sums"][2] == 0.0


@pytest.mark.parametrize("bits,group", [(2, 128), (4, 32)])
def test_power_of_two_rescaling_and_in_group_permutation(bits, group):
    rng = np.random.default_rng(7)
    rows, K = 4, 2 * group
    w = np.asarray(rng.normal(size=(rows, K)) * 0.05, np.float32)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)        # truncate to BF16
    wf = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    imp = rng.uniform(0.1, 3.0, size=K).astype(np.float32)
    a = O.quantize(wb, bits, group, 12, imp)
    b = O.quantize(bf16_bits(wf * 8.0), bits, group, 12, imp)
    assert np.array_equal(a["codes"], b["codes"])
    sa = np.array([[O.f16_to_f64(int(h)) for h in r] for r in a["scales"]])
    sb = np.array([[O.f16_to_f64(int(h)) for h in r] for r in b["scales"]])
    assert np.array_equal(sb, sa * 8.0)
    # permute the channels inside each group (and their importance)
    perm = np.concatenate([g * group + rng.permutation(group) for g in range(K // group)])
    c = O.quantize(wb[:, perm], bits, group, 12, imp[perm])
    assert np.array_equal(c["scales"], a["scales"])
    qa, _ = decoded(a, K, bits, group)
    qc, _ = decoded(c, K, bits, group)
    assert np.array_equal(qc, qa[:, perm])


def test_importance_uniform_equals_unweighted_and_scale_free():
    rng = np.random.default_rng(11)
    w = (np.asarray(rng.normal(size=(6, 256)), np.float32).view(np.uint32) >> 16).astype(np.uint16)
    a = O.quantize(w, 2, 64, 10)
    b = O.quantize(w, 2, 64, 10, np.ones(256, np.float32))
    c = O.quantize(w, 2, 64, 10, np.full(256, 4.0, np.float32))
    for r in (b, c):
        assert np.array_equal(r["codes"], a["codes"]) and np.array_equal(r["scales"], a["scales"])
    assert b["sums"][2] == a["sums"][0] and b["sums"][3] == a["sums"][1]


@pytest.mark.parametrize("bits", [2, 4])
def test_weighted_search_beats_plain_rtn_and_nested_grids_never_lose(bits):
    rng = np.random.default_rng(20 + bits)
    K, group = 512, 128
    w = (np.asarray(rng.standard_t(4, size=(8, K)) * 0.02, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    imp = np.asarray(rng.lognormal(0, 1.5, size=K), np.float32)
    rtn = O.quantize(w, bits, group, 1, imp)
    prev = rtn
    for C in (2, 4, 8, 16):
        r = O.quantize(w, bits, group, C, imp)
        assert r["sums"][2] <= prev["sums"][2] * (1 + 1e-12)   # grid of C is inside grid of 2C
        prev = r
    assert prev["sums"][2] < rtn["sums"][2]
    # the weighted winner is no worse, by the weighted error, than the unweighted one
    unw = O.quantize(w, bits, group, 16)
    qd, sd = decoded(unw, K, bits, group)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    alt = float((imp.astype(np.float64) * (wf - qd * sd) ** 2).sum())
    assert prev["sums"][2] <= alt * (1 + 1e-12)


def test_error_sums_match_the_decoded_reconstruction():
    rng = np.random.default_rng(5)
    K, group, bits = 256, 32, 4
    w = (np.asarray(rng.normal(size=(7, K)), np.float32).view(np.uint32) >> 16).astype(np.uint16)
    imp = np.asarray(rng.uniform(0, 2, size=K), np.float32)
    r = O.quantize(w, bits, group, 6, imp)
    qd, sd = decoded(r, K, bits, group)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d2 = (wf - qd * sd) ** 2
    im = imp.astype(np.float64)
    ref = np.array([d2.sum(), (wf ** 2).sum(), (im * d2).sum(), (im * wf ** 2).sum()])
    np.testing.assert_allclose(r["sums"], ref, rtol=1e-12)


def test_plain_rtn_error_bound_and_zero_groups():
    rng = np.random.default_rng(9)
    K, group, bits = 256, 64, 2
    wf = np.asarray(rng.normal(size=(5, K)), np.float32)
    wf[2, 64:128] = 0.0                                   # an all-zero group
    w = (wf.view(np.uint32) >> 16).astype(np.uint16)
    r = O.quantize(w, bits, group, 1)
    qd, sd = decoded(r, K, bits, group)
    x = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(x - qd * sd)
    # round to nearest: within half a step, or one step at the clamped top end
    inside = x / np.where(sd > 0, sd, 1) < (1 << (bits - 1)) - 0.5
    assert np.all(err[inside] <= sd[inside] / 2 + 1e-12)
    assert np.all(err <= sd * 1.01 + 1e-12)
    assert r["scales"][2, 1] == 0 and np.all(qd[2, 64:128] == 0)
    # every candidate of a zero group ties at zero error: the first one wins
    r8 = O.quantize(w, bits, group, 8)
    assert r8["choice"][2, 1] == 0


def test_codes_round_half_to_even():
    """Plain RTN with amax = 1.5 * 2^-3 (2-bit: the base scale is exactly
    2^-3): w / s = 0.5 rounds to 0 and -1.5 to -2 (ties to even), 2.5 * s
    (4-bit span) to 2."""
    s2 = 2.0 ** -3
    w = np.zeros((1, 32))
    w[0, :4] = [1.5 * s2, 0.5 * s2, -1.5 * s2, -0.5 * s2]
    r = O.quantize(bf16_bits(w), 2, 32, 1)
    q, sd = decoded(r, 32, 2, 32)
    assert sd[0, 0] == s2
    assert list(q[0, :4]) == [1, 0, -2, 0]
    s4 = 2.0 ** -4                          # 4-bit: amax = 7.5 * s4
    w = np.zeros((1, 32))
    w[0, :4] = [7.5 * s4, 2.5 * s4, 3.5 * s4, -6.5 * s4]
    r = O.quantize(bf16_bits(w), 4, 32, 1)
    q, sd = decoded(r, 32, 4, 32)
    assert sd[0, 0] == s4
    assert list(q[0, :4]) == [7, 2, 4, -6]
