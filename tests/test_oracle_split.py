"""Oracle pins: weight splitting (FlashOptim digest, "Core method > Weight
splitting: ULP-based error correction", Eq. 1-2, Alg. 1; Fig. 3 in the
experiments section).

theta' is theta rounded to BF16; theta lies within ULP(theta')/2 of it, so the
error normalised by ULP(theta')/2 is in [-1, 1] and is quantised uniformly to
an INT8 code.  The tests compute the code from that definition in float64,
taking ULP(theta') as the gap from |theta'| to the next BF16 value (a route
independent of the oracle's exponent arithmetic), with torch's BF16 cast for
theta'.
"""
import numpy as np
import pytest
import torch


def bf16_torch(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bf16_value(b):
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def half_ulp_by_successor(tb):
    """Half the gap from |theta'| to the next larger BF16 magnitude."""
    mag = (tb & 0x7FFF).astype(np.uint32)
    here = bf16_value(mag.astype(np.uint16))
    nxt = bf16_value(np.minimum(mag + 1, 0x7F7F).astype(np.uint16))
    gap = nxt - here
    gap = np.where(mag == 0x7F7F, 2.0 ** 120, gap)   # successor of the largest is Inf
    return gap / 2.0


def ref_split(x):
    x = np.asarray(x, np.float32)
    tb = bf16_torch(x)
    t = bf16_value(tb)
    fin = np.isfinite(t)
    h = half_ulp_by_successor(tb)
    with np.errstate(invalid="ignore"):
        e = (x.astype(np.float64) - t) / h          # exact in float64
        rho = np.clip(np.rint(e * 127.0), -127, 127)
    rho = np.where(fin, rho, 0).astype(np.int8)
    return tb, rho, e, h


def binade(exp_field, sign=0):
    m = np.arange(1 << 23, dtype=np.uint32)
    return ((np.uint32(sign) << 31) | (np.uint32(exp_field) << 23) | m).view(np.float32)


@pytest.mark.parametrize("exp_field", [0, 1, 9, 118, 126, 127, 200, 254])
def test_split_matches_definition_exhaustive_binade(orc, exp_field):
    for sign in (0, 1):
        x = binade(exp_field, sign)
        tb, rho = orc.split(x)
        rtb, rrho, e, h = ref_split(x)
        np.testing.assert_array_equal(tb, rtb)
        np.testing.assert_array_equal(rho, rrho)
        fin = np.isfinite(bf16_value(tb))
        assert np.all(np.abs(e[fin]) <= 1.0)       # the error interval the method rests on


def test_split_random_normal_and_specials(orc):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(1 << 20) * 0.02).astype(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max,
                         -np.finfo(np.float32).max, np.finfo(np.float32).tiny,
                         1.4e-45, -1.4e-45, 1.0, -1.0, 2.0 ** -133, 2.0 ** -134], np.float32)
    x = np.concatenate([x, specials])
    tb, rho = orc.split(x)
    rtb, rrho, _, _ = ref_split(x)
    np.testing.assert_array_equal(tb, rtb)
    np.testing.assert_array_equal(rho, rrho)
    nan_tb, nan_rho = orc.split(np.array([np.nan], np.float32))
    assert (nan_tb[0] & 0x7F80) == 0x7F80 and (nan_tb[0] & 0x7F) and nan_rho[0] == 0


def all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[np.isfinite(bf16_value(b))]


def test_unsplit_closed_forms(orc):
    tb = all_finite_bf16()
    t = bf16_value(tb)
    h = half_ulp_by_successor(tb)
    for code, expect in ((0, t), (127, t + h), (-127, t - h)):
        rho = np.full(tb.shape, code, np.int8)
        out = orc.unsplit(tb, rho).astype(np.float64)
        np.testing.assert_array_equal(out, expect)


def test_unsplit_within_rounding_of_exact_value(orc):
    # every finite bf16 value x every code: |theta_hat - (t + rho*h/127)| is one
    # final rounding plus the (tiny) rounding of rho/127
    tb = np.repeat(all_finite_bf16(), 255)
    rho = np.tile(np.arange(-127, 128, dtype=np.int8), tb.size // 255)
    out = orc.unsplit(tb, rho)
    t = bf16_value(tb)
    h = half_ulp_by_successor(tb)
    exact = t + rho.astype(np.float64) * h / 127.0
    ulp = np.spacing(np.abs(out)).astype(np.float64)
    err = np.abs(out.astype(np.float64) - exact)
    assert np.all(err <= 0.5 * ulp + h * 2.0 ** -22 + 2.0 ** -150)


@pytest.mark.parametrize("exp_field", [0, 5, 127, 140])
def test_roundtrip_error_bound(orc, exp_field):
    x = binade(exp_field)
    tb, rho = orc.split(x)
    y = orc.unsplit(tb, rho)
    h = half_ulp_by_successor(tb)
    err = np.abs(y.astype(np.float64) - x.astype(np.float64))
    bound = h / 254.0 + 0.5 * np.spacing(np.abs(x)).astype(np.float64) + h * 2.0 ** -22
    assert np.all(err <= bound)
    # the 8-bit code resolves 1/127 of the half-ULP: max error ~ h/254
    assert err.max() / h.max() > 0.9 / 254


def test_split_of_unsplit(orc):
    """Re-encoding a decoded weight.  For an interior code (|rho| < 127, and not
    below -63 when theta' is a power of two, where the spacing below is half)
    the decoded value rounds back to theta' and re-encodes to the same code.
    At rho = +-127 the decoded value is a BF16 midpoint and may legitimately
    re-round to the even neighbour; the value itself then moves by at most the
    round-trip bound."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(1 << 18) * 0.02).astype(np.float32)
    tb, rho = orc.split(x)
    y = orc.unsplit(tb, rho)
    tb2, rho2 = orc.split(y)
    pow2 = (tb & 0x7F) == 0
    interior = (np.abs(rho.astype(np.int32)) < 127) & ~(pow2 & (rho < -63))
    np.testing.assert_array_equal(tb2[interior], tb[interior])
    np.testing.assert_array_equal(rho2[interior], rho[interior])
    assert interior.mean() > 0.99
    y2 = orc.unsplit(tb2, rho2)
    h = np.maximum(half_ulp_by_successor(tb), half_ulp_by_successor(tb2))
    drift = np.abs(y2.astype(np.float64) - y.astype(np.float64))
    assert np.all(drift <= h / 254.0 + np.spacing(np.abs(y)).astype(np.float64) + h * 2.0 ** -22)


def test_general_code_range_reduces_to_int8(orc):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(1 << 16) * 0.02).astype(np.float32)
    tb, rho = orc.split(x)
    tbq, rhoq = orc.split_q(x, 127)
    np.testing.assert_array_equal(tb, tbq)
    np.testing.assert_array_equal(rho.astype(np.int32), rhoq)
    np.testing.assert_array_equal(orc.unsplit(tb, rho), orc.unsplit_q(tbq, rhoq, 127))


def _bit_perfect(orc, x, qmax):
    tb, rho = orc.split_q(x, qmax)
    y = orc.unsplit_q(tb, rho, qmax)
    same = y.view(np.uint32) == x.view(np.uint32)
    rel = np.abs(y.astype(np.float64) - x) / np.abs(x.astype(np.float64))
    return same.mean(), rel.mean(), rel.max()


def test_sixteen_bit_correction_claim(orc):
    """Fig. 3 / experiments section: a 16-bit correction on a BF16 weight
    rebuilds the FP32 value bit-perfectly about 99.92% of the time, with error
    below 1e-9.  Under the round-to-nearest reading with ULP taken above
    |theta'| the rate is 99.7-99.8%, and every miss is one FP32 ulp off, in
    one of two places the arithmetic predicts:

      * theta' rounded up to a power of two 2^k: h is the half-ULP above 2^k,
        twice the one below, so the code's step (h/32767) is about two FP32
        ulps of x < 2^k and about half of those x cannot be hit;
      * |rho| close to 2^14 (|x - theta'| close to h/2): the step is
        (1 + 2^-15) FP32 ulps, so after ~2^14 steps the decoded offset has
        drifted by half an ulp and the final rounding goes either way.

    So the test pins the exact miss counts (exhaustive over [1, 2) and on a
    seeded N(0, 0.02) sample, both deterministic in IEEE arithmetic), that no
    miss lies outside those two places, and reads 'error < 1e-9' as the mean
    relative error.  A ULP taken below |theta'| at powers of two (or in the
    direction of x) removes the first kind of miss and gives 99.99%+; no
    convention found reproduces 99.92% exactly."""
    one_binade = binade(127)                               # [1, 2), exhaustive
    rng = np.random.default_rng(6)
    normal = (rng.standard_normal(1 << 22) * 0.02).astype(np.float32)
    normal = normal[normal != 0]
    # (values, misses where theta' rounded up to a power of two, misses at |rho| ~ 2^14)
    for x, n_top, n_band in ((one_binade, 16385, 6375), (normal, 5840, 3302)):
        frac, mean_rel, max_rel = _bit_perfect(orc, x, 32767)
        assert mean_rel < 1e-9, mean_rel
        assert max_rel <= 2.0 ** -22
        tb, rho = orc.split_q(x, 32767)
        y = orc.unsplit_q(tb, rho, 32767)
        miss = y.view(np.uint32) != x.view(np.uint32)
        ulps = np.abs(y.view(np.int32).astype(np.int64) - x.view(np.int32).astype(np.int64))
        assert ulps.max() == 1
        t = bf16_value(tb)
        top = ((tb & 0x7F) == 0) & (np.abs(t) > np.abs(x))  # theta' = 2^k rounded up from below
        r = np.abs(rho.astype(np.int64))
        band = (r >= 16352) & (r <= 16416)
        assert (miss & top).sum() == n_top
        assert (miss & band & ~top).sum() == n_band
        assert not (miss & ~top & ~band).any()
        assert frac == 1.0 - (n_top + n_band) / x.size
    # exhaustive over [1, 2): 99.7287% bit-perfect (the page: 99.92%)
    assert abs((1.0 - (16385 + 6375) / 2 ** 23) - 0.997287) < 1e-6


def test_ulp_correction_beats_bf16_plus_bf16(orc):
    """Fig. 3: the ULP-normalised correction has orders-of-magnitude lower mean
    and max error than storing theta - theta' as a second BF16 (same 32 bits)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(1 << 20) * 0.02).astype(np.float32)
    x = x[x != 0]
    hi = bf16_value(bf16_torch(x))
    resid = bf16_value(bf16_torch((x.astype(np.float64) - hi).astype(np.float32)))
    base = (hi + resid).astype(np.float32)
    base_rel = np.abs(base.astype(np.float64) - x) / np.abs(x)
    _, ulp_mean, ulp_max = _bit_perfect(orc, x, 32767)
    assert ulp_mean * 100 < base_rel.mean()
    assert ulp_max * 10 < base_rel.max()
    # 8-bit correction: relative error bounded by (h/254)/|theta| <= 2^-8/254,
    # plus the final binary32 rounding (2^-24 relative)
    _, m8, x8 = _bit_perfect(orc, x, 127)
    assert x8 <= 2.0 ** -8 / 254 + 2.0 ** -24 + 2.0 ** -30 and m8 < x8
