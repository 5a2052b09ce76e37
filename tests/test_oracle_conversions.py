"""Oracle pins: bf16 / fp16 conversions against independent library routines.

The oracle writes both conversions from the IEEE-754 definition of the
formats (round to nearest, ties to even, gradual underflow).  torch's CPU
bfloat16 / float16 casts and numpy's float16 cast are independent
implementations of the same definition; they must agree bit for bit on every
non-NaN input.  Coverage: every (sign, exponent, kept-mantissa) pattern times
every class of discarded tail (0, 1 ulp, just below / at / above the halfway
point, all ones, plus random tails), and whole binades exhaustively.
"""
import numpy as np
import pytest
import torch


def _tails(nbits, rng, extra=24):
    half = 1 << (nbits - 1)
    full = (1 << nbits) - 1
    fixed = [0, 1, 2, half - 2, half - 1, half, half + 1, half + 2, full - 1, full]
    rnd = rng.integers(0, 1 << nbits, extra)
    return np.unique(np.array(fixed + list(rnd), dtype=np.uint32))


def _structured(kept_bits_total, tail_bits, rng):
    tops = np.arange(1 << kept_bits_total, dtype=np.uint32) << tail_bits
    tails = _tails(tail_bits, rng)
    return (tops[:, None] | tails[None, :]).reshape(-1)


def _not_nan(bits):
    x = bits.view(np.float32)
    return ~np.isnan(x)


def test_env(orc):
    assert orc.lib().orc_env_ok() == 1


def test_bf16_structured_vs_torch(orc):
    rng = np.random.default_rng(0)
    bits = _structured(16, 16, rng)             # all 2^16 upper halves x 34 tails
    bits = bits[_not_nan(bits)]
    ours = orc.bf16_rne(bits.view(np.float32))
    ref = torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(ours, ref.view(np.uint16))


@pytest.mark.parametrize("first_exp", [0, 1, 120, 127, 254])
def test_bf16_binade_exhaustive_vs_torch(orc, first_exp):
    # one whole binade (both signs): exponent field first_exp, all 2^23 mantissas
    m = np.arange(1 << 23, dtype=np.uint32)
    for sign in (0, 1):
        bits = (np.uint32(sign) << 31) | (np.uint32(first_exp) << 23) | m
        x = bits.view(np.float32)
        ours = orc.bf16_rne(x)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(ours, ref)


def test_bf16_specials(orc):
    x = np.array([np.inf, -np.inf, 0.0, -0.0, 3.3895314e38, 3.3961e38, 3.4e38], np.float32)
    b = orc.bf16_rne(x)
    assert list(b[:4]) == [0x7F80, 0xFF80, 0x0000, 0x8000]
    assert b[4] == 0x7F7F and b[6] == 0x7F80
    nan = orc.bf16_rne(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_f16_structured_vs_torch_and_numpy(orc):
    rng = np.random.default_rng(1)
    bits = _structured(19, 13, rng)             # sign+exp+10 kept mantissa bits x tails
    bits = bits[_not_nan(bits)]
    x = bits.view(np.float32)
    ours = orc.f16_rne(x)
    ref_t = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref_t)
    sub = x[::97]
    with np.errstate(over="ignore"):
        ref_n = sub.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(orc.f16_rne(sub), ref_n)


def test_f16_small_binades_exhaustive(orc):
    # every fp32 whose magnitude lies in [2^-26, 2^-13): the fp16 subnormal
    # range, its underflow-to-zero boundary and the first normal binade
    m = np.arange(1 << 23, dtype=np.uint32)
    exps = np.arange(127 - 26, 127 - 13, dtype=np.uint32)
    bits = ((exps[:, None] << 23) | m[None, :]).reshape(-1)
    x = bits.view(np.float32)
    ours = np.empty(x.size, np.uint16)
    def run(lo, hi):
        ours[lo:hi] = orc.f16_rne(x[lo:hi])
    orc.chunked(run, None, None, x.size)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(orc.f16_rne(-x[::1001]), ref[::1001] | 0x8000)


def test_f16_to_f32_all_patterns(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok].view(np.uint32), ref[ok].view(np.uint32))
    assert np.isnan(ours[~ok]).all()


def test_f16_specials(orc):
    x = np.array([65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0001,
                  np.inf], np.float32)
    assert list(orc.f16_rne(x)) == [0x7BFF, 0x7BFF, 0x7C00, 0x7C00, 0x0001, 0x0000, 0x0001,
                                    0x7C00]
