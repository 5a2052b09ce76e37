"""Oracle pins for Lion with FlashOptim's compressed momentum.

The FlashOptim digest names FlashLion among the optimizers the method
covers ("Core method", "Practical advice") but prints no Lion update; the
oracle takes the published Lion rule: the step direction is the sign of the
interpolation c = beta1*m + (1-beta1)*g, the momentum is updated with beta2,
and weight decay is decoupled (theta <- (1 - lr*wd)*theta - lr*sign(c)).
These tests pin that structure through behaviour a plausible slip would
change: the direction of the step, which beta feeds which quantity, whether
the sign is taken of c, of g or of the new momentum, sign(0) = 0, and
decoupled versus coupled decay.  Rebuilt weights are compared within the
weight split's own precision; momenta within the companded quantiser's
error (both bounds are pinned in the split / quantiser tests).
"""
import numpy as np
import pytest

from test_oracle_steps import bf16_bits, bf16_f32

LR = 2.0 ** -10


def rebuilt(orc, st):
    return orc.unsplit(st.tb, st.rho).astype(np.float64)


def split_tol(x):
    # the BF16 + INT8 split keeps |error| <= ULP_bf16(x)/2 / 127 (plus rounding)
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64) * 2.0 ** 16 / 254 \
        + 2.0 ** -140


def start(orc, n, seed=0):
    rng = np.random.default_rng(seed)
    # weights in [0.5, 0.75): theta_hat -/+ 2^-10 stays inside [0.25, 1), where it is exact
    theta = (0.5 + rng.integers(0, 2 ** 18, n) * 2.0 ** -20).astype(np.float32)
    st = orc.State(theta, "lion")
    return st, rng


def test_first_step_moves_against_the_gradient_sign_by_lr(orc):
    n = 32 * 40 + 5
    st, rng = start(orc, n)
    theta0 = rebuilt(orc, st)
    g = bf16_bits(rng.standard_normal(n))
    g[::7] = 0                                      # sign(0) = 0: no move
    hp = dict(lr=LR, beta1=0.9, beta2=0.99, weight_decay=0.0)
    th, m = orc.step(st, g, 1, hp, want_fp32=True)
    expect = theta0 - LR * np.sign(bf16_f32(g))      # m = 0, so sign(c) = sign(g)
    np.testing.assert_array_equal(th.astype(np.float64), expect)
    assert np.all(np.abs(rebuilt(orc, st) - expect) <= split_tol(expect))


def test_momentum_uses_beta2_and_direction_uses_beta1(orc):
    n = 32 * 8
    st, _ = start(orc, n, seed=1)
    hp = dict(lr=LR, beta1=0.5, beta2=0.9, weight_decay=0.0)
    g = bf16_bits(np.full(n, 1.0, np.float32))
    _, m1 = orc.step(st, g, 1, hp, want_fp32=True)
    # from m = 0 the new momentum is (1 - beta2) g = 0.1, not (1 - beta1) g = 0.5
    np.testing.assert_allclose(m1, 0.1, rtol=1e-6)
    mq = orc.dequant_m(st.qm, st.sm)
    np.testing.assert_allclose(mq, 0.1, rtol=2e-2)


def test_direction_is_the_interpolation_not_the_gradient(orc):
    # m = 0.01 > 0 and g < 0 with beta1 = 0.9: c = 0.009 - 0.0005 > 0, so the
    # weight moves down although the gradient is negative
    n = 32 * 4
    st, _ = start(orc, n, seed=2)
    hp = dict(lr=LR, beta1=0.9, beta2=0.99, weight_decay=0.0)
    orc.step(st, bf16_bits(np.full(n, 1.0, np.float32)), 1, hp)        # m <- 0.01
    before = rebuilt(orc, st)
    orc.step(st, bf16_bits(np.full(n, -0.005, np.float32)), 2, hp)
    d = rebuilt(orc, st) - before
    assert np.all(np.abs(d + LR) <= 2 * split_tol(before)), d[:4]


def test_direction_is_not_the_new_momentum(orc):
    # beta1 = 0 makes c = g < 0 while the new momentum (beta2 = 0.99) stays > 0:
    # the weight moves up
    n = 32 * 4
    st, _ = start(orc, n, seed=3)
    hp = dict(lr=LR, beta1=0.0, beta2=0.99, weight_decay=0.0)
    orc.step(st, bf16_bits(np.full(n, 1.0, np.float32)), 1, hp)
    before = rebuilt(orc, st)
    _, m2 = orc.step(st, bf16_bits(np.full(n, -0.005, np.float32)), 2, hp, want_fp32=True)
    assert np.all(m2 > 0)
    d = rebuilt(orc, st) - before
    assert np.all(np.abs(d - LR) <= 2 * split_tol(before)), d[:4]


@pytest.mark.parametrize("wd", [0.1, 1.0])
def test_weight_decay_is_decoupled(orc, wd):
    # zero gradient and zero momentum: sign(c) = 0, so only the decay acts and
    # theta_new = (1 - lr*wd) * theta.  Coupled decay (wd*theta added to the
    # gradient) would instead move every weight by a full lr.
    n = 32 * 10 + 3
    st, _ = start(orc, n, seed=4)
    theta0 = rebuilt(orc, st)
    hp = dict(lr=LR, beta1=0.9, beta2=0.99, weight_decay=wd)
    th, m = orc.step(st, np.zeros(n, np.uint16), 1, hp, want_fp32=True)
    expect = (1.0 - LR * wd) * theta0
    assert np.all(np.abs(th - expect) <= np.spacing(np.float32(expect)).astype(np.float64))
    assert not m.any() and not st.qm.any() and not st.sm.any()


def test_fused_requant_and_resplit_equal_the_codec(orc):
    # the stored state after a step is exactly the pinned quantiser and split
    # applied to the step's fp32 outputs
    n = 32 * 50 + 17
    rng = np.random.default_rng(5)
    st = orc.State((rng.standard_normal(n) * 0.02).astype(np.float32), "lion")
    hp = dict(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.1)
    for t in (1, 2, 3):
        g = bf16_bits(rng.standard_normal(n) * 1e-3)
        th, m = orc.step(st, g, t, hp, want_fp32=True)
        qm, sm = orc.quant_m(m)
        tb, rho = orc.split(th)
        np.testing.assert_array_equal(st.qm, qm)
        np.testing.assert_array_equal(st.sm, sm)
        np.testing.assert_array_equal(st.tb, tb)
        np.testing.assert_array_equal(st.rho, rho)
