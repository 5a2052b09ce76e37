"""Oracle pins: compression switched off for a layer (FlashOptim page,
"Practical advice": compression can be disabled per layer).  The state is an
FP32 master weight and FP32 moments, the update the same AdamW / SGD / Lion
as the compressed step, and the BF16 weight the model computes with is the
new master weight rounded to nearest.

Pinned against torch.optim.AdamW / torch.optim.SGD run in float64 from the
same state, torch's BF16 cast, Lion's closed forms, and a 40-step AdamW
trajectory in float64.
"""
import numpy as np
import pytest
import torch

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
SGD = dict(lr=0.1, momentum=0.9, weight_decay=1e-4)
LION = dict(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.1)


def ulp32(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


def bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bf16_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def random_state(orc, n, optimizer, seed):
    rng = np.random.default_rng(seed)
    st = orc.StateFP32((rng.standard_normal(n) * 0.02).astype(np.float32), optimizer)
    st.m[:] = (rng.standard_normal(n) * 3e-4).astype(np.float32)
    if st.v is not None:
        st.v[:] = ((rng.standard_normal(n) * 1e-3) ** 2 + 1e-9).astype(np.float32)
    return st, rng


@pytest.mark.parametrize("t,hp", [
    (1, HP), (2, HP), (50, HP),
    (5, dict(lr=3e-2, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1)),
])
def test_adamw_fp32_matches_torch_float64(orc, t, hp):
    n = 32 * 300 + 7
    st, rng = random_state(orc, n, "adamw", seed=t)
    if t == 1:
        st.m[:] = 0
        st.v[:] = 0
    g = bf16_bits(rng.standard_normal(n) * 1e-3)
    theta, m, v = (st.theta.astype(np.float64), st.m.astype(np.float64),
                   st.v.astype(np.float64))
    orc.step_fp32(st, g, t, hp)

    p = torch.tensor(theta, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    p.grad = torch.tensor(bf16_f32(g).astype(np.float64))
    opt.state[p] = {"step": torch.tensor(float(t - 1), dtype=torch.float64),
                    "exp_avg": torch.tensor(m), "exp_avg_sq": torch.tensor(v)}
    opt.step()
    ref_t = p.detach().numpy()
    ref_m = opt.state[p]["exp_avg"].numpy()
    ref_v = opt.state[p]["exp_avg_sq"].numpy()

    gg = bf16_f32(g).astype(np.float64)
    big_m = np.maximum.reduce([np.abs(hp["beta1"] * m), np.abs((1 - hp["beta1"]) * gg),
                               np.abs(ref_m)])
    assert np.all(np.abs(st.m - ref_m) <= 3 * ulp32(big_m) + 1e-45)
    assert np.all(np.abs(st.v - ref_v) <= 4 * ulp32(np.maximum(hp["beta2"] * v, ref_v)) + 1e-45)
    decayed = theta * (1 - hp["lr"] * hp["weight_decay"])
    step = decayed - ref_t
    alpha = hp["lr"] / (1 - hp["beta1"] ** t)
    denom = np.sqrt(ref_v / (1 - hp["beta2"] ** t)) + hp["eps"]
    bound = (2 * ulp32(np.maximum(np.abs(decayed), np.abs(ref_t))) + 8 * ulp32(step)
             + 1.01 * alpha * 3 * ulp32(big_m) / denom + 1e-45)
    assert np.all(np.abs(st.theta - ref_t) <= bound)
    # theta' is the model's BF16 weight: the new master weight rounded to nearest
    np.testing.assert_array_equal(st.tb, bf16_bits(st.theta))
    if t == 1:
        # closed form of the first bias-corrected step: lr * |g| / (|g| + eps)
        mv = np.abs(decayed - st.theta.astype(np.float64))
        expect = hp["lr"] * np.abs(gg) / (np.abs(gg) + hp["eps"])
        assert np.all(np.abs(mv - expect) <= 4 * ulp32(theta) + 1e-5 * hp["lr"])


def test_sgd_fp32_matches_torch_float64(orc):
    n = 32 * 200 + 3
    for t in (1, 2, 9):
        st, rng = random_state(orc, n, "sgd", seed=40 + t)
        if t == 1:
            st.m[:] = 0
        g = bf16_bits(rng.standard_normal(n) * 1e-2)
        theta, b = st.theta.astype(np.float64), st.m.astype(np.float64)
        orc.step_fp32(st, g, t, SGD)
        p = torch.tensor(theta, dtype=torch.float64, requires_grad=True)
        opt = torch.optim.SGD([p], lr=SGD["lr"], momentum=SGD["momentum"],
                              weight_decay=SGD["weight_decay"], foreach=False)
        p.grad = torch.tensor(bf16_f32(g).astype(np.float64))
        if t > 1:
            opt.state[p] = {"momentum_buffer": torch.tensor(b)}
        opt.step()
        ref_b = opt.state[p]["momentum_buffer"].numpy()
        ref_t = p.detach().numpy()
        gg = bf16_f32(g).astype(np.float64)
        big = np.maximum.reduce([np.abs(gg), np.abs(SGD["momentum"] * b), np.abs(ref_b)])
        assert np.all(np.abs(st.m - ref_b) <= 3 * ulp32(big) + 1e-45)
        step = theta - ref_t
        assert np.all(np.abs(st.theta - ref_t) <= 2 * ulp32(np.maximum(np.abs(theta), np.abs(
            ref_t))) + 4 * ulp32(step) + 1.01 * SGD["lr"] * 3 * ulp32(big) + 1e-45)
        np.testing.assert_array_equal(st.tb, bf16_bits(st.theta))


def test_lion_fp32_closed_forms(orc):
    """From zero momentum the first step moves every weight by exactly
    -lr*sign(g) after the decoupled decay (exact for theta in [0.5, 0.75) with
    lambda*theta rounded once), the momentum becomes RN((1-beta2)*g), and a
    zero gradient leaves only the decay."""
    n = 4096
    rng = np.random.default_rng(50)
    theta0 = rng.uniform(0.5, 0.75, n).astype(np.float32)
    st = orc.StateFP32(theta0, "lion")
    g = bf16_bits(rng.standard_normal(n) * 1e-3)
    g[:64] = 0
    gg = bf16_f32(g)
    orc.step_fp32(st, g, 1, LION)
    lam = np.float32(1.0 - LION["lr"] * LION["weight_decay"])
    decayed = (lam * theta0).astype(np.float32)
    sign = np.sign(gg).astype(np.float32)
    expect = (decayed - np.float32(LION["lr"]) * sign).astype(np.float32)
    np.testing.assert_array_equal(st.theta, expect)
    np.testing.assert_array_equal(st.theta[:64], decayed[:64])
    np.testing.assert_array_equal(st.m, (np.float32(1 - LION["beta2"]) * gg).astype(np.float32))
    np.testing.assert_array_equal(st.tb, bf16_bits(st.theta))
    # second step: the direction is sign(beta1*m + (1-beta1)*g) in float64 terms
    g2 = bf16_bits(-gg * rng.uniform(0.0, 3.0, n))
    m1 = st.m.astype(np.float64)
    th1 = st.theta.copy()
    orc.step_fp32(st, g2, 2, LION)
    c = LION["beta1"] * m1 + (1 - LION["beta1"]) * bf16_f32(g2).astype(np.float64)
    moved = (lam * th1).astype(np.float32) - st.theta
    clear = np.abs(c) > 1e-6 * np.abs(m1).max()
    np.testing.assert_array_equal(np.sign(moved[clear]), np.sign(c[clear]))


def test_fp32_adamw_trajectory_tracks_float64(orc):
    """40 steps: the FP32 master weight stays within the rounding of 40
    binary32 updates of AdamW in float64 fed the same gradients (there is no
    quantisation error), and the BF16 weight is always the master rounded."""
    n = 32 * 128
    rng = np.random.default_rng(60)
    theta0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    st = orc.StateFP32(theta0, "adamw")
    p = torch.tensor(theta0.astype(np.float64), requires_grad=True)
    opt = torch.optim.AdamW([p], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False)
    for t in range(1, 41):
        g = bf16_bits(rng.standard_normal(n) * 1e-3)
        orc.step_fp32(st, g, t, HP)
        p.grad = torch.tensor(bf16_f32(g).astype(np.float64))
        opt.step()
    ref = p.detach().numpy()
    moved = np.abs(ref - theta0.astype(np.float64))
    err = np.abs(st.theta - ref)
    assert np.median(moved) > 1e-3                   # the weights did move
    # at most ~2 roundings per step at the scale the weight has had
    path = np.maximum(np.abs(theta0), np.abs(ref)) + HP["lr"] * 40
    assert np.all(err <= 40 * ulp32(path))
    assert np.median(err / ulp32(path)) < 2
    np.testing.assert_array_equal(st.tb, bf16_bits(st.theta))


@pytest.mark.parametrize("optimizer,hp", [("adamw", HP), ("sgd", SGD), ("lion", LION)])
def test_fp32_and_compressed_steps_share_the_update(orc, optimizer, hp):
    """Fed the compressed state's rebuilt weight and dequantised moments, the
    FP32 step produces the compressed step's FP32 outputs bit for bit: the
    two differ only in what they store."""
    n = 32 * 100 + 11
    rng = np.random.default_rng(70)
    st = orc.State((rng.standard_normal(n) * 0.02).astype(np.float32), optimizer)
    for t in range(1, 4):
        orc.step(st, bf16_bits(rng.standard_normal(n) * 1e-3), t, hp)
    f = orc.StateFP32(orc.unsplit(st.tb, st.rho), optimizer)
    f.m[:] = orc.dequant_m(st.qm, st.sm)
    if optimizer == "adamw":
        f.v[:] = orc.dequant_v(st.qv, st.sv)
    g = bf16_bits(rng.standard_normal(n) * 1e-3)
    outs = orc.step(st, g, 4, hp, want_fp32=True)
    orc.step_fp32(f, g, 4, hp)
    np.testing.assert_array_equal(f.theta.view(np.uint32), outs[0].view(np.uint32))
    np.testing.assert_array_equal(f.m.view(np.uint32), outs[1].view(np.uint32))
    if optimizer == "adamw":
        np.testing.assert_array_equal(f.v.view(np.uint32), outs[2].view(np.uint32))


def _phi_inv(z):
    return z / (2.0 - np.abs(z))


def _adam_quotient(m, v, kappa, eps):
    return m / (kappa * np.sqrt(np.maximum(v, 0.0)) + eps)


@pytest.mark.parametrize("n", [64, 1024])
def test_compressed_trajectory_stays_near_fp32_adamw(orc, n):
    """The compressed AdamW run against the uncompressed one (pinned above to
    torch in float64), from the same weights and gradients, 10 steps.  The
    two share the update bit for bit (previous test), so they differ only by
    what the compressed state stores, and the deviation is bounded, element
    by element and step by step, by the quantisation errors the pinned bounds
    allow:

      m:  |m_hat - m_f| <= Bm(t) = b1 Bm(t-1) + Qm(t), with Qm the momentum
          dequantisation bound (companded error s/254, the bound pinned in
          test_oracle_quant, carried through phi_m^-1);
      v:  |v_hat - v_f| <= Bv(t) = b2 Bv(t-1) + Qv(t), Qv from the variance
          bound (error s/510 of sqrt(v));
      theta: |theta_hat - theta_f| <= B(t) = lambda B(t-1) + alpha_t du(t)
          + h/254 + rounding, where du(t) is the largest change of the Adam
          quotient m'/(kappa sqrt(v') + eps) over the box m' +- b1 Bm(t-1),
          v' +- b2 Bv(t-1) around the compressed run's values (the quotient is
          monotone in each, so its extremes are at the corners), and h/254 the
          split's bound (h = ULP(theta')/2).

    That is the sum over steps of lr-scaled quotient errors plus the split's
    h/254, with the companding bounds as the only source.  A few float32
    roundings per operation are added as slack; everything else is exact."""
    rng = np.random.default_rng(n)
    th0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    st = orc.State(th0, "adamw")
    f = orc.StateFP32(orc.unsplit(st.tb, st.rho), "adamw")
    b_theta = np.zeros(n)
    b_m = np.zeros(n)
    b_v = np.zeros(n)
    group = lambda a: np.repeat(a.view(np.float16).astype(np.float64), 32)[:n]
    for t in range(1, 11):
        g = bf16_bits(rng.standard_normal(n) * 1e-3)
        b1, c1, b2, c2, alpha, kappa, eps, lam = (float(x) for x in orc.adamw_scalars(
            HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], t))
        theta_n, m_new, v_new = (x.astype(np.float64) for x in orc.step(st, g, t, HP,
                                                                          want_fp32=True))
        orc.step_fp32(f, g, t, HP)
        # the update's inputs: m' and v' of the two runs differ by at most
        dm = b1 * b_m + 3 * ulp32(np.abs(m_new) + b1 * b_m)
        dv = b2 * b_v + 3 * ulp32(np.abs(v_new) + b2 * b_v)
        corners = [_adam_quotient(m_new + a * dm, v_new + b * dv, kappa, eps)
                   for a in (-1, 1) for b in (-1, 1)]
        u = _adam_quotient(m_new, v_new, kappa, eps)
        du = np.maximum(np.max(corners, axis=0) - u, u - np.min(corners, axis=0)) \
            + 6 * ulp32(np.abs(u) + 1e-30)
        e = (st.tb.astype(np.int64) >> 7) & 0xFF                # the new theta' exponent field
        h = 2.0 ** (np.maximum(e, 1) - 135)                     # ULP(theta')/2
        b_theta = lam * b_theta + alpha * du + h / 254 + 4 * ulp32(np.abs(theta_n) + b_theta)
        # the codes just written: dequantisation bounds around the stored values
        m_hat = orc.dequant_m(st.qm, st.sm).astype(np.float64)
        z_hat = 2 * m_hat / (1 + np.abs(m_hat))
        dz = group(st.sm) / 254 * 1.01 + 8 * ulp32(z_hat)
        assert np.all(np.abs(z_hat) + dz < 2)
        q_m = np.maximum(_phi_inv(z_hat + dz) - m_hat, m_hat - _phi_inv(z_hat - dz))
        v_hat = orc.dequant_v(st.qv, st.sv).astype(np.float64)
        w_hat = np.sqrt(v_hat)
        dw = group(st.sv) / 510 * 1.01 + 8 * ulp32(w_hat)
        q_v = np.maximum((w_hat + dw) ** 2 - v_hat, v_hat - np.maximum(w_hat - dw, 0) ** 2) \
            + ulp32(v_hat)
        b_m = dm + q_m
        b_v = dv + q_v
        assert np.all(np.abs(m_hat - f.m) <= b_m), t
        assert np.all(np.abs(v_hat - f.v) <= b_v), t
        dev = np.abs(orc.unsplit(st.tb, st.rho).astype(np.float64) - f.theta)
        assert np.all(dev <= b_theta), (t, float((dev / b_theta).max()))
        # not vacuous: the bound stays a few percent of the distance moved
        moved = np.abs(f.theta - th0.astype(np.float64))
        assert np.median(b_theta / np.maximum(moved, 1e-12)) < 0.1, t
        assert np.median(dev / np.maximum(moved, 1e-12)) < 0.02