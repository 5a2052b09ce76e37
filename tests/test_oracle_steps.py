"""Oracle pins: the fused step (FlashOptim digest, "Core method > Fused
optimizer step", Alg. 4: dequantise, rebuild the master weight, standard
AdamW update, requantise, re-split; SGD with momentum is the other optimizer
the background section names).

The update itself is pinned against torch.optim.AdamW / torch.optim.SGD run
in float64 from the same dequantised state; the fused requantise / re-split
is pinned against the separately tested codec functions applied to the
step's fp32 outputs.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
SGD = dict(lr=0.1, momentum=0.9, weight_decay=1e-4)


def ulp32(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


def bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bf16_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def warm_state(orc, n, steps, seed, optimizer="adamw", hp=HP, gscale=1e-3):
    rng = np.random.default_rng(seed)
    st = orc.State((rng.standard_normal(n) * 0.02).astype(np.float32), optimizer)
    for t in range(1, steps + 1):
        g = bf16_bits(rng.standard_normal(n) * gscale)
        orc.step(st, g, t, hp)
    return st, rng


@pytest.mark.parametrize("t,hp", [
    (1, HP), (2, HP), (11, HP), (1000, HP),
    (5, dict(lr=3e-2, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1)),
    (7, dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)),
])
def test_adamw_update_matches_torch_float64(orc, t, hp):
    n = 32 * 512 + 19
    st, rng = warm_state(orc, n, t - 1, seed=t, hp=hp)
    g = bf16_bits(rng.standard_normal(n) * 1e-3)
    theta_hat = orc.unsplit(st.tb, st.rho).astype(np.float64)
    m = orc.dequant_m(st.qm, st.sm).astype(np.float64)
    v = orc.dequant_v(st.qv, st.sv).astype(np.float64)
    theta_n, m_n, v_n = orc.adamw_step(st, g, t, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                       hp["weight_decay"], want_fp32=True)

    p = torch.tensor(theta_hat, dtype=torch.float64, requires_grad=True)
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
    assert np.all(np.abs(m_n - ref_m) <= 3 * ulp32(big_m) + 1e-45)
    big_v = np.maximum(hp["beta2"] * v, ref_v)
    assert np.all(np.abs(v_n - ref_v) <= 4 * ulp32(big_v) + 1e-45)
    decayed = theta_hat * (1 - hp["lr"] * hp["weight_decay"])
    step = decayed - ref_t
    err = np.abs(theta_n - ref_t)
    # propagated bound: roundings of the decay and of the result, the step's
    # own relative error, and the absolute error of m' (which can cancel)
    # carried through alpha / (sqrt(v_hat) + eps)
    alpha = hp["lr"] / (1 - hp["beta1"] ** t)
    denom = np.sqrt(ref_v / (1 - hp["beta2"] ** t)) + hp["eps"]
    m_abs = 3 * ulp32(big_m)
    assert np.all(err <= 2 * ulp32(np.maximum(np.abs(decayed), np.abs(ref_t)))
                  + 8 * ulp32(step) + 1.01 * alpha * m_abs / denom + 1e-45)
    # the update is not a no-op: the step term is resolved, not lost in rounding
    assert np.median(np.abs(step)) > 100 * np.median(ulp32(ref_t)) * 1e-3


def test_fused_requant_equals_codec_composition(orc):
    n = 32 * 777 + 5
    st, rng = warm_state(orc, n, 4, seed=21)
    g = bf16_bits(rng.standard_normal(n) * 1e-3)
    theta_n, m_n, v_n = orc.adamw_step(st, g, 5, **{k: HP[k] for k in HP}, want_fp32=True)
    qm, sm = orc.quant_m(m_n)
    qv, sv = orc.quant_v(v_n)
    tb, rho = orc.split(theta_n)
    for a, b in ((st.qm, qm), (st.sm, sm), (st.qv, qv), (st.sv, sv), (st.tb, tb),
                 (st.rho, rho)):
        np.testing.assert_array_equal(a, b)


def test_sgd_update_matches_torch_float64(orc):
    n = 32 * 300 + 9
    for t in (1, 2, 6):
        st, rng = warm_state(orc, n, t - 1, seed=30 + t, optimizer="sgd", hp=SGD, gscale=1e-2)
        g = bf16_bits(rng.standard_normal(n) * 1e-2)
        theta_hat = orc.unsplit(st.tb, st.rho).astype(np.float64)
        b = orc.dequant_m(st.qm, st.sm).astype(np.float64)
        theta_n, b_n = orc.sgd_step(st, g, t, SGD["lr"], SGD["momentum"], SGD["weight_decay"],
                                    want_fp32=True)
        p = torch.tensor(theta_hat, dtype=torch.float64, requires_grad=True)
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
        assert np.all(np.abs(b_n - ref_b) <= 3 * ulp32(big) + 1e-45)
        step = theta_hat - ref_t
        # plus the absolute error of b' (which can cancel) scaled by lr
        assert np.all(np.abs(theta_n - ref_t) <= 2 * ulp32(np.maximum(np.abs(theta_hat), np.abs(
            ref_t))) + 4 * ulp32(step) + 1.01 * SGD["lr"] * 3 * ulp32(big) + 1e-45)
        qm, sm = orc.quant_m(b_n)
        tb, rho = orc.split(theta_n)
        np.testing.assert_array_equal(st.qm, qm)
        np.testing.assert_array_equal(st.sm, sm)
        np.testing.assert_array_equal(st.tb, tb)
        np.testing.assert_array_equal(st.rho, rho)


def test_host_scalars_exact(orc):
    for t in (1, 2, 10, 1000):
        lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
        sc = orc.adamw_scalars(lr, b1, b2, eps, wd, t)
        p1 = Fraction(b1) ** t
        p2 = Fraction(b2) ** t
        alpha = float(Fraction(lr) / (1 - p1))
        kappa = 1.0 / math.sqrt(float(1 - p2))
        assert sc[0] == np.float32(b1) and sc[2] == np.float32(b2)
        assert sc[1] == np.float32(1 - b1) and sc[3] == np.float32(1 - b2)
        assert abs(float(sc[4]) - alpha) <= ulp32(alpha)
        assert abs(float(sc[5]) - kappa) <= ulp32(kappa)
        assert sc[6] == np.float32(eps) and sc[7] == np.float32(1 - lr * wd)


def test_adamw_zero_betas_is_state_independent(orc):
    hp = dict(HP, beta1=0.0, beta2=0.0)
    n = 32 * 64
    a, rng = warm_state(orc, n, 3, seed=40)
    b = a.copy()
    b.qm[:] = np.random.default_rng(1).integers(-127, 128, n).astype(np.int8)
    b.qv[:] = np.random.default_rng(2).integers(0, 256, n).astype(np.uint8)
    b.sm[:] = 0x2000
    b.sv[:] = 0x1800
    g = bf16_bits(rng.standard_normal(n) * 1e-3)
    ta = orc.step(a, g, 4, hp, want_fp32=True)
    tbv = orc.step(b, g, 4, hp, want_fp32=True)
    np.testing.assert_array_equal(ta[0], tbv[0])
    np.testing.assert_array_equal(a.tb, b.tb)
    np.testing.assert_array_equal(a.qm, b.qm)


def test_adamw_zero_grad_first_step_is_pure_decay(orc):
    rng = np.random.default_rng(41)
    theta = (rng.standard_normal(32 * 10 + 3) * 0.02).astype(np.float32)
    st = orc.State(theta)
    theta_hat = orc.unsplit(st.tb, st.rho)
    lam = np.float32(1 - HP["lr"] * HP["weight_decay"])
    out = orc.step(st, np.zeros(theta.size, np.uint16), 1, HP, want_fp32=True)
    np.testing.assert_array_equal(out[0], lam * theta_hat)
    assert not st.qm.any() and not st.qv.any() and not st.sm.any() and not st.sv.any()


def test_sgd_zero_momentum_closed_form(orc):
    hp = dict(SGD, momentum=0.0)
    n = 32 * 33 + 1
    st, rng = warm_state(orc, n, 2, seed=42, optimizer="sgd", hp=SGD, gscale=1e-2)
    theta_hat = orc.unsplit(st.tb, st.rho)
    g = bf16_bits(rng.standard_normal(n) * 1e-2)
    out = orc.step(st, g, 3, hp, want_fp32=True)
    eta, omega = np.float32(hp["lr"]), np.float32(hp["weight_decay"])
    expect = theta_hat - eta * (bf16_f32(g) + omega * theta_hat)     # numpy float32 ops
    np.testing.assert_array_equal(out[0], expect)


def test_chunked_threads_and_resume_are_identical(orc):
    n = 32 * 5000 + 17
    a, rng = warm_state(orc, n, 0, seed=50)
    b = a.copy()
    grads = [bf16_bits(rng.standard_normal(n) * 1e-3) for _ in range(6)]
    for t, g in enumerate(grads, 1):
        orc.step(a, g, t, HP)
        orc.step_chunked(b, g, t, HP, nthreads=7)
        if t == 3:
            b = b.copy()          # "checkpoint": codes + scales + t are the whole state
    for k in ("tb", "rho", "qm", "sm", "qv", "sv"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))


def test_groups_restart_per_tensor(orc):
    rng = np.random.default_rng(60)
    x1 = (rng.standard_normal(40) * 0.02).astype(np.float32)
    x2 = (rng.standard_normal(50) * 0.5).astype(np.float32)
    g = bf16_bits(rng.standard_normal(90) * 1e-3)
    s1, s2, cat = orc.State(x1), orc.State(x2), orc.State(np.concatenate([x1, x2]))
    orc.step(s1, g[:40], 1, HP)
    orc.step(s2, g[40:], 1, HP)
    orc.step(cat, g, 1, HP)
    assert s1.sm.size + s2.sm.size == 4 and cat.sm.size == 3
    np.testing.assert_array_equal(cat.qm[:32], s1.qm[:32])        # first whole group agrees
    assert not np.array_equal(cat.qm[40:], s2.qm)                 # straddling groups differ


def test_tracks_uncompressed_adamw(orc):
    """Quality check of the compressed trajectory against float64 AdamW with
    uncompressed state (same gradients, config-1 hyper-parameters, 10 steps):
    the weight movement agrees to within the 8-bit state quantisation."""
    n = 32 * 256
    rng = np.random.default_rng(70)
    theta0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    st = orc.State(theta0)
    p = torch.tensor(theta0.astype(np.float64), requires_grad=True)
    opt = torch.optim.AdamW([p], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False)
    for t in range(1, 11):
        g = bf16_bits(rng.standard_normal(n) * 1e-3)
        orc.step(st, g, t, HP)
        p.grad = torch.tensor(bf16_f32(g).astype(np.float64))
        opt.step()
    flash = orc.unsplit(st.tb, st.rho).astype(np.float64) - theta0
    ref = p.detach().numpy() - theta0
    rel = np.linalg.norm(flash - ref) / np.linalg.norm(ref)
    assert rel < 0.05, rel
    assert np.corrcoef(flash, ref)[0, 1] > 0.998
