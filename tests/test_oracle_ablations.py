"""Oracle pins for the codec ablations of the FlashOptim page ("Core method >
Weight splitting", Fig. 3: BF16 versus FP16 base weights and the width of
the correction; "Optimizer-state quantisation with companding", Fig. 4-5:
linear group quantisation without companding).

The FP16-base split is pinned against its definition in float64 with numpy's
float16 cast for theta' and ULP(theta') taken as the gap to the next FP16
value; the linear quantisers against the group-scale definition.  The last
tests pin the mechanisms the figures show: more correction bits shrink the
rebuild error, the FP16 base's extra mantissa bits make an 8-bit correction
about 8 times more accurate than on BF16 where both are in range, and
without companding the variance of small-gradient groups falls below the
FP16 scale's reach and is stored as zero.
"""
import numpy as np
import pytest

GROUP = 32


def f16_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f16_value(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def half_ulp_f16_by_successor(hb):
    mag = (np.asarray(hb, np.uint16) & 0x7FFF).astype(np.uint32)
    here = f16_value(mag.astype(np.uint16))
    nxt = f16_value(np.minimum(mag + 1, 0x7BFF).astype(np.uint16))
    gap = np.where(mag == 0x7BFF, 32.0, nxt - here)      # the successor of 65504 is Inf
    return gap / 2.0


def ref_split_f16(x, qmax):
    x = np.asarray(x, np.float32)
    hb = f16_bits(x)
    t = f16_value(hb)
    fin = np.isfinite(t)
    h = half_ulp_f16_by_successor(hb)
    with np.errstate(invalid="ignore"):
        e = (x.astype(np.float64) - t) / h               # exact
        rho = np.clip(np.rint(e * qmax), -qmax, qmax)    # e * qmax is exact in float64
    rho = np.where(fin, rho, 0).astype(np.int32)
    return hb, rho, e


def binade(exp_field, sign=0):
    m = np.arange(1 << 23, dtype=np.uint32)
    return ((np.uint32(sign) << 31) | (np.uint32(exp_field) << 23) | m).view(np.float32)


@pytest.mark.parametrize("qmax", [7, 127, 2047])
@pytest.mark.parametrize("exp_field", [100, 113, 127, 142])
def test_split_f16_matches_definition(orc, qmax, exp_field):
    # exponent fields: inside FP16's subnormal range (100), its smallest normal
    # binade (113), 1.0 (127), the largest binade (142 -> Inf past 65520)
    x = binade(exp_field, exp_field % 2)
    hb, rho = orc.split_f16_q(x, qmax)
    rhb, rrho, e = ref_split_f16(x, qmax)
    np.testing.assert_array_equal(hb, rhb)
    np.testing.assert_array_equal(rho, rrho)
    fin = np.isfinite(f16_value(hb))
    assert np.all(np.abs(e[fin]) <= 1.0)


def test_split_f16_specials(orc):
    x = np.array([0.0, -0.0, 65504.0, -65504.0, 65519.99, 65520.0, np.inf, -np.inf,
                  2.0 ** -24, 2.0 ** -25, 2.0 ** -26, 1.4e-45, 1.0], np.float32)
    hb, rho = orc.split_f16_q(x, 127)
    rhb, rrho, _ = ref_split_f16(x, 127)
    np.testing.assert_array_equal(hb, rhb)
    np.testing.assert_array_equal(rho, rrho)
    assert hb[5] == 0x7C00 and rho[5] == 0               # rounds to Inf: no correction


@pytest.mark.parametrize("qmax", [127, 2047])
def test_split_f16_roundtrip_bound(orc, qmax):
    rng = np.random.default_rng(20)
    x = (rng.standard_normal(1 << 20) * 0.02).astype(np.float32)
    hb, rho = orc.split_f16_q(x, qmax)
    y = orc.unsplit_f16_q(hb, rho, qmax).astype(np.float64)
    h = half_ulp_f16_by_successor(hb)
    bound = h / (2 * qmax) * (1 + 2.0 ** -20) + np.spacing(np.abs(x)).astype(np.float64)
    assert np.all(np.abs(y - x) <= bound)


def test_correction_bits_and_base_format(orc):
    """Fig. 3's ordering: error falls with the correction width; on weights
    that FP16 represents as normals, an 8-bit correction on an FP16 base is
    about 2^3 times more accurate than on a BF16 base (three more mantissa
    bits), and BF16 + 16 bits is exact to a few parts in 10^10."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(1 << 20) * 0.02).astype(np.float32)
    x = x[np.abs(x) > 2.0 ** -13]                        # FP16 normal range
    x64 = x.astype(np.float64)

    def rel(y):
        return np.abs(y.astype(np.float64) - x64) / np.abs(x64)

    bf = {}
    for q in (7, 127, 32767):
        tb, rho = orc.split_q(x, q)
        bf[q] = rel(orc.unsplit_q(tb, rho, q)).mean()
    hb, rho = orc.split_f16_q(x, 127)
    f16_8 = rel(orc.unsplit_f16_q(hb, rho, 127)).mean()
    assert bf[7] > 10 * bf[127] > 100 * bf[32767]
    assert bf[32767] < 1e-9
    assert 5 < bf[127] / f16_8 < 12


def _group_scale_ref(z, cap):
    n = z.size
    pad = (-n) % GROUP
    zg = np.concatenate([np.abs(z), np.zeros(pad)]).reshape(-1, GROUP)
    with np.errstate(over="ignore"):
        s = zg.max(axis=1).astype(np.float32).astype(np.float16).view(np.uint16)
    return np.minimum(s, cap)


@pytest.mark.parametrize("scale", [1e-6, 1e-3, 1.0, 1e4])
def test_linear_quant_m_against_definition(orc, scale):
    rng = np.random.default_rng(int(scale * 1e6) % 997)
    n = 32 * 2048 + 5
    m = (rng.standard_t(3, n) * scale).astype(np.float32)
    q, s = orc.quant_lin_m(m)
    np.testing.assert_array_equal(s, _group_scale_ref(m.astype(np.float64), 0x7BFF))
    sg = np.repeat(s.view(np.float16).astype(np.float64), GROUP)[:n]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(sg > 0, m.astype(np.float64) * 127.0 / sg, 0.0)
    q_ref = np.clip(np.rint(y), -127, 127)
    near_half = np.abs(np.abs(y - np.trunc(y)) - 0.5) < 1e-4
    assert not ((q != q_ref) & ~near_half).any()
    back = orc.dequant_lin_m(q, s).astype(np.float64)
    np.testing.assert_allclose(back, q * (sg * np.float32(1 / 127)), rtol=2.0 ** -22, atol=1e-45)


@pytest.mark.parametrize("scale", [1e-8, 1e-4, 1.0])
def test_linear_quant_v_against_definition(orc, scale):
    rng = np.random.default_rng(int(scale * 1e8) % 991)
    n = 32 * 2048 + 9
    v = ((rng.standard_normal(n) * scale) ** 2).astype(np.float32)
    q, s = orc.quant_lin_v(v)
    np.testing.assert_array_equal(s, _group_scale_ref(v.astype(np.float64), 0x7BFF))
    sg = np.repeat(s.view(np.float16).astype(np.float64), GROUP)[:n]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(sg > 0, v.astype(np.float64) * 255.0 / sg, 0.0)
    q_ref = np.clip(np.rint(y), 0, 255)
    near_half = np.abs(np.abs(y - np.trunc(y)) - 0.5) < 1e-4
    assert not ((q != q_ref) & ~near_half).any()


def test_without_companding_small_variances_vanish(orc):
    """Fig. 5's failure mechanism: variances of small gradients (v ~ 1e-10)
    sit below the smallest FP16 scale, so the linear quantiser stores the
    whole group as 0 (the step then divides by eps alone); sqrt companding
    keeps them (sqrt(1e-10) = 1e-5 is an FP16 subnormal)."""
    rng = np.random.default_rng(22)
    v = ((rng.standard_normal(32 * 64) * 1e-5) ** 2).astype(np.float32)
    q, s = orc.quant_lin_v(v)
    assert not s.any() and not q.any()
    assert not orc.dequant_lin_v(q, s).any()
    qc, sc = orc.quant_v(v)
    assert sc.all()
    back = orc.dequant_v(qc, sc).astype(np.float64)
    nmse = ((back - v) ** 2).sum() / (v.astype(np.float64) ** 2).sum()
    assert nmse < 0.05


def test_companding_shrinks_the_variance_error_tail(orc):
    """Fig. 4: within groups whose gradient scale varies (log-normal, sigma
    0.5), linear codes send one variance in seven to 0 while sqrt companding
    keeps all but one in a hundred; the error tail and the NMSE both shrink."""
    rng = np.random.default_rng(23)
    g = rng.standard_normal(32 * 4096) * np.exp(rng.standard_normal(32 * 4096) * 0.5) * 1e-3
    v = (g * g).astype(np.float32)
    ql, sl = orc.quant_lin_v(v)
    qc, sc = orc.quant_v(v)
    v64 = v.astype(np.float64)
    ok = v64 > 0
    bl = orc.dequant_lin_v(ql, sl).astype(np.float64)
    bc = orc.dequant_v(qc, sc).astype(np.float64)
    rl = np.abs(bl - v64)[ok] / v64[ok]
    rc = np.abs(bc - v64)[ok] / v64[ok]
    assert np.quantile(rc, 0.9) * 4 < np.quantile(rl, 0.9)
    assert (rl >= 1.0).mean() > 5 * (rc >= 1.0).mean()
    nmse_l = ((bl - v64) ** 2).sum() / (v64 ** 2).sum()
    nmse_c = ((bc - v64) ** 2).sum() / (v64 ** 2).sum()
    assert nmse_l > 3 * nmse_c


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _bf16_bits(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _warm(orc, kind, n, steps, seed, gscale=1e-3):
    rng = np.random.default_rng(seed)
    st = orc.State((rng.standard_normal(n) * 0.02).astype(np.float32), kind)
    for t in range(1, steps + 1):
        orc.step(st, _bf16_bits(rng.standard_normal(n) * gscale), t, HP)
    return st, rng


def test_linear_variance_step_is_the_codec_composition(orc):
    """The Fig. 5 ablation step (variance without companding): its codes are
    the linear quantiser of its FP32 v', the method's quantiser of m', and
    the split of theta_n; its update equals the pinned FP32 step fed the
    same rebuilt weight and dequantised moments."""
    n = 32 * 300 + 13
    st, rng = _warm(orc, "adamw_linv", n, 3, seed=24)
    f = orc.StateFP32(orc.unsplit(st.tb, st.rho), "adamw")
    f.m[:] = orc.dequant_m(st.qm, st.sm)
    f.v[:] = orc.dequant_lin_v(st.qv, st.sv)
    g = _bf16_bits(rng.standard_normal(n) * 1e-3)
    th, m, v = orc.step(st, g, 4, HP, want_fp32=True)
    orc.step_fp32(f, g, 4, HP)
    for a, b in ((th, f.theta), (m, f.m), (v, f.v)):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    qv, sv = orc.quant_lin_v(v)
    qm, sm = orc.quant_m(m)
    tb, rho = orc.split(th)
    for a, b in ((st.qv, qv), (st.sv, sv), (st.qm, qm), (st.sm, sm), (st.tb, tb), (st.rho, rho)):
        np.testing.assert_array_equal(a, b)


def test_linear_variance_sends_small_variances_to_zero_and_steps_explode(orc):
    """Fig. 5's failure: in groups where four elements see gradients 30 times
    larger than the other 28, the linear codes store the quiet elements'
    variance (900 times smaller) as 0 while their momentum survives; on a
    step where those gradients are 0 the update is alpha*m'/eps, thousands
    of times lr.  With square-root companding the variance survives and the
    step stays below ~lr."""
    n = 32 * 256
    rng = np.random.default_rng(25)
    scale = np.where(np.arange(n) % 32 < 4, 1e-2, 1e-2 / 30)
    quiet = scale < 1e-2
    steps = {}
    for kind in ("adamw", "adamw_linv"):
        st = orc.State((rng.standard_normal(n) * 0.02).astype(np.float32), kind)
        r = np.random.default_rng(26)
        for t in range(1, 10):
            orc.step(st, _bf16_bits(r.standard_normal(n) * scale), t, HP)
        v = (orc.dequant_lin_v if kind == "adamw_linv" else orc.dequant_v)(st.qv, st.sv)
        lost = (v[quiet] == 0).mean()
        assert (lost > 0.9) if kind == "adamw_linv" else (lost == 0)
        assert (orc.dequant_m(st.qm, st.sm)[quiet] != 0).mean() > 0.8   # momentum kept
        before = orc.unsplit(st.tb, st.rho).astype(np.float64)
        g = r.standard_normal(n) * scale
        g[quiet] = 0.0
        orc.step(st, _bf16_bits(g), 10, HP)
        steps[kind] = np.abs(orc.unsplit(st.tb, st.rho).astype(np.float64) - before)[quiet]
    assert np.quantile(steps["adamw"], 0.99) < 2 * HP["lr"]
    assert np.median(steps["adamw_linv"]) > 1000 * HP["lr"]
