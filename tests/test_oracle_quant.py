"""Oracle pins: companding and group quantisation (FlashOptim digest, "Core
method > Optimizer-state quantisation with companding", Alg. 2-3).

phi_m(x) = 2x/(1+|x|) with inverse z/(2-|z|); phi_v(x) = sqrt(x) with inverse
z^2; groups of 32 elements, one FP16 scale each; momentum INT8, variance
UINT8; companding first, then group scaling and integer quantisation.
References here are the formulas evaluated in float64 and numpy's own
float32 sqrt / float16 cast.
"""
import numpy as np
import pytest

GROUP = 32


def ulp32(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


def test_phi_m_closed_forms(orc):
    x = np.array([0.0, -0.0, 1.0, -1.0, 3.0, -3.0, 1e30, -1e30, 2.0 ** 25], np.float32)
    z = orc.phi_m(x)
    assert z[0] == 0 and z[2] == 1.0 and z[3] == -1.0
    assert z[4] == 1.5 and z[5] == -1.5              # 6/4 exactly
    assert z[6] == 2.0 and z[7] == -2.0 and z[8] == 2.0   # saturates at the range edge


def test_phi_m_against_float64_formula(orc):
    rng = np.random.default_rng(10)
    x = np.concatenate([rng.standard_normal(1 << 18) * s for s in (1e-6, 1e-3, 1.0, 1e3)])
    x = x.astype(np.float32)
    z = orc.phi_m(x)
    x64 = x.astype(np.float64)
    ref = 2 * x64 / (1 + np.abs(x64))
    # RN(1+|x|) is off by <= 2^-24 relative, the quotient by <= 1/2 ulp: 1.5 ulp
    assert np.all(np.abs(z - ref) <= 1.5 * ulp32(ref))
    np.testing.assert_array_equal(orc.phi_m(-x), -z)             # odd
    # the exact function increases; the binary32 evaluation can step back by
    # its rounding where RN(1+|x|) jumps, never by more
    order = np.argsort(x, kind="stable")
    zs = z[order]
    assert np.all(np.diff(zs.astype(np.float64)) >= -3 * ulp32(zs[1:]))
    assert np.all(np.abs(z) <= 2.0)


def test_phi_m_inverse_against_float64_formula(orc):
    rng = np.random.default_rng(11)
    z = rng.uniform(-1.999, 1.999, 1 << 20).astype(np.float32)
    m = orc.phi_m_inv(z)
    z64 = z.astype(np.float64)
    ref = z64 / (2 - np.abs(z64))
    assert np.all(np.abs(m - ref) <= 1.5 * ulp32(ref) + 1e-45)
    assert orc.phi_m_inv(np.array([1.0, -1.0, 0.0], np.float32)).tolist() == [1.0, -1.0, 0.0]


def test_phi_m_roundtrip_conditioning(orc):
    # phi_m^-1 has slope 2/(2-|z|)^2 = (1+|x|)^2/2: the round trip error grows
    # with |x| like (1+|x|) ulp
    rng = np.random.default_rng(12)
    for hi, max_ulps in ((1.0, 3), (10.0, 16), (100.0, 128)):
        x = rng.uniform(-hi, hi, 1 << 18).astype(np.float32)
        back = orc.phi_m_inv(orc.phi_m(x))
        err_ulps = np.abs(back.astype(np.float64) - x) / ulp32(x)
        assert err_ulps.max() <= max_ulps


def test_phi_v_against_numpy(orc):
    rng = np.random.default_rng(13)
    v = np.abs(rng.standard_normal(1 << 20) * 1e-6).astype(np.float32) ** 2
    v = np.concatenate([v, np.array([0.0, 1.0, 4.0, 2.0 ** -149, 3e38], np.float32)])
    np.testing.assert_array_equal(orc.phi_v(v), np.sqrt(v))            # IEEE sqrt
    z = np.sqrt(v)
    np.testing.assert_array_equal(orc.phi_v_inv(z), z * z)
    back = orc.phi_v_inv(orc.phi_v(v))
    normal = v >= np.finfo(np.float32).tiny
    assert np.all(np.abs(back[normal].astype(np.float64) - v[normal]) <= ulp32(v[normal]))


def _f16(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16)


def _groups(a):
    n = a.size
    pad = (-n) % GROUP
    return np.concatenate([a, np.zeros(pad, a.dtype)]).reshape(-1, GROUP), n


@pytest.mark.parametrize("scale", [1e-7, 1e-5, 1e-3, 0.1, 1.0, 30.0])
def test_quant_m_against_float64_definition(orc, scale):
    rng = np.random.default_rng(int(scale * 1e7) % 1000)
    n = 32 * 4096 + 13                                  # ragged last group
    m = (rng.standard_t(3, n) * scale).astype(np.float32)
    q, s = orc.quant_m(m)
    assert q.dtype == np.int8 and s.size == (n + 31) // 32
    assert q.min() >= -127
    # scale: FP16 of the group's largest |phi_m|, capped at 0x3FFF
    z64 = 2 * m.astype(np.float64) / (1 + np.abs(m.astype(np.float64)))
    zg, _ = _groups(np.abs(z64))
    amax = zg.max(axis=1)
    s_ref = np.minimum(_f16(amax).view(np.uint16), 0x3FFF)
    diff = np.abs(s.astype(np.int32) - s_ref.astype(np.int32))
    assert diff.max() <= 1 and (diff == 0).mean() > 0.999
    # codes: rne(z * 127 / s); exact except where z*127/s lies within rounding of .5
    sv = _f16(0).astype(np.float64) + s.view(np.float16).astype(np.float64)
    sg = np.repeat(sv, GROUP)[:n]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(sg > 0, z64 * 127.0 / sg, 0.0)
    q_ref = np.clip(np.rint(y), -127, 127)
    near_half = np.abs(np.abs(y - np.trunc(y)) - 0.5) < 1e-4
    bad = (q != q_ref) & ~near_half
    assert not bad.any()
    assert np.all(np.abs(q - q_ref) <= 1)


def test_quant_m_zero_tiny_and_saturated_groups(orc):
    m = np.zeros(96, np.float32)
    m[32:64] = 1e-9                                     # |phi_m| ~ 2e-9 < 2^-25: scale rounds to 0
    m[64:96] = np.float32(1e9) * np.sign(np.arange(32) - 15.5)   # phi_m -> 2: scale capped
    q, s = orc.quant_m(m)
    assert s[0] == 0 and s[1] == 0 and not q[:64].any()
    assert s[2] == 0x3FFF
    assert set(np.abs(q[64:]).tolist()) == {127}
    back = orc.dequant_m(q, s)
    assert np.all(np.isfinite(back))                    # 2 - |z| stays positive


def test_quant_groups_restart_and_tail_is_valid_only(orc):
    rng = np.random.default_rng(14)
    m = (rng.standard_normal(80) * 1e-3).astype(np.float32)
    longer = np.concatenate([m, np.full(16, 5.0, np.float32)])   # huge values past n
    q1, s1 = orc.quant_m(m)
    q2, s2 = orc.quant_m(longer)
    np.testing.assert_array_equal(q1[:64], q2[:64])
    np.testing.assert_array_equal(s1[:2], s2[:2])
    assert s1[2] != s2[2]                               # group 2 differs only via elements >= 80
    # chunks of whole groups quantise independently
    qa, sa = orc.quant_m(m[:64])
    qb, sb = orc.quant_m(m[64:])
    np.testing.assert_array_equal(np.concatenate([qa, qb]), q1)
    np.testing.assert_array_equal(np.concatenate([sa, sb]), s1)


@pytest.mark.parametrize("scale", [1e-4, 1e-2, 1.0])
def test_dequant_m_error_bound(orc, scale):
    rng = np.random.default_rng(15)
    m = (rng.standard_normal(32 * 2048) * scale).astype(np.float32)
    q, s = orc.quant_m(m)
    back = orc.dequant_m(q, s).astype(np.float64)
    z = 2 * m / (1 + np.abs(m.astype(np.float64)))
    zb = 2 * back / (1 + np.abs(back))
    sg = np.repeat(s.view(np.float16).astype(np.float64), GROUP)
    # companded-domain error: half a code step, s/254, plus the scale's
    # rounding below the group max (codes clamp) and float32 roundings
    assert np.all(np.abs(z - zb) <= sg / 254 * 1.01 + 4 * ulp32(z) + 1e-12)


def test_quant_idempotent_on_normal_scales(orc):
    rng = np.random.default_rng(16)
    m = (rng.standard_t(3, 32 * 8192) * 1e-3).astype(np.float32)
    q, s = orc.quant_m(m)
    q2, s2 = orc.quant_m(orc.dequant_m(q, s))
    normal = s >= 0x0400                                # fp16 normal scales
    gq = np.repeat(normal, GROUP)
    np.testing.assert_array_equal(s2[normal], s[normal])
    np.testing.assert_array_equal(q2[gq], q[gq])
    v = (rng.standard_t(3, 32 * 8192) * 1e-3).astype(np.float32) ** 2
    qv, sv = orc.quant_v(v)
    qv2, sv2 = orc.quant_v(orc.dequant_v(qv, sv))
    normal = sv >= 0x0400
    np.testing.assert_array_equal(sv2[normal], sv[normal])
    np.testing.assert_array_equal(qv2[np.repeat(normal, GROUP)], qv[np.repeat(normal, GROUP)])


@pytest.mark.parametrize("scale", [1e-5, 1e-3, 1.0])
def test_quant_v_against_float64_definition(orc, scale):
    rng = np.random.default_rng(17)
    n = 32 * 4096 + 7
    v = ((rng.standard_t(3, n) * scale) ** 2).astype(np.float32)
    q, s = orc.quant_v(v)
    assert q.dtype == np.uint8 and s.size == (n + 31) // 32
    w = np.sqrt(v)                                      # numpy float32 sqrt: IEEE
    wg, _ = _groups(w)
    s_ref = np.minimum(_f16(wg.max(axis=1)).view(np.uint16), 0x7BFF)
    np.testing.assert_array_equal(s, s_ref)
    sg = np.repeat(s.view(np.float16).astype(np.float64), GROUP)[:n]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(sg > 0, w.astype(np.float64) * 255.0 / sg, 0.0)
    q_ref = np.clip(np.rint(y), 0, 255)
    near_half = np.abs(np.abs(y - np.trunc(y)) - 0.5) < 1e-4
    assert not ((q != q_ref) & ~near_half).any()
    back = orc.dequant_v(q, s).astype(np.float64)
    wb = np.sqrt(back)
    assert np.all(np.abs(wb - w) <= sg / 510 * 1.01 + 4 * ulp32(w) + 1e-30)


def test_quant_v_saturates(orc):
    v = np.full(32, 1e12, np.float32)                   # sqrt = 1e6 > 65504
    q, s = orc.quant_v(v)
    assert s[0] == 0x7BFF and np.all(q == 255)
