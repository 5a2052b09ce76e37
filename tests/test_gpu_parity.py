"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle,
bit for bit on every BF16 / INT8 / UINT8 code and FP16 scale, and on the
rebuilt FP32 weights.  Sizes span several 2048-element tiles and ragged tails;
the five workloads run at full size, the large ones compared on sampled groups
in the same launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import oracle
from compressed_adamw_state_amd import flashopt as F
from compressed_adamw_state_amd import workloads as W

from parity import Run, i8, log, state_fields, u16, u8

pytestmark = pytest.mark.gpu

RAGGED = [1, 31, 32, 33, 511, 512, 513, 1000, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 4097, 6143, 32 * 777 + 5,
          (1 << 20) + 7, 0, 64]


def dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).cuda()


def special_floats(rng, n):
    """Normal weights plus zeros, subnormals, bf16 ties, huge and tiny values."""
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    bits = x.view(np.uint32)
    k = n // 16
    bits[:k] = (bits[:k] & 0xFFFF0000) | 0x8000                       # exact bf16 ties
    bits[k:2 * k] = rng.integers(1, 1 << 23, k).astype(np.uint32)     # fp32 subnormals
    bits[2 * k:3 * k] = 0
    extremes = np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F7FFF, 0x00800000, 0x80000001,
                         0x3F800000, 0xBF800000, 0x7F000000], np.uint32)
    room = min(extremes.size, n - 3 * k)
    bits[3 * k:3 * k + room] = extremes[:room]
    return bits.view(np.float32)


@pytest.mark.parametrize("n", [1, 31, 513, 4097, (1 << 20) + 7])
def test_split_unsplit(n):
    rng = np.random.default_rng(n)
    x = special_floats(rng, n)
    tb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    rho = torch.empty(n, dtype=torch.int8, device="cuda")
    F.flashopt_split(dev(x), tb, rho)
    otb, orho = oracle.split(x)
    np.testing.assert_array_equal(u16(tb), otb)
    np.testing.assert_array_equal(i8(rho), orho)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    F.flashopt_unsplit(tb, rho, out)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32),
                                  oracle.unsplit(otb, orho).view(np.uint32))


def test_split_structured_all_upper_halves():
    # every bf16 pattern x 16 tails (ties, neighbours, random) -- covers every
    # exponent, sign, Inf and NaN input of the encoder
    rng = np.random.default_rng(1)
    tails = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF] + list(rng.integers(0, 1 << 16, 10)),
                     np.uint32)
    bits = ((np.arange(1 << 16, dtype=np.uint32)[:, None] << 16) | tails[None, :]).reshape(-1)
    x = bits.view(np.float32)
    finite = np.isfinite(x)
    tb = torch.empty(x.size, dtype=torch.bfloat16, device="cuda")
    rho = torch.empty(x.size, dtype=torch.int8, device="cuda")
    F.flashopt_split(dev(x), tb, rho)
    otb, orho = oracle.split(x)
    gtb, grho = u16(tb), i8(rho)
    np.testing.assert_array_equal(gtb[finite], otb[finite])
    np.testing.assert_array_equal(grho, orho)
    nan = ~finite & np.isnan(x)
    assert np.all((gtb[nan] & 0x7F80) == 0x7F80) and np.all(gtb[nan] & 0x7F)


def test_unsplit_every_pattern_and_code():
    tb = np.repeat(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16), 256)
    rho = np.tile(np.arange(-128, 128, dtype=np.int16).astype(np.int8), 1 << 16)
    out = torch.empty(tb.size, dtype=torch.float32, device="cuda")
    F.flashopt_unsplit(dev(tb).view(torch.bfloat16), dev(rho), out)
    got = out.cpu().numpy()
    exp = oracle.unsplit(tb, rho)
    fin = np.isfinite(exp)
    np.testing.assert_array_equal(got[fin].view(np.uint32), exp[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(exp))


@pytest.mark.parametrize("scale", [1e-7, 1e-5, 1e-3, 1.0, 1e3])
@pytest.mark.parametrize("n", [33, 4097, 100_003])
def test_quantizers(scale, n):
    rng = np.random.default_rng(int(n + scale * 1e7) % 99991)
    m = (rng.standard_t(3, n) * scale).astype(np.float32)
    m[: n // 20] = 0.0
    q = torch.empty(n, dtype=torch.int8, device="cuda")
    s = torch.empty((n + 31) // 32, dtype=torch.float16, device="cuda")
    F.flashopt_quantize_m(dev(m), q, s)
    oq, os_ = oracle.quant_m(m)
    np.testing.assert_array_equal(i8(q), oq)
    np.testing.assert_array_equal(u16(s), os_)
    back = torch.empty(n, dtype=torch.float32, device="cuda")
    F.flashopt_dequantize_m(q, s, back)
    np.testing.assert_array_equal(back.cpu().numpy().view(np.uint32),
                                  oracle.dequant_m(oq, os_).view(np.uint32))
    v = (m.astype(np.float64) ** 2).astype(np.float32)
    qv = torch.empty(n, dtype=torch.uint8, device="cuda")
    F.flashopt_quantize_v(dev(v), qv, s)
    oqv, osv = oracle.quant_v(v)
    np.testing.assert_array_equal(u8(qv), oqv)
    np.testing.assert_array_equal(u16(s), osv)
    F.flashopt_dequantize_v(qv, s, back)
    np.testing.assert_array_equal(back.cpu().numpy().view(np.uint32),
                                  oracle.dequant_v(oqv, osv).view(np.uint32))


def test_quantizer_every_code_and_scale():
    # dequantise every (code, FP16 scale) pair the format can hold
    s = np.arange(0x7C00, dtype=np.uint16)                 # all finite non-negative scales
    n = s.size * 32
    q = (np.arange(n) * 37 % 255 - 127).astype(np.int8)
    back = torch.empty(n, dtype=torch.float32, device="cuda")
    F.flashopt_dequantize_m(dev(q), dev(np.minimum(s, 0x3FFF)).view(torch.float16), back)
    exp = oracle.dequant_m(q, np.minimum(s, 0x3FFF))
    np.testing.assert_array_equal(back.cpu().numpy().view(np.uint32), exp.view(np.uint32))
    qv = (np.arange(n) * 53 % 256).astype(np.uint8)
    F.flashopt_dequantize_v(dev(qv), dev(s).view(torch.float16), back)
    np.testing.assert_array_equal(back.cpu().numpy().view(np.uint32),
                                  oracle.dequant_v(qv, s).view(np.uint32))


@pytest.mark.parametrize("opt", ["adamw", "sgd", "lion"])
def test_ragged_list_every_step(opt):
    w = W.ragged(RAGGED, seed=11, steps=4, optimizer=opt, grad_scale=1e-2 if opt == "sgd" else 1e-3)
    r = Run(w, "full")
    r.compare("init")
    for t in range(1, w.steps + 1):
        r.step(t)
        r.compare(f"step {t}")


@pytest.mark.parametrize("grad_dist", ["normal", "mixed"])
def test_linear_variance_kind_every_step(grad_dist):
    """The fused step's ablation kind (variance with linear codes) against
    the oracle, every code and scale: with mixed gradients (exact zeros,
    outliers, subnormals) many variances code to 0 and their quotients leave
    the short sequence's window, so the general fallback runs too."""
    base = W.ragged(RAGGED, seed=15, steps=4, optimizer="adamw_linv")
    w = W.Workload(base.name, base.tensors, "adamw_linv", 4, base.seed, grad_dist,
                   base.grad_scale, base.hparams)
    r = Run(w, "full")
    for t in range(1, w.steps + 1):
        r.step(t)
        r.compare(f"linear variance {grad_dist} step {t}")
    st = r.states[RAGGED.index(32 * 777 + 5)]
    th, m, v = (torch.empty(st.numel, device="cuda") for _ in range(3))
    F.flashopt_tensor_export(st, th, m, v)
    o = r.orc[RAGGED.index(32 * 777 + 5)]
    np.testing.assert_array_equal(v.cpu().numpy().view(np.uint32),
                                  oracle.dequant_lin_v(o.qv, o.sv).view(np.uint32))


@pytest.mark.parametrize("opt", ["adamw", "sgd", "lion", "adamw_linv"])
def test_release_mode_matches_list_mode(opt):
    base = W.ragged(RAGGED[:12], seed=12, steps=3, optimizer=opt)
    rel = W.Workload(base.name, base.tensors, opt, 3, base.seed, base.grad_dist, base.grad_scale,
                     base.hparams, release=True)
    a, b = Run(base, "full"), Run(rel, "full")
    for t in range(1, 4):
        a.step(t)
        b.step(t)
        b.compare(f"release step {t}")
        for sa, sb in zip(a.states, b.states):
            assert torch.equal(sa.theta.view(torch.int16), sb.theta.view(torch.int16))
            assert torch.equal(sa.codes, sb.codes) and torch.equal(sa.scales, sb.scales)


@pytest.mark.parametrize("opt", ["adamw", "lion"])
def test_release_launches_in_the_hybrid_form(opt):
    """Gradient-release launches of at least 16384 tiles take the hybrid form
    (whole tiles, then the last tiles as 512-element sub-tile waves): a tensor
    just past that size with a ragged tail, one with exactly 20000 tiles, and
    a range launch over both, against the whole-list launch, bit for bit,
    for two steps; sampled groups against the oracle, including groups of the
    sub-tile part and the partial last tile."""
    tile = 2048
    sizes = [16384 * tile + 1000, 20000 * tile]
    base = W.ragged(sizes, seed=31, steps=2, optimizer=opt)
    rel = W.Workload(base.name, base.tensors, opt, 2, base.seed, base.grad_dist, base.grad_scale,
                     base.hparams, release=True)
    last = [(n - 1) // 32 for n in sizes]
    extra = [g - k for g in last for k in (1, 7, 64, 5000, 80000)]
    a, b = Run(base, "sampled", seed=31, extra_groups=extra), Run(rel, "sampled", seed=31,
                                                                  extra_groups=extra)
    for t in (1, 2):
        a.step(t)
        b.step(t)
        b.compare(f"hybrid release step {t}")
        for sa, sb in zip(a.states, b.states):
            assert torch.equal(sa.theta.view(torch.int16), sb.theta.view(torch.int16))
            assert torch.equal(sa.codes, sb.codes) and torch.equal(sa.scales, sb.scales)
    hp = base.hparams
    for t in (3, 4):                      # a range launch (bucket) over both tensors
        grads = [W.draw_grad(base, i, t, "cuda") for i in range(2)]
        for i in range(2):
            a.grads[i].copy_(grads[i])
        F.step(a.lst, opt, hp, t)
        F.step_range(b.lst, opt, 0, grads, hp, t)
        torch.cuda.synchronize()
        for sa, sb in zip(a.states, b.states):
            assert torch.equal(sa.theta.view(torch.int16), sb.theta.view(torch.int16))
            assert torch.equal(sa.codes, sb.codes) and torch.equal(sa.scales, sb.scales)


def test_hyperparameter_variants():
    w = W.ragged([4097, 33, 2048 * 3 + 1], seed=13, steps=3)
    r = Run(w, "full")
    for t, hp in enumerate([dict(lr=3e-2, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1),
                            dict(lr=1e-4, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0),
                            dict(lr=1e-3, beta1=0.99, beta2=0.9999, eps=1e-12, weight_decay=0.5)],
                           1):
        r.step(t, hp)
        r.compare(f"hp {t}")
    r.step(1000, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01))
    r.compare("t=1000")


@pytest.mark.parametrize("grad_scale", [1e-4, 1e18, 1e-38])
def test_adam_quotient_window_edges(grad_scale):
    # zeros, subnormal and outlier gradients (1e18: squares overflow, so some
    # denominators are Inf; 1e-38: quotients far below the fast window) under
    # eps values that move the window (1e-30 narrows it, 1e-40 is subnormal in
    # binary32 and closes it, 1e3 is large)
    base = W.ragged([4097, 1000, 33], seed=15, steps=1)
    w = W.Workload("quotient_edges", base.tensors, "adamw", 4, 15, "mixed", grad_scale,
                   W.ADAMW_HP, special_theta=True)
    r = Run(w, "full")
    for t, eps in enumerate([1e-8, 1e-30, 1e-40, 1e3], 1):
        r.step(t, dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=eps, weight_decay=0.01))
        r.compare(f"grad scale {grad_scale}, eps {eps}")


def test_lion_hyperparameter_variants_and_edge_gradients():
    # zero, subnormal and outlier gradients (sign(0) = 0 leaves only the decay),
    # special weights, and settings that isolate each coefficient
    base = W.ragged([4097, 1000, 33, 2048 * 2], seed=16, steps=1, optimizer="lion")
    w = W.Workload("lion_edges", base.tensors, "lion", 6, 16, "mixed", 1e-3, W.LION_HP,
                   special_theta=True)
    r = Run(w, "full")
    for t, hp in enumerate([W.LION_HP,
                            dict(lr=1e-3, beta1=0.0, beta2=0.0, weight_decay=0.0),
                            dict(lr=3e-4, beta1=0.99, beta2=0.5, weight_decay=1.0),
                            dict(lr=0.0, beta1=0.9, beta2=0.99, weight_decay=0.1),
                            dict(lr=1e-2, beta1=0.5, beta2=0.999, weight_decay=0.0),
                            W.LION_HP], 1):
        r.step(t, hp)
        r.compare(f"lion hp {t}")


def test_sgd_hyperparameter_variants_and_edge_gradients():
    # zero, subnormal and outlier gradients, special weights (zeros,
    # subnormals, powers of two), and settings that isolate each coefficient:
    # no momentum (the closed form theta - lr*(g + wd*theta)), no decay, a
    # frozen step (lr = 0), heavy momentum and a large rate
    base = W.ragged([4097, 1000, 33, 2048 * 2], seed=22, steps=1, optimizer="sgd")
    w = W.Workload("sgd_edges", base.tensors, "sgd", 6, 22, "mixed", 1e-2, W.SGD_HP,
                   special_theta=True)
    r = Run(w, "full")
    for t, hp in enumerate([W.SGD_HP,
                            dict(lr=0.1, momentum=0.0, weight_decay=1e-4),
                            dict(lr=0.05, momentum=0.9, weight_decay=0.0),
                            dict(lr=0.0, momentum=0.9, weight_decay=1e-4),
                            dict(lr=0.01, momentum=0.99, weight_decay=5e-4),
                            dict(lr=3.0, momentum=0.5, weight_decay=1e-2)], 1):
        r.step(t, hp)
        r.compare(f"sgd hp {t}")


@pytest.mark.parametrize("opt", ["adamw", "sgd", "lion"])
def test_non_finite_gradients_stay_in_their_groups(opt):
    """Non-finite gradients are outside the contract, but they must neither
    fault nor leak: with NaN and +-Inf gradients in a few 32-element groups,
    every other group's codes and scales still equal the oracle's bit for
    bit, step after step (groups are independent in the method)."""
    n = 32 * 64 + 9
    rng = np.random.default_rng(16)
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    st = F.TensorState(n, opt, "cuda")
    F.flashopt_tensor_init(st, torch.from_numpy(theta).cuda())
    o = oracle.State(theta, opt)
    g = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    lst = F.FlashoptList([st], [g])
    bad_groups = [3, 17, 64]                             # 64: the partial last group
    hp = W.HPARAMS[opt]
    for t in (1, 2, 3):
        x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        x[3 * 32 + 5] = np.nan
        x[17 * 32] = np.inf
        x[17 * 32 + 31] = -np.inf
        x[64 * 32 + 2] = np.nan
        gb = torch.from_numpy(x).to(torch.bfloat16)
        g.copy_(gb)
        F.step(lst, opt, hp, t)
        oracle.step(o, gb.view(torch.int16).numpy().view(np.uint16), t, hp)
        torch.cuda.synchronize()
        f = state_fields(st)
        ok = np.ones(n, bool)
        for b in bad_groups:
            ok[b * 32:(b + 1) * 32] = False
        gok = np.ones((n + 31) // 32, bool)
        gok[bad_groups] = False
        keys = [("theta", "tb"), ("rho", "rho"), ("m_code", "qm")]
        if opt == "adamw":
            keys.append(("v_code", "qv"))
        for k, ok_name in keys:
            np.testing.assert_array_equal(f[k][ok], getattr(o, ok_name)[ok], err_msg=f"{k} {t}")
        np.testing.assert_array_equal(f["m_scale"][gok], o.sm[gok])
        if opt == "adamw":
            np.testing.assert_array_equal(f["v_scale"][gok], o.sv[gok])


@pytest.mark.parametrize("opt", ["adamw", "sgd", "lion", "adamw_fp32"])
def test_arena_state_equals_per_tensor_state(opt):
    """The same ragged list stepped with its state in one StateArena and with
    one allocation per tensor: every theta', code and scale equal bit for bit
    after each step (the layout inside each tensor's state is the same)."""
    sizes = [4097, 0, 33, 2048 * 3, 1, (1 << 17) + 5]
    rng = np.random.default_rng(17)
    thetas = [torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).cuda()
              for n in sizes]
    arena = F.StateArena(sizes, opt, "cuda")
    a = [arena.state(i) for i in range(len(sizes))]
    b = [F.TensorState(n, opt, "cuda") for n in sizes]
    for sa, sb, th in zip(a, b, thetas):
        F.flashopt_tensor_init(sa, th)
        F.flashopt_tensor_init(sb, th)
    grads = [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
    la, lb = F.FlashoptList(a, grads), F.FlashoptList(b, grads)
    base = F.base_optimizer(opt)
    hp = W.HPARAMS[base]
    for t in (1, 2, 3):
        for g in grads:
            g.copy_(torch.from_numpy((rng.standard_normal(g.numel()) * 1e-3)
                                     .astype(np.float32)).to(torch.bfloat16))
        F.step(la, base, hp, t)
        F.step(lb, base, hp, t)
        torch.cuda.synchronize()
        for i, (sa, sb) in enumerate(zip(a, b)):
            assert torch.equal(sa.theta.view(torch.int16), sb.theta.view(torch.int16)), (t, i)
            assert torch.equal(sa.codes, sb.codes), (t, i)
            assert torch.equal(sa.scales, sb.scales), (t, i)


@pytest.mark.parametrize("opt", ["adamw", "sgd", "lion", "adamw_fp32", "adamw_linv"])
def test_bucketed_range_steps_equal_the_whole_list_step(opt):
    """flashopt_*_step_range over buckets of consecutive tensors, issued in
    backward order with fresh gradient tensors each step (and an empty
    range), equals the whole-list step bit for bit."""
    sizes = [4097, 0, 33, 2048 * 3, 1, (1 << 17) + 5, 2048, 7]
    buckets = [(6, 2), (5, 1), (2, 3), (2, 0), (0, 2)]      # (first, count), backward order
    assert sorted(i for f, c in buckets for i in range(f, f + c)) == list(range(len(sizes)))
    rng = np.random.default_rng(18)
    thetas = [torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).cuda()
              for n in sizes]
    arena = F.StateArena(sizes, opt, "cuda")
    a = [arena.state(i) for i in range(len(sizes))]
    b = [F.TensorState(n, opt, "cuda") for n in sizes]
    for sa, sb, th in zip(a, b, thetas):
        F.flashopt_tensor_init(sa, th)
        F.flashopt_tensor_init(sb, th)
    ga = [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
    la = F.FlashoptList(a, ga)
    lb = F.FlashoptList(b, [None] * len(sizes))
    base = F.base_optimizer(opt)
    hp = W.HPARAMS[base]
    for t in (1, 2, 3):
        gs = [torch.from_numpy((rng.standard_normal(n) * 1e-3).astype(np.float32))
              .to(torch.bfloat16).cuda() for n in sizes]
        for g, d in zip(ga, gs):
            g.copy_(d)
        F.step(la, base, hp, t)
        for first, count in buckets:
            F.step_range(lb, base, first, [gs[i] if sizes[i] else None
                                           for i in range(first, first + count)], hp, t)
        torch.cuda.synchronize()
        for i, (sa, sb) in enumerate(zip(a, b)):
            assert torch.equal(sa.theta.view(torch.int16), sb.theta.view(torch.int16)), (t, i)
            assert torch.equal(sa.codes, sb.codes), (t, i)
            assert torch.equal(sa.scales, sb.scales), (t, i)


@pytest.mark.parametrize("opt", ["adamw", "sgd"])
def test_list_of_three_thousand_small_tensors(opt):
    """A list of 3000 tensors with sizes around the group, sub-tile and tile
    boundaries (and many empty ones): the tile table's search, gradient
    pointers replaced in 15 batches between steps, every code and scale
    against the oracle."""
    cycle = [0, 1, 31, 32, 33, 0, 511, 512, 513, 2047, 2048, 2049, 5000, 0, 7]
    sizes = [cycle[i % len(cycle)] for i in range(3000)]
    w = W.ragged(sizes, seed=21, steps=3, optimizer=opt)
    r = Run(w, "full")
    r.step(1)
    r.compare("step 1")
    new = [torch.zeros(st.numel, dtype=torch.bfloat16, device="cuda") for st in r.states]
    F.flashopt_list_set_grads(r.lst, new)
    r.grads = new
    for t in (2, 3):
        r.step(t)
        r.compare(f"step {t}")


def test_set_grads_and_state_zero():
    w = W.ragged([3000, 70], seed=14, steps=2)
    r = Run(w, "full")
    r.step(1)
    new = [torch.zeros(s.numel, dtype=torch.bfloat16, device="cuda") for s in r.states]
    F.flashopt_list_set_grads(r.lst, new)
    r.grads = new
    r.step(2)
    r.compare("after set_grads")
    before = [state_fields(s) for s in r.states]
    F.flashopt_state_zero(r.lst)
    torch.cuda.synchronize()
    for s, b in zip(r.states, before):
        f = state_fields(s)
        for k in ("m_code", "v_code", "m_scale", "v_scale"):
            assert not f[k].any(), k
        np.testing.assert_array_equal(f["rho"], b["rho"])       # the weight split is kept
        np.testing.assert_array_equal(f["theta"], b["theta"])


@pytest.mark.parametrize("opt", ["adamw", "lion"])
def test_tensor_beyond_2_to_31_elements(opt):
    # one tensor past 32-bit element indices (and past 2^32 code-record bytes
    # for AdamW), in the launch shape of the benchmark; compared at the first
    # and last groups, random ones, and the groups around element 2^31
    n = (1 << 31) + (1 << 20) + 7
    w = W.Workload("huge", (W.TensorSpec("huge", (n,), "normal"),), opt, 2, 21, "normal", 1e-3,
                   W.HPARAMS[opt])
    edge = (1 << 31) // 32
    r = Run(w, "sampled", samples_per_tensor=8, extra_groups=range(edge - 2, edge + 3))
    for t in (1, 2):
        r.step(t)
        n_cmp = r.compare(f"{opt} huge step {t}")
    log(f"{opt} tensor of {n} elements: {n_cmp} sampled elements compared")


def test_range_launch_gradients_serve_that_launch_only():
    """After a range launch the list holds no gradient for those tensors: a
    whole-list step is refused (FLASHOPT_ERR_NULL) until set_grads gives them
    again, and the binding keeps no reference to the released gradients."""
    sizes = [4097, 33]
    states = [F.TensorState(n, "adamw", "cuda") for n in sizes]
    for st in states:
        F.flashopt_tensor_init(st, torch.zeros(st.numel, device="cuda"))
    gs = [torch.ones(n, dtype=torch.bfloat16, device="cuda") * 1e-3 for n in sizes]
    lst = F.FlashoptList(states, gs)
    F.step(lst, "adamw", W.ADAMW_HP, 1)                  # the list's own gradients
    g0 = torch.ones(sizes[0], dtype=torch.bfloat16, device="cuda")
    F.step_range(lst, "adamw", 0, [g0], W.ADAMW_HP, 2)
    assert lst.grads[0] is None and lst.grads[1] is gs[1]
    with pytest.raises(F.FlashoptError) as e:
        F.step(lst, "adamw", W.ADAMW_HP, 3)
    assert e.value.status == -1                          # FLASHOPT_ERR_NULL
    F.flashopt_list_set_grads(lst, gs)
    F.step(lst, "adamw", W.ADAMW_HP, 3)
    torch.cuda.synchronize()


def test_range_launch_of_a_large_tensor_after_a_small_one():
    """A range launch whose first tile is not 0 in the one-wave-per-tile form
    (the range holds 16384 tiles): equal to the whole-list step bit for bit."""
    sizes = [1000, 16384 * 2048 - 3]
    rng = np.random.default_rng(20)
    thetas = [torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).cuda()
              for n in sizes]
    a = [F.TensorState(n, "adamw", "cuda") for n in sizes]
    b = [F.TensorState(n, "adamw", "cuda") for n in sizes]
    for sa, sb, th in zip(a, b, thetas):
        F.flashopt_tensor_init(sa, th)
        F.flashopt_tensor_init(sb, th)
    del thetas
    gs = [torch.from_numpy((rng.standard_normal(n) * 1e-3).astype(np.float32))
          .to(torch.bfloat16).cuda() for n in sizes]
    la, lb = F.FlashoptList(a, gs), F.FlashoptList(b, [None, None])
    for t in (1, 2):
        F.step(la, "adamw", W.ADAMW_HP, t)
        F.step_range(lb, "adamw", 1, [gs[1]], W.ADAMW_HP, t)
        F.step_range(lb, "adamw", 0, [gs[0]], W.ADAMW_HP, t)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(a[i].theta.view(torch.int16), b[i].theta.view(torch.int16)), (t, i)
            assert torch.equal(a[i].codes, b[i].codes) and torch.equal(a[i].scales, b[i].scales)


@pytest.mark.parametrize("extra_tiles", [0, 1])
def test_both_sides_of_the_split_launch_threshold(extra_tiles):
    """Lists of 16383 tiles (the split form: one wave per 512-element
    sub-tile) and 16384 tiles (one wave per tile), with a partial last tile in
    each tensor, against the oracle on sampled groups (including groups of
    the last, partial tile of every tensor) for two steps."""
    tile = 2048
    sizes = [16000 * tile - 7, 381 * tile + 100 + extra_tiles * tile, 1000]
    assert sum(-(-n // tile) for n in sizes) == 16383 + extra_tiles
    w = W.ragged(sizes, seed=19, steps=2)
    last = [(n - 1) // 32 for n in sizes]
    r = Run(w, "sampled", samples_per_tensor=6, seed=19,
            extra_groups=[g - k for g in last for k in (1, 5, 17, 40)])
    for t in (1, 2):
        r.step(t)
        r.compare(f"{16383 + extra_tiles} tiles, step {t}")


def test_config1_flat1m_all_steps():
    w = W.WORKLOADS["flat1m"]
    r = Run(w, "full")
    for t in range(1, w.steps + 1):
        r.step(t)
        n = r.compare(f"step {t}")
    log(f"flat1m: {w.steps} steps, {n} elements compared per step")


def test_config3_resnet50_sgd():
    w = W.WORKLOADS["resnet50"]
    r = Run(w, "full")
    for t in range(1, w.steps + 1):
        r.step(t, threads=16)
        if t in (1, 2, w.steps):
            n = r.compare(f"step {t}")
            log(f"resnet50 step {t}: {n} elements compared")


def test_llama8b_lion_sampled():
    w = W.WORKLOADS["llama31_8b_lion"]
    r = Run(w, "sampled", samples_per_tensor=4)
    log("llama8b lion: state built")
    for t in range(1, w.steps + 1):
        r.step(t)
        if t in (1, 2, w.steps):
            n = r.compare(f"step {t}")
            log(f"llama8b lion step {t}: {n} sampled elements compared")
