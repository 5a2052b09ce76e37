"""The drop-in optimizers (compressed_adamw_state_amd/optim.py) against the
oracle: FlashAdamW / FlashSGD / FlashLion steps over FP32 and BF16
parameters give the oracle's codes and scales bit for bit; a checkpoint
(state_dict of codes and scales, theta' as the model's BF16 weights) resumes
bit for bit; gradient release from backward hooks equals stepping after
backward and, end to end over a stack of linear layers, lowers the peak of
allocated memory by about the gradients' 2 B/param; and the checkpoint holds 3.125 (AdamW) / 2.0625 (SGD, Lion) bytes
per parameter besides theta'."""
import numpy as np
import pytest
import torch

import oracle
from compressed_adamw_state_amd import optim as O

from parity import log, state_fields, u16

pytestmark = pytest.mark.gpu

HP = {"adamw": dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
      "sgd": dict(lr=0.05, momentum=0.9, weight_decay=1e-4),
      "lion": dict(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.1)}
SHAPES = [(4097,), (33, 64), (2048,), (7,)]


def make_opt(kind, params, release=False, streams=1):
    hp = HP[kind]
    if kind == "adamw":
        return O.FlashAdamW(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], gradient_release=release,
                            release_streams=streams)
    if kind == "sgd":
        return O.FlashSGD(params, lr=hp["lr"], momentum=hp["momentum"],
                          weight_decay=hp["weight_decay"], gradient_release=release,
                          release_streams=streams)
    return O.FlashLion(params, lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]),
                       weight_decay=hp["weight_decay"], gradient_release=release,
                       release_streams=streams)


def compare(opt, params, orcs, label):
    keys = [("theta", "tb"), ("rho", "rho"), ("m_code", "qm"), ("m_scale", "sm")]
    if opt.kind == "adamw":
        keys += [("v_code", "qv"), ("v_scale", "sv")]
    for i, (p, o) in enumerate(zip(params, orcs)):
        f = state_fields(opt.state[p]["flash"])
        np.testing.assert_array_equal(u16(p.data.view(-1)), f["theta"])    # theta' is p
        for k, ok in keys:
            np.testing.assert_array_equal(f[k], getattr(o, ok), err_msg=f"{label} param {i} {k}")


@pytest.mark.parametrize("kind", ["adamw", "sgd", "lion"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_optimizer_steps_match_oracle(kind, dtype):
    rng = np.random.default_rng(3)
    init = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in SHAPES]
    if dtype == torch.bfloat16:   # the oracle starts from the same BF16 values (rho = 0)
        init = [torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in init]
    params = [torch.nn.Parameter(torch.from_numpy(x).cuda().to(dtype)) for x in init]
    opt = make_opt(kind, params)
    assert all(p.dtype == torch.bfloat16 for p in params)
    orcs = [oracle.State(x.reshape(-1), kind) for x in init]
    compare(opt, params, orcs, "init")
    for t in range(1, 4):
        for p, o in zip(params, orcs):
            g = torch.from_numpy((rng.standard_normal(p.shape) * 1e-3).astype(np.float32))
            g = g.to(torch.bfloat16)
            p.grad = g.cuda()
            oracle.step(o, g.view(torch.int16).numpy().view(np.uint16).reshape(-1), t, HP[kind])
        opt.step()
        torch.cuda.synchronize()
        compare(opt, params, orcs, f"step {t}")


@pytest.mark.parametrize("kind", ["adamw", "lion"])
def test_checkpoint_resumes_bit_for_bit(kind):
    rng = np.random.default_rng(4)
    init = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in SHAPES]
    grads = [[torch.from_numpy((rng.standard_normal(s) * 1e-3).astype(np.float32))
              .to(torch.bfloat16).cuda() for s in SHAPES] for _ in range(6)]

    def run(params, opt, steps):
        for gs in steps:
            for p, g in zip(params, gs):
                p.grad = g.clone()
            opt.step()

    a = [torch.nn.Parameter(torch.from_numpy(x).cuda()) for x in init]
    oa = make_opt(kind, a)
    run(a, oa, grads)                                    # six steps without a break

    b = [torch.nn.Parameter(torch.from_numpy(x).cuda()) for x in init]
    ob = make_opt(kind, b)
    run(b, ob, grads[:3])
    sd = ob.state_dict()
    weights = [p.detach().clone() for p in b]            # theta', saved with the model
    nbytes = sum(s["codes"].numel() + 2 * s["scales"].numel() for s in sd["state"].values())
    numel = sum(p.numel() for p in b)
    del ob, b
    c = [torch.nn.Parameter(w) for w in weights]         # a fresh model from the checkpoint
    oc = make_opt(kind, c)
    oc.load_state_dict(sd)
    run(c, oc, grads[3:])
    torch.cuda.synchronize()
    for pa, pc in zip(a, c):
        assert torch.equal(pa.view(torch.int16), pc.view(torch.int16))
        sa, sc = oa.state[pa]["flash"], oc.state[pc]["flash"]
        assert torch.equal(sa.codes, sc.codes) and torch.equal(sa.scales, sc.scales)
    # the state and its padding only: AdamW's codes in whole 1536-byte blocks of
    # 512 elements, Lion's in 16-byte records of 8; the scales per 32
    per = {"adamw": 3.125, "lion": 2.0625}[kind]
    blk, unit, scl, pad = {"adamw": (512, 1536, 4, 1536), "lion": (8, 16, 2, 64)}[kind]
    exact = sum((p.numel() + blk - 1) // blk * unit + (p.numel() + 31) // 32 * scl for p in c)
    assert nbytes == exact and nbytes <= per * numel + pad * len(c)
    # a checkpoint whose codes are placed otherwise is refused, not reinterpreted
    for tag in ("records24", None):
        with pytest.raises(ValueError, match="codes layout"):
            oc.load_state_dict({**sd, "codes_layout": tag})


@pytest.mark.parametrize("streams", [1, 2])
@pytest.mark.parametrize("kind", ["adamw", "sgd", "lion"])
def test_gradient_release_equals_step_after_backward(kind, streams):
    # an elementwise loss (no reductions whose order could vary between the
    # two runs): the gradient of sum(c*p + k*p^2/2) is c + k*p
    torch.manual_seed(5)
    dims = [(256, 512), (512,), (512, 96), (96,)]
    init = [torch.randn(d) * 0.02 for d in dims]
    coef = [(torch.randn(d) * 1e-3).cuda() for d in dims]
    x = 0.5

    def model(ps, k):
        loss = 0.0
        for p, c in zip(ps, coef):
            pf = p.float()
            loss = loss + (c * pf + 0.5 * k * pf * pf).sum()
        return loss

    a = [torch.nn.Parameter(t.clone().cuda()) for t in init]
    b = [torch.nn.Parameter(t.clone().cuda()) for t in init]
    oa = make_opt(kind, a)
    ob = make_opt(kind, b, release=True, streams=streams)
    for it in range(3):
        inp = x * (1 + it)
        model(a, inp).backward()
        oa.step()
        oa.zero_grad()
        model(b, inp).backward()                         # hooks step each parameter
        assert all(p.grad is None for p in b)            # gradients released
        ob.step()
    torch.cuda.synchronize()
    for pa, pb in zip(a, b):
        assert torch.equal(pa.view(torch.int16), pb.view(torch.int16))
        sa, sb = oa.state[pa]["flash"], ob.state[pb]["flash"]
        assert torch.equal(sa.codes, sb.codes) and torch.equal(sa.scales, sb.scales)


def test_export_fp32_matches_oracle_rebuild():
    rng = np.random.default_rng(6)
    init = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in SHAPES]
    params = [torch.nn.Parameter(torch.from_numpy(x).cuda()) for x in init]
    opt = make_opt("adamw", params)
    orcs = [oracle.State(x.reshape(-1), "adamw") for x in init]
    for p, o in zip(params, orcs):
        g = torch.from_numpy((rng.standard_normal(p.shape) * 1e-3).astype(np.float32))
        g = g.to(torch.bfloat16)
        p.grad = g.cuda()
        oracle.step(o, g.view(torch.int16).numpy().view(np.uint16).reshape(-1), 1, HP["adamw"])
    opt.step()
    for p, o in zip(params, orcs):
        th, m, v = opt.export_fp32(p)
        np.testing.assert_array_equal(th.cpu().numpy().view(np.uint32),
                                      oracle.unsplit(o.tb, o.rho).view(np.uint32))
        np.testing.assert_array_equal(m.cpu().numpy().view(np.uint32),
                                      oracle.dequant_m(o.qm, o.sm).view(np.uint32))
        np.testing.assert_array_equal(v.cpu().numpy().view(np.uint32),
                                      oracle.dequant_v(o.qv, o.sv).view(np.uint32))


@pytest.mark.parametrize("kind", ["adamw", "lion", "sgd"])
def test_training_tracks_the_uncompressed_optimizer(kind):
    """Fig. 2's claim on a synthetic regression task: a small MLP trained
    with the compressed optimizer (BF16 weights theta', compressed state)
    follows the loss curve of torch's optimizer on FP32 weights.  The model
    computes in FP32 (weights upcast in the forward), so no BF16 GEMM runs."""
    torch.manual_seed(7)
    n, d, h = 4096, 64, 256
    X = torch.randn(n, d, device="cuda")
    a = torch.randn(d, device="cuda") / d ** 0.5
    y = (torch.sin(3 * X @ a) + 0.1 * torch.randn(n, device="cuda")).unsqueeze(1)
    init = [torch.randn(h, d) / d ** 0.5, torch.zeros(h), torch.randn(1, h) / h ** 0.5,
            torch.zeros(1)]

    def loss_of(ps):
        w1, b1, w2, b2 = (p.float() for p in ps)
        return ((torch.relu(X @ w1.t() + b1) @ w2.t() + b2 - y) ** 2).mean()

    hp = {"adamw": dict(lr=3e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01),
          "lion": dict(lr=3e-4, betas=(0.9, 0.99), weight_decay=0.1),
          "sgd": dict(lr=0.05, momentum=0.9, weight_decay=1e-4)}[kind]
    flash = [torch.nn.Parameter(t.clone().cuda()) for t in init]
    ref = [torch.nn.Parameter(t.clone().cuda()) for t in init]
    fo = {"adamw": O.FlashAdamW, "lion": O.FlashLion, "sgd": O.FlashSGD}[kind](flash, **hp)
    if kind == "adamw":
        ro = torch.optim.AdamW(ref, **hp)
    elif kind == "sgd":
        ro = torch.optim.SGD(ref, **hp)
    else:
        ro = None                                        # torch has no Lion: reference below
        m_ref = [torch.zeros_like(p) for p in ref]
    curves = {"flash": [], "ref": []}
    for it in range(300):
        for ps, opt, key in ((flash, fo, "flash"), (ref, ro, "ref")):
            loss = loss_of(ps)
            curves[key].append(loss.item())
            if ps is flash:
                opt.zero_grad()
                loss.backward()
                opt.step()
            else:
                for p in ps:
                    p.grad = None
                loss.backward()
                if ro is not None:
                    ro.step()
                else:                                    # the published Lion rule, FP32
                    with torch.no_grad():
                        b1, b2 = hp["betas"]
                        for p, m in zip(ps, m_ref):
                            c = b1 * m + (1 - b1) * p.grad
                            p.mul_(1 - hp["lr"] * hp["weight_decay"]).sub_(hp["lr"] * torch.sign(c))
                            m.mul_(b2).add_((1 - b2) * p.grad)
    f, r = np.array(curves["flash"]), np.array(curves["ref"])
    log(f"{kind}: loss {f[0]:.4f} -> flash {f[-1]:.4f}, reference {r[-1]:.4f}")
    assert f[-1] < 0.5 * f[0] and r[-1] < 0.5 * r[0]    # both learn
    # the curves stay together: within 10 % (plus the noise floor) at every 25th step
    for k in range(25, 300, 25):
        assert abs(f[k] - r[k]) <= 0.1 * r[k] + 2e-3, (k, f[k], r[k])


def test_parameters_without_gradients_are_skipped():
    """As torch.optim: a parameter whose .grad is None is left untouched
    (weights, codes and scales), and each parameter keeps its own step count,
    so a parameter skipped once is later stepped with its own bias
    correction (the oracle steps it with t = 1, 2 while the others reach 3)."""
    rng = np.random.default_rng(8)
    init = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in SHAPES]
    params = [torch.nn.Parameter(torch.from_numpy(x).cuda()) for x in init]
    opt = make_opt("adamw", params)
    orcs = [oracle.State(x.reshape(-1), "adamw") for x in init]
    counts = [0] * len(params)
    for it in range(3):
        before = [(p.detach().clone(), opt.state[p]["flash"].codes.clone()) for p in params]
        for i, (p, o) in enumerate(zip(params, orcs)):
            if it == 1 and i == 1:
                p.grad = None                            # skipped this step
                continue
            g = torch.from_numpy((rng.standard_normal(p.shape) * 1e-3).astype(np.float32))
            g = g.to(torch.bfloat16)
            p.grad = g.cuda()
            counts[i] += 1
            oracle.step(o, g.view(torch.int16).numpy().view(np.uint16).reshape(-1), counts[i],
                        HP["adamw"])
        opt.step()
        torch.cuda.synchronize()
        if it == 1:
            assert torch.equal(params[1].view(torch.int16), before[1][0].view(torch.int16))
            assert torch.equal(opt.state[params[1]]["flash"].codes, before[1][1])
        compare(opt, params, orcs, f"iteration {it}")
    assert [opt.state[p]["step"] for p in params] == counts == [3, 2, 3, 3]
    # and the per-parameter counts survive a checkpoint
    sd = opt.state_dict()
    assert [sd["state"][i]["step"] for i in range(len(params))] == counts


def test_add_param_group_after_construction():
    """torch.optim's add_param_group after construction: the new group gets
    its compressed state (and its own hyper-parameters) and is stepped like
    the first, matching the oracle."""
    rng = np.random.default_rng(9)
    a0 = (rng.standard_normal(4097) * 0.02).astype(np.float32)
    b0 = (rng.standard_normal((33, 64)) * 0.02).astype(np.float32)
    pa = torch.nn.Parameter(torch.from_numpy(a0).cuda())
    pb = torch.nn.Parameter(torch.from_numpy(b0).cuda())
    opt = make_opt("adamw", [pa])
    hp_b = dict(HP["adamw"], lr=3e-4)
    opt.add_param_group({"params": [pb], "lr": hp_b["lr"]})
    assert pb.dtype == torch.bfloat16 and "flash" in opt.state[pb]
    oa, ob = oracle.State(a0, "adamw"), oracle.State(b0.reshape(-1), "adamw")
    for t in (1, 2):
        for p, o, hp in ((pa, oa, HP["adamw"]), (pb, ob, hp_b)):
            g = torch.from_numpy((rng.standard_normal(p.shape) * 1e-3).astype(np.float32))
            g = g.to(torch.bfloat16)
            p.grad = g.cuda()
            oracle.step(o, g.view(torch.int16).numpy().view(np.uint16).reshape(-1), t, hp)
        opt.step()
        torch.cuda.synchronize()
        compare(opt, [pa, pb], [oa, ob], f"step {t}")


@pytest.mark.parametrize("streams,bucket", [(1, 0), (2, 0), (1, 4 << 20)])
def test_gradient_release_saves_the_gradient_memory_end_to_end(streams, bucket):
    """Forward + backward + step of a stack of BF16 linear layers: with
    gradient release the peak of allocated memory during an iteration is lower
    by about the gradients' 2 B/param (all but the few gradients in flight, or
    in the open bucket), and the weights after two iterations equal stepping
    after backward bit for bit."""
    layers, width, batch = 8, 1024, 4
    n = layers * width * width
    x = torch.randn(batch, width, device="cuda", dtype=torch.bfloat16,
                    generator=torch.Generator("cuda").manual_seed(5))
    peaks, weights = {}, {}
    for release in (False, True):
        torch.cuda.manual_seed(6)
        model = torch.nn.Sequential(*[torch.nn.Linear(width, width, bias=False, device="cuda",
                                                      dtype=torch.bfloat16)
                                      for _ in range(layers)])
        opt = O.FlashAdamW(model.parameters(), lr=1e-3, gradient_release=release,
                           release_streams=streams, release_bucket_bytes=bucket)

        def iteration():
            model(x).float().pow(2).mean().backward()
            opt.step()
            opt.zero_grad(set_to_none=True)

        iteration()
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        iteration()
        torch.cuda.synchronize()
        peaks[release] = torch.cuda.max_memory_allocated() - base
        weights[release] = [p.detach().view(torch.int16).clone() for p in model.parameters()]
        del opt, model
        torch.cuda.empty_cache()
    saving = (peaks[False] - peaks[True]) / n
    log(f"release ({streams} stream(s), bucket {bucket}): peak {peaks[False] / 2**20:.1f} MiB -> "
        f"{peaks[True] / 2**20:.1f} MiB, {saving:.3f} B/param saved")
    grad = 2 * width * width                           # one layer's gradient
    assert peaks[False] >= 2 * n                       # every gradient alive at the step
    assert peaks[True] <= max(bucket, grad) + 2 * grad + (1 << 20), (peaks, saving)
    for a, b in zip(weights[False], weights[True]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("kind", ["adamw", "sgd", "lion"])
@pytest.mark.parametrize("bucket", [1, 3 * 2 ** 20, 2 ** 40])
def test_bucketed_gradient_release_equals_step_after_backward(kind, bucket):
    """release_bucket_bytes: buckets of consecutive parameters stepped by one
    range launch (a bucket of one parameter, buckets of a few MiB, and one
    bucket left for step()) give the same weights and state as stepping after
    backward, bit for bit, over several iterations of a small MLP with
    parameters of mixed sizes."""
    torch.cuda.manual_seed(7)
    widths = [256, 1024, 64, 512, 8]
    x = torch.randn(16, widths[0], device="cuda", dtype=torch.bfloat16,
                    generator=torch.Generator("cuda").manual_seed(8))
    results = []
    for release in (False, True):
        torch.cuda.manual_seed(9)
        layers = []
        for a, b in zip(widths[:-1], widths[1:]):
            layers += [torch.nn.Linear(a, b, device="cuda", dtype=torch.bfloat16), torch.nn.Tanh()]
        model = torch.nn.Sequential(*layers)
        params = list(model.parameters())
        opt = make_opt(kind, params, release=release)
        if release:
            opt.release_bucket_bytes = bucket
        for _ in range(3):
            model(x).float().pow(2).mean().backward()
            opt.step()
            opt.zero_grad(set_to_none=True)
        torch.cuda.synchronize()
        results.append([(p.detach().view(torch.int16).clone(), opt.state[p]["flash"].codes.clone(),
                         opt.state[p]["flash"].scales.clone(), opt.state[p]["step"])
                        for p in params])
    for (ta, ca, sa, na), (tb, cb, sb, nb) in zip(*results):
        assert torch.equal(ta, tb) and torch.equal(ca, cb) and torch.equal(sa, sb) and na == nb


@pytest.mark.parametrize("kind", ["adamw", "sgd", "lion"])
def test_step_keeps_no_gradient_alive(kind):
    """As with torch's optimizers, step() followed by zero_grad() leaves no
    gradient allocated: between iterations the allocated memory is the
    parameters and the optimizer state only (a list that kept the last
    gradients would hold 2 B/param more through the next forward and
    backward)."""
    width, layers = 1024, 4
    torch.cuda.manual_seed(10)
    model = torch.nn.Sequential(*[torch.nn.Linear(width, width, bias=False, device="cuda",
                                                  dtype=torch.bfloat16) for _ in range(layers)])
    x = torch.randn(8, width, device="cuda", dtype=torch.bfloat16,
                    generator=torch.Generator("cuda").manual_seed(11))
    # one forward and backward first: the BLAS library's workspace is
    # allocated on a process's first products and stays
    model(x).float().pow(2).mean().backward()
    model.zero_grad(set_to_none=True)
    opt = make_opt(kind, list(model.parameters()))
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    for _ in range(2):
        model(x).float().pow(2).mean().backward()
        opt.step()
        opt.zero_grad(set_to_none=True)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == base


def test_checkpoint_during_bucketed_release_includes_the_open_bucket():
    """state_dict() taken after backward but before step() with a bucket
    still open steps that bucket first: the checkpoint equals the one taken
    after step(), codes, scales and step counts."""
    torch.cuda.manual_seed(12)
    model = torch.nn.Sequential(*[torch.nn.Linear(256, 256, device="cuda", dtype=torch.bfloat16)
                                  for _ in range(3)])
    x = torch.randn(4, 256, device="cuda", dtype=torch.bfloat16,
                    generator=torch.Generator("cuda").manual_seed(13))
    opt = make_opt("adamw", list(model.parameters()), release=True)
    opt.release_bucket_bytes = 1 << 40                   # one bucket, open until step()
    model(x).float().pow(2).mean().backward()
    assert opt._bucket is not None
    early = opt.state_dict()
    opt.step()
    late = opt.state_dict()
    for i in late["state"]:
        a, b = early["state"][i], late["state"][i]
        assert a["step"] == b["step"] == 1
        assert torch.equal(a["codes"], b["codes"]) and torch.equal(a["scales"], b["scales"])


@pytest.mark.parametrize("what", ["state_dict", "load_state_dict", "export_fp32"])
def test_checkpoint_and_export_wait_for_side_stream_release(what):
    """With release_streams=2 the release launches run on side streams:
    state_dict(), load_state_dict() and export_fp32() taken after backward
    with a bucket still open step it and wait for every release launch
    before touching the state, so they read (or overwrite) the state after
    the step, equal to the single-stream optimizer's.  The layers are large
    enough (4 x 4096 x 4096) that a range launch still runs when the copies
    are queued."""
    width, layers = 4096, 4
    x = torch.randn(4, width, device="cuda", dtype=torch.bfloat16,
                    generator=torch.Generator("cuda").manual_seed(15))
    runs = []
    for streams in (1, 2):
        torch.cuda.manual_seed(14)
        model = torch.nn.Sequential(*[torch.nn.Linear(width, width, bias=False, device="cuda",
                                                      dtype=torch.bfloat16)
                                      for _ in range(layers)])
        params = list(model.parameters())
        opt = make_opt("adamw", params, release=True, streams=streams)
        opt.release_bucket_bytes = 3 * width * width * 2    # closes once, one bucket stays open
        model(x).float().pow(2).mean().backward()
        if what == "state_dict":
            sd = opt.state_dict()
            runs.append([(sd["state"][i]["codes"], sd["state"][i]["scales"])
                         for i in sorted(sd["state"])])
        elif what == "export_fp32":
            runs.append([opt.export_fp32(p) for p in params])
        else:
            ckpt = {"kind": "adamw", "codes_layout": O.CODES_LAYOUT,
                    "param_groups": [dict(opt.param_groups[0], params=list(range(layers)))],
                    "state": {i: {"numel": p.numel(),
                                  "codes": torch.full_like(opt.state[p]["flash"].codes, 7),
                                  "scales": torch.full_like(opt.state[p]["flash"].scales, 9),
                                  "step": 5} for i, p in enumerate(params)}}
            opt.load_state_dict(ckpt)
            torch.cuda.synchronize()
            for i, p in enumerate(params):
                st = opt.state[p]["flash"]
                assert torch.equal(st.codes, ckpt["state"][i]["codes"]), (streams, i)
                assert torch.equal(st.scales, ckpt["state"][i]["scales"]), (streams, i)
            runs.append(None)
        torch.cuda.synchronize()
    if what == "state_dict":
        for (ca, sa), (cb, sb) in zip(*runs):
            assert torch.equal(ca, cb) and torch.equal(sa, sb)
    elif what == "export_fp32":
        for a, b in zip(*runs):
            for ta, tb in zip(a, b):
                assert torch.equal(ta, tb)
