"""The graph-capturable AdamW step (flashopt_adamw_step_scheduled): the step
counter, bias-correction powers and hyper-parameters in a device schedule.

* Called directly it equals flashopt_adamw_step with the same t, bit for bit,
  including across an lr change written into the schedule on the device.
* Captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed, with
  new gradients copied in and host synchronisations between replays, every
  replay equals the eager host-driven step.
* The scalars the schedule's kernel forms in binary64 on the device equal
  the oracle's host scalars at t from 1 to 10^6.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_adamw_state_amd import flashopt as F
from compressed_adamw_state_amd import workloads as W

from parity import log

pytestmark = pytest.mark.gpu

SIZES = [4097, 33, 2048 * 3, 1, (1 << 18) + 5]
HP = dict(W.ADAMW_HP)


def make(seed, opt="adamw"):
    w = W.ragged(SIZES, seed=seed, steps=6, optimizer=opt)
    states = []
    for i, spec in enumerate(w.tensors):
        st = F.TensorState(spec.numel, opt, "cuda")
        F.flashopt_tensor_init(st, W.draw_theta(w, i, "cuda"))
        states.append(st)
    grads = [torch.zeros(s.numel, dtype=torch.bfloat16, device="cuda") for s in states]
    return w, states, grads, F.FlashoptList(states, grads)


def same(a, b, label):
    for i, (sa, sb) in enumerate(zip(a, b)):
        assert torch.equal(sa.theta.view(torch.int16), sb.theta.view(torch.int16)), (label, i)
        assert torch.equal(sa.codes, sb.codes), (label, i)
        assert torch.equal(sa.scales, sb.scales), (label, i)


def test_scheduled_step_equals_host_step():
    w, a, ga, la = make(40)
    _, b, gb, lb = make(40)
    sched = F.DeviceSchedule(HP, t=0)
    hp = dict(HP)
    for t in range(1, 7):
        if t == 4:                                       # an lr schedule, on the device
            hp["lr"] = 3e-4
            sched.set("lr", 3e-4)
        for i in range(len(SIZES)):
            g = W.draw_grad(w, i, t, "cuda")
            ga[i].copy_(g)
            gb[i].copy_(g)
        F.flashopt_adamw_step(la, hp, t)
        F.flashopt_adamw_step_scheduled(lb, sched)
        torch.cuda.synchronize()
        same(a, b, f"step {t}")
    r = sched.read()
    assert r.t == 6 and r.lr == 3e-4


@pytest.mark.parametrize("opt", ["sgd", "lion"])
def test_scheduled_sgd_and_lion_equal_host_steps(opt):
    w, a, ga, la = make(44, opt)
    _, b, gb, lb = make(44, opt)
    hp = dict(W.HPARAMS[opt])
    sched = F.DeviceSchedule(hp, t=0, optimizer=opt)
    for t in range(1, 7):
        if t == 4:
            hp["lr"] = hp["lr"] / 3
            sched.set("lr", hp["lr"])
        if t == 5:
            k = "momentum" if opt == "sgd" else "beta1"
            hp[k] = 0.5
            sched.set(k, 0.5)
        for i in range(len(SIZES)):
            g = W.draw_grad(w, i, t, "cuda")
            ga[i].copy_(g)
            gb[i].copy_(g)
        F.step(la, opt, hp, t)
        F.step_scheduled(lb, sched)
        torch.cuda.synchronize()
        same(a, b, f"{opt} step {t}")
    assert sched.read().t == 6


def test_captured_graph_replays_equal_eager_steps():
    w, a, ga, la = make(41)
    _, b, gb, lb = make(41)
    sched = F.DeviceSchedule(HP, t=0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            F.flashopt_adamw_step_scheduled(lb, sched)
    torch.cuda.synchronize()
    assert sched.read().t == 0                           # capture ran nothing
    for t in range(1, 6):
        for i in range(len(SIZES)):                      # eager work between replays
            g = W.draw_grad(w, i, t, "cuda")
            ga[i].copy_(g)
            gb[i].copy_(g)
        torch.cuda.synchronize()
        F.flashopt_adamw_step(la, HP, t)
        graph.replay()
        torch.cuda.synchronize()
        same(a, b, f"replay {t}")
        assert sched.read().t == t
    log("graph: 5 replays equal the eager steps bit for bit")


@pytest.mark.parametrize("hp", [HP, dict(lr=3e-2, beta1=0.8, beta2=0.95, eps=1e-6,
                                         weight_decay=0.1),
                                dict(lr=1e-4, beta1=0.9, beta2=0.99999, eps=1e-30,
                                     weight_decay=0.0)])
def test_device_scalars_equal_the_host_definition(hp):
    # a list whose only tensor is empty: the call advances the schedule (its
    # one-thread kernel) and launches no step
    zero = F.FlashoptList([F.TensorState(0, "adamw", "cuda")], [None])
    for t in (1, 2, 3, 10, 100, 1000, 12345, 10 ** 6):
        sched = F.DeviceSchedule(hp, t=t - 1)
        F.flashopt_adamw_step_scheduled(zero, sched)
        r = sched.read()
        assert r.t == t
        dev = np.frombuffer(bytes(r.scalars), np.uint32)[:8].view(np.float32)
        host = oracle.adamw_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                    hp["weight_decay"], t)
        np.testing.assert_array_equal(dev.view(np.uint32), host.view(np.uint32), err_msg=str(t))


@pytest.mark.parametrize("kind", ["adamw", "sgd", "lion"])
def test_capturable_optimizer_in_a_graph(kind):
    """capturable=True: opt.step() captured once with static gradients,
    replayed every step (an lr change pushed between replays with
    update_schedules), equals the eager optimizer bit for bit; its
    checkpoint carries the device step count."""
    from compressed_adamw_state_amd import optim as O
    rng = np.random.default_rng(43)
    shapes = [(4097,), (33, 64), (2048,), (7,)]
    init = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes]
    ref = [torch.nn.Parameter(torch.from_numpy(x).cuda()) for x in init]
    cap = [torch.nn.Parameter(torch.from_numpy(x).cuda()) for x in init]
    cls, kw = {"adamw": (O.FlashAdamW, dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8,
                                            weight_decay=0.01)),
               "sgd": (O.FlashSGD, dict(lr=0.05, momentum=0.9, weight_decay=1e-4)),
               "lion": (O.FlashLion, dict(lr=1e-4, betas=(0.9, 0.99), weight_decay=0.1))}[kind]
    ro = cls(ref, **kw)
    co = cls(cap, capturable=True, **kw)
    static = [torch.zeros_like(p) for p in cap]            # BF16, like the parameters
    for p, g in zip(cap, static):
        p.grad = g
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            co.step()
    torch.cuda.synchronize()
    for t in range(1, 6):
        if t == 3:
            for o in (ro, co):
                o.param_groups[0]["lr"] = kw["lr"] / 2
            co.update_schedules()
        gs = [torch.from_numpy((rng.standard_normal(s) * 1e-3).astype(np.float32))
              .to(torch.bfloat16).cuda() for s in shapes]
        for p, g, sg in zip(ref, gs, static):
            p.grad = g.view(p.shape)
            sg.copy_(g.view(sg.shape))
        ro.step()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, cap):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), t
            sa, sb = ro.state[a]["flash"], co.state[b]["flash"]
            assert torch.equal(sa.codes, sb.codes) and torch.equal(sa.scales, sb.scales), t
    sd = co.state_dict()
    assert all(sd["state"][i]["step"] == 5 for i in range(len(cap)))
