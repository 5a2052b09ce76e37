"""GPU parity of the uncompressed state kinds (compression switched off for a
layer: FP32 master weight and moments, FlashOptim page "Practical advice")
with the oracle's FP32 steps, bit for bit: whole ragged lists, gradient
release, init / export / zero, a tensor past 2^31 elements, and the drop-in
optimizers with one parameter group left uncompressed."""
import numpy as np
import pytest
import torch

import oracle
from compressed_adamw_state_amd import flashopt as F
from compressed_adamw_state_amd import optim as O
from compressed_adamw_state_amd import workloads as W

from parity import log, u16

pytestmark = pytest.mark.gpu

RAGGED = [1, 7, 8, 9, 31, 33, 511, 512, 513, 1023, 1536, 2047, 2048, 2049, 2560, 4095, 4097,
          6143, 32 * 777 + 5, (1 << 20) + 7, 0, 64]
HP = W.HPARAMS


def fp32_fields(st: F.TensorState, idx=None):
    """theta (FP32 master), m, v (AdamW) of elements idx, read out of the
    512-element blocks of FP32 fields (include/flashopt.h)."""
    nf = F.FP32_FIELDS[st.optimizer]
    words = st.codes.view(torch.float32)
    if idx is None:
        idx = torch.arange(st.numel, device=st.codes.device)
    base = (idx >> 9) * (512 * nf) + (idx & 511)
    out = {"theta": words[base].cpu().numpy(), "m": words[base + 512].cpu().numpy()}
    if st.optimizer == "adamw_fp32":
        out["v"] = words[base + 1024].cpu().numpy()
    return out


def compare(states, orcs, label):
    for i, (st, o) in enumerate(zip(states, orcs)):
        if st.numel == 0:
            continue
        f = fp32_fields(st)
        np.testing.assert_array_equal(u16(st.theta), o.tb, err_msg=f"{label} tensor {i} theta'")
        np.testing.assert_array_equal(f["theta"].view(np.uint32), o.theta.view(np.uint32),
                                      err_msg=f"{label} tensor {i} theta")
        np.testing.assert_array_equal(f["m"].view(np.uint32), o.m.view(np.uint32),
                                      err_msg=f"{label} tensor {i} m")
        if o.v is not None:
            np.testing.assert_array_equal(f["v"].view(np.uint32), o.v.view(np.uint32),
                                          err_msg=f"{label} tensor {i} v")


def make(opt, sizes, seed):
    w = W.ragged(sizes, seed=seed, steps=3, optimizer=opt)
    kind = opt + "_fp32"
    states, orcs = [], []
    for i, spec in enumerate(w.tensors):
        theta = W.draw_theta(w, i, "cpu")
        st = F.TensorState(spec.numel, kind, "cuda")
        F.flashopt_tensor_init(st, theta.cuda())
        states.append(st)
        orcs.append(oracle.StateFP32(theta.numpy(), opt))
    return w, states, orcs


def grads_of(w, t):
    return [W.draw_grad(w, i, t, "cpu") for i in range(len(w.tensors))]


def gbits(g):
    return g.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("opt", ["adamw", "sgd", "lion"])
def test_fp32_ragged_list_every_step(opt):
    w, states, orcs = make(opt, RAGGED, seed=31)
    compare(states, orcs, "init")
    grads = grads_of(w, 1)
    lst = F.FlashoptList(states, [g.cuda() for g in grads], optimizer=opt + "_fp32")
    for t in range(1, 4):
        grads = grads_of(w, t)
        dg = [g.cuda() for g in grads]
        F.flashopt_list_set_grads(lst, dg)
        F.step(lst, opt, HP[opt], t)
        for o, g in zip(orcs, grads):
            oracle.step_fp32(o, gbits(g), t, HP[opt])
        torch.cuda.synchronize()
        compare(states, orcs, f"{opt} step {t}")


@pytest.mark.parametrize("opt", ["adamw", "lion"])
def test_fp32_release_equals_list(opt):
    w, a, _ = make(opt, RAGGED[:14], seed=32)
    _, b, orcs = make(opt, RAGGED[:14], seed=32)
    la = F.FlashoptList(a, [None] * len(a), optimizer=opt + "_fp32")
    lb = F.FlashoptList(b, [None] * len(b), optimizer=opt + "_fp32")
    for t in (1, 2):
        grads = [g.cuda() for g in grads_of(w, t)]
        F.flashopt_list_set_grads(la, grads)
        F.step(la, opt, HP[opt], t)
        for i in reversed(range(len(b))):                # backward order
            F.step_one(lb, opt, i, grads[i], HP[opt], t)
    torch.cuda.synchronize()
    for sa, sb in zip(a, b):
        assert torch.equal(sa.codes, sb.codes) and torch.equal(sa.theta.view(torch.int16),
                                                                sb.theta.view(torch.int16))


def test_fp32_init_export_zero():
    w, states, orcs = make("adamw", [4097, 33, 0], seed=33)
    lst = F.FlashoptList(states, [g.cuda() for g in grads_of(w, 1)], optimizer="adamw_fp32")
    F.step(lst, "adamw", HP["adamw"], 1)
    for o, g in zip(orcs, grads_of(w, 1)):
        oracle.step_fp32(o, gbits(g), 1, HP["adamw"])
    for st, o in zip(states, orcs):
        th, m, v = (torch.empty(st.numel, device="cuda") for _ in range(3))
        F.flashopt_tensor_export(st, th, m, v)
        for a, b in ((th, o.theta), (m, o.m), (v, o.v)):
            np.testing.assert_array_equal(a.cpu().numpy().view(np.uint32), b.view(np.uint32))
    F.flashopt_state_zero(lst)
    torch.cuda.synchronize()
    for st, o in zip(states, orcs):
        if st.numel == 0:
            continue
        f = fp32_fields(st)
        assert not f["m"].any() and not f["v"].any()
        np.testing.assert_array_equal(f["theta"].view(np.uint32), o.theta.view(np.uint32))


def test_fp32_kinds_host_checks():
    st = F.TensorState(100, "adamw_fp32", "cuda")
    assert st.scales.numel() == 0 and st.codes.numel() == 512 * 4 * 3
    d = st.descriptor()
    assert d.scales is None
    lst = F.FlashoptList([st], [None], optimizer="adamw_fp32")
    with pytest.raises(F.FlashoptError):                 # an SGD step on an AdamW list
        F.flashopt_sgd_step(lst, HP["sgd"], 1)
    with pytest.raises(F.FlashoptError):                 # the probe is for compressed AdamW
        F.flashopt_stream_probe(lst)


@pytest.mark.parametrize("opt", ["adamw"])
def test_fp32_tensor_beyond_2_to_31_elements(opt):
    """One tensor past 32-bit element indices and 2^32 record bytes; the FP32
    step is elementwise, so the oracle steps sampled elements alone."""
    n = (1 << 31) + (1 << 20) + 7
    st = F.TensorState(n, opt + "_fp32", "cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(41)
    theta = torch.randn(n, generator=gen, device="cuda") * 0.02
    F.flashopt_tensor_init(st, theta)
    del theta
    rng = np.random.default_rng(41)
    idx = np.unique(np.concatenate([np.arange(8), np.arange(n - 13, n),
                                    np.arange((1 << 31) - 9, (1 << 31) + 9),
                                    rng.integers(0, n, 64)]))
    ti = torch.from_numpy(idx).cuda()
    f = fp32_fields(st, ti)
    o = oracle.StateFP32(f["theta"], opt)
    lst = F.FlashoptList([st], [None], optimizer=opt + "_fp32")
    for t in (1, 2):
        g = (torch.randn(n, generator=gen, device="cuda") * 1e-3).to(torch.bfloat16)
        F.flashopt_list_set_grads(lst, [g])
        F.step(lst, opt, HP[opt], t)
        oracle.step_fp32(o, u16(g[ti]), t, HP[opt])
        del g
        f = fp32_fields(st, ti)
        np.testing.assert_array_equal(f["theta"].view(np.uint32), o.theta.view(np.uint32))
        np.testing.assert_array_equal(f["m"].view(np.uint32), o.m.view(np.uint32))
        np.testing.assert_array_equal(f["v"].view(np.uint32), o.v.view(np.uint32))
        np.testing.assert_array_equal(u16(st.theta[ti]), o.tb)
    log(f"fp32 tensor of {n} elements: {idx.size} sampled elements compared")


@pytest.mark.parametrize("kind", ["adamw", "sgd", "lion"])
def test_optimizer_with_an_uncompressed_group(kind):
    """The drop-in optimizer with one parameter group left uncompressed: the
    compressed group matches the compressed oracle, the other the FP32
    oracle, and a checkpoint of both resumes bit for bit."""
    hp = {"adamw": dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01),
          "sgd": dict(lr=0.05, momentum=0.9, weight_decay=1e-4),
          "lion": dict(lr=1e-4, betas=(0.9, 0.99), weight_decay=0.1)}[kind]
    ohp = {"adamw": dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
           "sgd": dict(lr=0.05, momentum=0.9, weight_decay=1e-4),
           "lion": dict(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.1)}[kind]
    cls = {"adamw": O.FlashAdamW, "sgd": O.FlashSGD, "lion": O.FlashLion}[kind]
    rng = np.random.default_rng(34)
    shapes_c, shapes_u = [(4097,), (33, 64)], [(768,), (7,)]
    init_c = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes_c]
    init_u = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes_u]

    def build():
        pc = [torch.nn.Parameter(torch.from_numpy(x).cuda()) for x in init_c]
        pu = [torch.nn.Parameter(torch.from_numpy(x).cuda()) for x in init_u]
        opt = cls([{"params": pc}, {"params": pu, "compress": False}], **hp)
        return pc, pu, opt

    pc, pu, opt = build()
    assert all(p.dtype == torch.bfloat16 for p in pc + pu)
    oc = [oracle.State(x.reshape(-1), kind) for x in init_c]
    ou = [oracle.StateFP32(x.reshape(-1), kind) for x in init_u]
    grads = [[(rng.standard_normal(p.shape) * 1e-3).astype(np.float32) for p in pc + pu]
             for _ in range(4)]
    for t in (1, 2):
        for p, g in zip(pc + pu, grads[t - 1]):
            p.grad = torch.from_numpy(g).to(torch.bfloat16).cuda()
        opt.step()
        for o, p in zip(oc + ou, pc + pu):
            gb = u16(p.grad.view(-1))
            (oracle.step if isinstance(o, oracle.State) else oracle.step_fp32)(o, gb, t, ohp)
    torch.cuda.synchronize()
    for p, o in zip(pc, oc):
        np.testing.assert_array_equal(u16(p.data.view(-1)), o.tb)
    for p, o in zip(pu, ou):
        np.testing.assert_array_equal(u16(p.data.view(-1)), o.tb)
        th, m, _ = opt.export_fp32(p)
        np.testing.assert_array_equal(th.cpu().numpy().view(np.uint32), o.theta.view(np.uint32))
        np.testing.assert_array_equal(m.cpu().numpy().view(np.uint32), o.m.view(np.uint32))
    # checkpoint after two steps, resume in a fresh optimizer, two more steps
    sd = opt.state_dict()
    weights = [p.detach().clone() for p in pc + pu]
    pc2 = [torch.nn.Parameter(w) for w in weights[:2]]
    pu2 = [torch.nn.Parameter(w) for w in weights[2:]]
    opt2 = cls([{"params": pc2}, {"params": pu2, "compress": False}], **hp)
    opt2.load_state_dict(sd)
    for t in (3, 4):
        for ps in ((pc, pu), (pc2, pu2)):
            for p, g in zip(ps[0] + ps[1], grads[t - 1]):
                p.grad = torch.from_numpy(g).to(torch.bfloat16).cuda()
        opt.step()
        opt2.step()
    torch.cuda.synchronize()
    for a, b in zip(pc + pu, pc2 + pu2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        sa, sb = opt.state[a]["flash"], opt2.state[b]["flash"]
        assert torch.equal(sa.codes, sb.codes) and torch.equal(sa.scales, sb.scales)
