"""Harness shared by the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on identical input bits and compare every code and scale.

Two comparison modes:
  full    -- the oracle steps every tensor (inputs drawn on the host and
             copied to the device);
  sampled -- inputs are drawn on the device; for a few 32-element groups of
             every tensor (always the first and the last group, plus random
             ones) the initial weights and each step's gradients are copied
             back, the oracle steps just those groups (groups are independent),
             and the device state at those groups is compared.
In sampled mode, step(t, every_element=True) also checks every element of
that step: the device state before the step is copied aside, and after the
GPU step the oracle steps each tensor from that copy with the step's
gradient, on the host, and every byte of the result is compared.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from compressed_adamw_state_amd import flashopt as F
from compressed_adamw_state_amd import workloads as W

GROUP = 32


def u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy().view(np.int8)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy().view(np.uint8)


def code_index(i: torch.Tensor, optimizer: str, field: int) -> torch.Tensor:
    """Byte index in `codes` of field `field` (0 rho, 1 m, 2 v) of elements i
    (include/flashopt.h): AdamW's 512-element blocks of three 512-byte
    planes, SGD's and Lion's 16-byte records of 8 elements."""
    if F.SCALES[optimizer] == 2:                           # AdamW layouts
        return (i >> 9) * 1536 + field * 512 + (i & 511)
    return (i >> 3) * 16 + field * 8 + (i & 7)


def state_fields(st: F.TensorState, idx=None, gidx=None) -> dict:
    """theta', rho, m_code, v_code (elements idx) and m_scale, v_scale (groups
    gidx) of a device TensorState as numpy arrays, read out of the code
    planes or records and the scale pairs (include/flashopt.h); None selects
    all."""
    dev = st.codes.device
    n = st.numel
    if idx is None:
        idx = torch.arange(n, device=dev)
    if gidx is None:
        gidx = torch.arange((n + GROUP - 1) // GROUP, device=dev)
    S, opt = F.SCALES[st.optimizer], st.optimizer
    out = {"theta": u16(st.theta[idx]), "rho": i8(st.codes[code_index(idx, opt, 0)]),
           "m_code": i8(st.codes[code_index(idx, opt, 1)]), "m_scale": u16(st.scales[gidx * S])}
    if S == 2:                                             # AdamW layouts
        out["v_code"] = u8(st.codes[code_index(idx, opt, 2)])
        out["v_scale"] = u16(st.scales[gidx * S + 1])
    return out


def record_fields(theta: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, n: int,
                  optimizer: str) -> dict:
    """theta', rho, m_code, v_code, m_scale, v_scale of one tensor from its
    device arrays (live state or a copy), unpacked from the code planes or
    records on the device and returned as contiguous host arrays."""
    S = F.SCALES[optimizer]
    ng = (n + GROUP - 1) // GROUP
    if S == 2:                                             # AdamW: [block][field][512]
        nblk = (n + 511) // 512
        fld = codes[:nblk * 1536].view(nblk, 3, 512)
    else:                                                  # SGD, Lion: [record][field][8]
        nrec = (n + 7) // 8
        fld = codes[:nrec * 16].view(nrec, 2, 8)
    sc = scales[:ng * S].view(ng, S)
    out = {"theta": u16(theta[:n]), "rho": i8(fld[:, 0].reshape(-1)[:n]),
           "m_code": i8(fld[:, 1].reshape(-1)[:n]), "m_scale": u16(sc[:, 0])}
    if S == 2:
        out["v_code"] = u8(fld[:, 2].reshape(-1)[:n])
        out["v_scale"] = u16(sc[:, 1])
    return out


def oracle_state(fields: dict, n: int, optimizer: str) -> oracle.State:
    """An oracle State holding the given fields (host arrays, stepped in place)."""
    o = oracle.State.__new__(oracle.State)
    o.n, o.optimizer = n, optimizer
    o.tb, o.rho, o.qm, o.sm = fields["theta"], fields["rho"], fields["m_code"], fields["m_scale"]
    o.qv, o.sv = fields.get("v_code"), fields.get("v_scale")
    return o


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class Run:
    def __init__(self, w: W.Workload, mode: str = "full", samples_per_tensor: int = 4,
                 seed: int = 0, extra_groups=()):
        """extra_groups: group indices compared in every tensor that has them
        (sampled mode), besides the first, the last and random ones."""
        assert mode in ("full", "sampled")
        self.w, self.mode = w, mode
        self.dev = torch.device("cuda")
        self.gen_dev = "cpu" if mode == "full" else "cuda"
        opt = w.optimizer
        rng = np.random.default_rng(seed)
        self.states, self.grads, self.orc, self.samples = [], [], [], []
        # the state and one gradient set in one StateArena, as bench.py lays them out
        arena = F.StateArena([spec.numel for spec in w.tensors], opt, self.dev, theta=True,
                             grad_sets=1)
        for i, spec in enumerate(w.tensors):
            n = spec.numel
            theta = W.draw_theta(w, i, self.gen_dev)
            st = arena.state(i)
            theta_d = theta.to(self.dev)
            F.flashopt_tensor_init(st, theta_d)
            self.states.append(st)
            self.grads.append(arena.grad(0, i))
            if mode == "full":
                self.orc.append(oracle.State(theta.numpy(), opt))
            else:
                ng = (n + GROUP - 1) // GROUP
                pick = {0, ng - 1} | set(rng.integers(0, ng, samples_per_tensor).tolist()) \
                    | set(extra_groups)
                pick = sorted(g for g in pick if 0 <= g < ng)
                self.samples.append(pick)
                idx = torch.cat([torch.arange(g * GROUP, min(n, g * GROUP + GROUP))
                                 for g in pick]).to(self.dev)
                host = theta_d[idx].cpu().numpy()
                per = []
                off = 0
                for g in pick:
                    ln = min(n, g * GROUP + GROUP) - g * GROUP
                    per.append(oracle.State(host[off:off + ln], opt))
                    off += ln
                self.orc.append(per)
            del theta_d
        self.lst = F.FlashoptList(self.states, self.grads)
        F.flashopt_state_zero(self.lst)
        torch.cuda.synchronize()

    def _sample_index(self, i):
        n = self.w.tensors[i].numel
        return torch.cat([torch.arange(g * GROUP, min(n, g * GROUP + GROUP))
                          for g in self.samples[i]]).to(self.dev)

    def step(self, t: int, hp: dict | None = None, threads: int | None = None,
             every_element: bool = False) -> int:
        """GPU step t (and the oracle on the compared groups); with
        every_element, also the every-element check of this step (returns the
        number of elements it compared)."""
        w = self.w
        hp = hp or w.hparams
        snap = None
        if every_element:
            assert self.mode == "sampled"
            snap = [(st.theta.clone(), st.codes.clone(), st.scales.clone()) for st in self.states]
        grads = []
        for i in range(len(w.tensors)):
            g = W.draw_grad(w, i, t, self.gen_dev)
            self.grads[i].copy_(g)
            grads.append(self.grads[i])
            if self.mode == "full":
                oracle.step_chunked(self.orc[i], u16(g), t, hp, nthreads=threads)
            else:
                gs = u16(grads[i][self._sample_index(i)])
                off = 0
                for st in self.orc[i]:
                    oracle.step(st, gs[off:off + st.n], t, hp)
                    off += st.n
        if w.release:
            for i in reversed(range(len(w.tensors))):        # backward order
                F.step_one(self.lst, w.optimizer, i, grads[i], hp, t)
        else:
            F.step(self.lst, w.optimizer, hp, t)
        torch.cuda.synchronize()
        self.t = t
        if snap is None:
            return 0
        checked = 0
        for i, st in enumerate(self.states):
            n = st.numel
            pre = record_fields(*snap[i], n, st.optimizer)
            snap[i] = None                                   # free the device copy
            o = oracle_state(pre, n, st.optimizer)
            oracle.step_chunked(o, u16(grads[i]), t, hp, nthreads=threads)
            post = record_fields(st.theta, st.codes, st.scales, n, st.optimizer)
            keys = [("theta", "tb"), ("rho", "rho"), ("m_code", "qm"), ("m_scale", "sm")]
            if "v_code" in post:
                keys += [("v_code", "qv"), ("v_scale", "sv")]
            for k, ok in keys:
                got, exp = post[k], getattr(o, ok)
                if not np.array_equal(got, exp):
                    bad = np.nonzero(got != exp)[0]
                    raise AssertionError(
                        f"every element, step {t}: tensor {i} ({w.tensors[i].name}) {k}: "
                        f"{bad.size} mismatches, first at {bad[:5].tolist()}: gpu "
                        f"{got[bad[:5]].tolist()} oracle {exp[bad[:5]].tolist()}")
            checked += n
        return checked

    def advance_to(self, t: int, compare_every: int = 0, label: str = "") -> None:
        """Steps self.t + 1 .. t (sampled comparisons every compare_every
        steps when it is positive)."""
        for k in range(getattr(self, "t", 0) + 1, t + 1):
            self.step(k)
            if compare_every and k % compare_every == 0:
                n = self.compare(f"{label} step {k}")
                log(f"{label} step {k}: {n} sampled elements compared")

    def compare(self, label: str = "") -> int:
        """Assert bit equality of every compared code and scale; return #elements."""
        checked = 0
        for i, st in enumerate(self.states):
            name = self.w.tensors[i].name
            keys = [("theta", "tb"), ("rho", "rho"), ("m_code", "qm"), ("m_scale", "sm")]
            if st.optimizer in ("adamw", "adamw_linv"):
                keys += [("v_code", "qv"), ("v_scale", "sv")]
            if self.mode == "full":
                o = self.orc[i]
                f = state_fields(st)
                pairs = [(k, f[k], getattr(o, ok)) for k, ok in keys]
                checked += st.numel
            else:
                idx = self._sample_index(i)
                gidx = torch.tensor(self.samples[i], device=self.dev)
                f = state_fields(st, idx, gidx)
                cat = lambda k: np.concatenate([getattr(s, k) for s in self.orc[i]])
                pairs = [(k, f[k], cat(ok)) for k, ok in keys]
                checked += int(idx.numel())
            for k, got, exp in pairs:
                if not np.array_equal(got, exp):
                    bad = np.nonzero(got != exp)[0]
                    raise AssertionError(
                        f"{label} tensor {i} ({name}) {k}: {bad.size} mismatches, first at "
                        f"{bad[:5].tolist()}: gpu {got[bad[:5]].tolist()} oracle "
                        f"{exp[bad[:5]].tolist()}")
        return checked
