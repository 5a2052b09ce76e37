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


def state_fields(st: F.TensorState, idx=None, gidx=None) -> dict:
    """theta', rho, m_code, v_code (elements idx) and m_scale, v_scale (groups
    gidx) of a device TensorState as numpy arrays, read out of the interleaved
    code records and scale pairs (include/flashopt.h); None selects all."""
    dev = st.codes.device
    n = st.numel
    if idx is None:
        idx = torch.arange(n, device=dev)
    if gidx is None:
        gidx = torch.arange((n + GROUP - 1) // GROUP, device=dev)
    R, S = F.RECORD[st.optimizer], F.SCALES[st.optimizer]
    base = (idx >> 3) * R + (idx & 7)
    out = {"theta": u16(st.theta[idx]), "rho": i8(st.codes[base]),
           "m_code": i8(st.codes[base + 8]), "m_scale": u16(st.scales[gidx * S])}
    if S == 2:                                             # AdamW layouts
        out["v_code"] = u8(st.codes[base + 16])
        out["v_scale"] = u16(st.scales[gidx * S + 1])
    return out


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
        # the state in one StateArena, as bench.py lays it out
        arena = F.StateArena([spec.numel for spec in w.tensors], opt, self.dev)
        for i, spec in enumerate(w.tensors):
            n = spec.numel
            theta = W.draw_theta(w, i, self.gen_dev)
            st = arena.state(i)
            theta_d = theta.to(self.dev)
            F.flashopt_tensor_init(st, theta_d)
            self.states.append(st)
            self.grads.append(None if w.release else
                              torch.zeros(n, dtype=torch.bfloat16, device=self.dev))
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

    def step(self, t: int, hp: dict | None = None, threads: int | None = None):
        w = self.w
        hp = hp or w.hparams
        grads = []
        for i in range(len(w.tensors)):
            g = W.draw_grad(w, i, t, self.gen_dev)
            if w.release:
                grads.append(g.to(self.dev))
            else:
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
