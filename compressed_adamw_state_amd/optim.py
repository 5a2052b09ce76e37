"""Drop-in optimizers over the fused compressed step: FlashAdamW, FlashSGD,
FlashLion ("FlashOptim: Optimizers for Memory Efficient Training", Practical
advice: replace the standard optimizer, keep the hyper-parameters).

Each parameter's BF16 data is theta' -- the weight the model computes with
-- and the optimizer keeps, per parameter, the codes (rho, momentum and, for
AdamW, variance codes) and the FP16 group scales in the layout of
include/flashopt.h.  A parameter given in FP32 is split once at
construction: its data becomes the BF16 theta' and rho keeps the rest of the
FP32 value.  Every step is one launch of the library's fused kernel per
parameter group (or, with gradient release, one launch per parameter from
its gradient hook, after which the gradient is dropped; with
release_bucket_bytes > 0, one launch per bucket of consecutive parameters
whose gradients arrived one after another, once the bucket holds that many
bytes of gradients, the last bucket at step()).  Gradient release steps at
every backward pass, so it is for training without gradient accumulation
over micro-batches (as the page's practical advice puts it).  As in torch.optim,
a parameter whose gradient is None is skipped and every parameter keeps its
own step count; a group where that leaves parameters out, or where the
counts differ, is stepped by one launch per parameter.

state_dict() holds the codes and scales (3.125 B/param for AdamW, 2.0625
for SGD and Lion) plus each parameter's step count; with theta' saved as
the model's own BF16 weights, an AdamW checkpoint is 5.125 B/param (the
page's 12 -> 5 B/param).  Loading it into a fresh optimizer resumes bit for
bit.

capturable=True keeps each group's step counter and hyper-parameters in a
device schedule (flashopt_*_step_scheduled), so step() can be captured in a
HIP graph (torch.cuda.graph) and replayed; update_schedules() pushes
changed hyper-parameters between replays (AdamW's betas stay fixed).  A
replay reads the gradients at the addresses captured, so they must stay
static (zero_grad(set_to_none=False)).

A parameter group with "compress": False (the page's practical advice:
compression can be switched off for layers that are sensitive to it) keeps
an FP32 master weight and FP32 moments instead (the library's _fp32 state
kinds, 14 B/param for AdamW); its parameters still compute in BF16, and the
group is stepped by the same kind of launch.  "linear_variance": True (AdamW
only) stores the variance with linear codes instead of square-root
companding -- the ablation of the page's Fig. 5, for experiments, not for
training.

This module only marshals: every arithmetic operation of the update runs in
the HIP library, and there is no fallback.
"""
from __future__ import annotations

from typing import Iterable, List, Optional

import torch

from . import flashopt as F

# Placement of the codes in a checkpoint's "codes" tensors (include/flashopt.h):
# "blocks512" -- AdamW's rho, m and v planes per 512-element block, SGD's and
# Lion's 16-byte records of 8 elements; the _FP32 kinds' FP32 field blocks.
CODES_LAYOUT = "blocks512"


class _FlashOptimizer(torch.optim.Optimizer):
    kind = ""                                    # "adamw" | "sgd" | "lion"

    def __init__(self, params, defaults: dict, gradient_release: bool = False,
                 release_streams: int = 1, release_bucket_bytes: int = 0,
                 capturable: bool = False):
        super().__init__(params, defaults)
        self.gradient_release = gradient_release
        self.capturable = capturable
        # release_bucket_bytes > 0: consecutive parameters of a group whose
        # gradients arrive one after another are stepped by one launch
        # (flashopt_*_step_range) once their gradients reach this many bytes;
        # the gradients of a bucket stay alive until its launch
        self.release_bucket_bytes = int(release_bucket_bytes)
        self._bucket = None
        if capturable and gradient_release:
            raise ValueError("capturable and gradient_release do not combine")
        # with release_streams > 1 the launches from the gradient hooks (per
        # parameter or per bucket) go round-robin over that many side streams
        # (default priority): each overlaps the rest of backward and the tail
        # of the previous one
        self._side = [torch.cuda.Stream() for _ in range(release_streams)] \
            if gradient_release and release_streams > 1 else []
        self._rr = 0
        self._lists: List[Optional[F.FlashoptList]] = []
        self._hooks = []
        for group in self.param_groups:
            self._init_params(group["params"], self._state_kind(group))
        self._build_lists()
        # capturable: per group, the step counter and hyper-parameters in a
        # device schedule, so step() launches nothing that depends on host
        # values and can be captured in a HIP graph
        self._sched: List[Optional[F.DeviceSchedule]] = []
        self._sched_hp: List[dict] = []
        if capturable:
            for group, lst in zip(self.param_groups, self._lists):
                if self._state_kind(group) != self.kind:
                    raise ValueError("capturable needs the compressed state in every group")
                self._sched.append(F.DeviceSchedule(self._hp(group), t=0, optimizer=self.kind)
                                   if lst else None)
                self._sched_hp.append(self._hp(group))
        if gradient_release:
            self._install_release_hooks()
        self._ready = True

    def add_param_group(self, param_group: dict) -> None:
        """torch.optim's add_param_group; after construction the new group's
        parameters get their compressed state, list, schedule and hooks."""
        super().add_param_group(param_group)
        if not getattr(self, "_ready", False):
            return                               # during __init__: set up there
        gi = len(self.param_groups) - 1
        group = self.param_groups[gi]
        kind = self._state_kind(group)
        self._init_params(group["params"], kind)
        states = [self.state[p]["flash"] for p in group["params"]]
        lst = F.FlashoptList(states, [None] * len(states), optimizer=kind) if states else None
        self._lists.append(lst)
        if self.capturable:
            if kind != self.kind:
                raise ValueError("capturable needs the compressed state in every group")
            self._sched.append(F.DeviceSchedule(self._hp(group), t=0, optimizer=self.kind)
                               if lst else None)
            self._sched_hp.append(self._hp(group))
        if self.gradient_release:
            for pi, p in enumerate(group["params"]):
                self._install_release_hook(gi, pi, p)

    # -- state -----------------------------------------------------------------
    def _state_kind(self, group) -> str:
        if not group.get("compress", True):
            return self.kind + "_fp32"
        if group.get("linear_variance", False):
            if self.kind != "adamw":
                raise ValueError("linear_variance applies to FlashAdamW only")
            return "adamw_linv"
        return self.kind

    def _init_params(self, params, kind: str) -> None:
        """Compressed state for one group's parameters: per device, their code
        records and scales are slices of one buffer each (F.StateArena)."""
        for p in params:
            if not p.is_cuda:
                raise ValueError("FlashOptim parameters must live on the GPU")
            if p.dtype not in (torch.float32, torch.bfloat16):
                raise ValueError(f"unsupported parameter dtype {p.dtype}")
            if p.dtype == torch.bfloat16 and not p.is_contiguous():
                raise ValueError("BF16 parameters must be contiguous")
        by_device = {}
        for p in params:
            by_device.setdefault(p.device, []).append(p)
        for device, ps in by_device.items():
            # FP32 parameters get their BF16 theta' from the arena (one region for
            # theta', one for the codes, one for the scales); BF16 parameters
            # keep their own storage as theta'
            arena = F.StateArena([p.numel() for p in ps], kind, device,
                                 theta=all(p.dtype == torch.float32 for p in ps))
            for i, p in enumerate(ps):
                if p.dtype == torch.float32:
                    st = arena.state(i)
                    F.flashopt_tensor_init(st, p.detach().reshape(-1).contiguous())
                    p.data = st.theta.view(p.shape)   # the model now computes with theta'
                else:
                    # theta' is the parameter's own storage; the split of its exact
                    # FP32 value rewrites the same BF16 bits and gives rho = 0
                    st = arena.state(i, theta=p.data.view(-1))
                    F.flashopt_tensor_init(st, p.detach().reshape(-1).float())
                self.state[p]["flash"] = st
                self.state[p]["step"] = 0        # this parameter's own t (as in torch.optim)

    def _build_lists(self) -> None:
        self._lists = []
        for group in self.param_groups:
            states = [self.state[p]["flash"] for p in group["params"]]
            grads = [None] * len(states)
            self._lists.append(F.FlashoptList(states, grads, optimizer=self._state_kind(group))
                               if states else None)

    def _hp(self, group) -> dict:
        raise NotImplementedError

    # -- the step ----------------------------------------------------------------
    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        if self.gradient_release:
            # the hooks already stepped every parameter of this iteration (a
            # last bucket is stepped now); the next forward must see their
            # updates
            self._join_release()
            return loss
        if self.capturable:
            self._step_scheduled()
            return loss
        for group, lst in zip(self.param_groups, self._lists):
            if lst is None:
                continue
            params = group["params"]
            for p in params:
                g = p.grad
                if g is not None and (g.dtype != torch.bfloat16 or not g.is_contiguous()):
                    raise ValueError("FlashOptim expects contiguous BF16 gradients")
            steps = {self.state[p]["step"] for p in params}
            if all(p.grad is not None for p in params) and len(steps) == 1:
                # the common case: one launch over the whole group
                t = steps.pop() + 1
                F.flashopt_list_set_grads(lst, [p.grad.view(-1) for p in params])
                F.step(lst, self.kind, self._hp(group), t)
                # the list keeps no gradient after the launch, so zero_grad()
                # frees them as with any torch optimizer (stream-ordered: the
                # memory is reused only after the launch has run)
                F.flashopt_list_set_grads(lst, [None] * len(params))
                for p in params:
                    self.state[p]["step"] = t
            else:
                # as torch.optim: a parameter without a gradient is skipped, and
                # each parameter keeps its own step count (bias correction)
                for i, p in enumerate(params):
                    if p.grad is None:
                        continue
                    t = self.state[p]["step"] + 1
                    F.step_one(lst, self.kind, i, p.grad.view(-1), self._hp(group), t)
                    self.state[p]["step"] = t
        return loss

    def update_schedules(self) -> None:
        """capturable: write changed hyper-parameters of the param groups
        into their device schedules.  step() does this itself when it
        runs eagerly; a replayed graph does not run step()'s host code, so
        call this (outside the graph) after changing hyper-parameters."""
        for i, (group, sched) in enumerate(zip(self.param_groups, self._sched)):
            if sched is None:
                continue
            hp = self._hp(group)
            settable = F.DeviceSchedule.SETTABLE[self.kind]
            for k, v in hp.items():
                if v == self._sched_hp[i][k]:
                    continue
                if k not in settable:
                    raise ValueError(f"{k} is fixed in a capturable {self.kind} schedule")
                sched.set(k, v)
            self._sched_hp[i] = hp

    def _step_scheduled(self) -> None:
        if not torch.cuda.is_current_stream_capturing():
            self.update_schedules()
        for group, lst, sched in zip(self.param_groups, self._lists, self._sched):
            if lst is None:
                continue
            grads = []
            for p in group["params"]:
                g = p.grad
                if g is None:
                    raise ValueError("capturable: every parameter needs a gradient at each step")
                if g.dtype != torch.bfloat16 or not g.is_contiguous():
                    raise ValueError("FlashOptim expects contiguous BF16 gradients")
                grads.append(g.view(-1))
            F.flashopt_list_set_grads(lst, grads)
            F.step_scheduled(lst, sched)

    def _install_release_hooks(self) -> None:
        for gi, group in enumerate(self.param_groups):
            for pi, p in enumerate(group["params"]):
                self._install_release_hook(gi, pi, p)

    def _install_release_hook(self, gi: int, pi: int, p: torch.Tensor) -> None:
        def hook(param, gi=gi, pi=pi):
            g = param.grad
            if g.dtype != torch.bfloat16 or not g.is_contiguous():
                raise ValueError("FlashOptim expects contiguous BF16 gradients")
            if self.release_bucket_bytes > 0:
                self._add_to_bucket(gi, pi, param, g)
                return
            stream = self._release_stream([g])
            t = self.state[param]["step"] + 1
            F.step_one(self._lists[gi], self.kind, pi, g.view(-1),
                       self._hp(self.param_groups[gi]), t, stream)
            self.state[param]["step"] = t
            param.grad = None            # gradient release: 2 B/param freed early
        self._hooks.append(p.register_post_accumulate_grad_hook(hook))

    def _release_stream(self, grads):
        """The stream a release launch goes on: the current one, or the next
        side stream (made to wait for the current one, which produced the
        gradients; they are recorded on it so they outlive their release).
        A hook fires once every backward node that read its parameter has
        run, so updating the parameter concurrently with the rest of
        backward is safe."""
        if not self._side:
            return None
        stream = self._side[self._rr % len(self._side)]
        self._rr += 1
        stream.wait_stream(torch.cuda.current_stream())
        for g in grads:
            g.record_stream(stream)
        return stream

    def _add_to_bucket(self, gi: int, pi: int, param, g) -> None:
        t = self.state[param]["step"] + 1
        b = self._bucket
        if b is not None and not (b["gi"] == gi and b["t"] == t and
                                  (pi == b["lo"] - 1 or pi == b["hi"] + 1)):
            self._flush_bucket()
            b = None
        if b is None:
            b = self._bucket = {"gi": gi, "t": t, "lo": pi, "hi": pi, "grads": {}, "bytes": 0}
        b["lo"], b["hi"] = min(b["lo"], pi), max(b["hi"], pi)
        b["grads"][pi] = g.view(-1)
        b["bytes"] += 2 * g.numel()
        self.state[param]["step"] = t
        param.grad = None                # the bucket holds the gradient until its launch
        if b["bytes"] >= self.release_bucket_bytes:
            self._flush_bucket()

    def _join_release(self) -> None:
        """Step a release bucket still open, then make the current stream
        wait for every release launch issued so far (on the side streams
        too): work queued on the current stream afterwards -- the next
        forward, a checkpoint's copies, an export -- sees the updated state,
        and no release launch still running can overwrite what it writes."""
        self._flush_bucket()
        cur = torch.cuda.current_stream()
        for s in self._side:
            cur.wait_stream(s)

    def _flush_bucket(self) -> None:
        b, self._bucket = self._bucket, None
        if b is None:
            return
        grads = [b["grads"][i] for i in range(b["lo"], b["hi"] + 1)]
        stream = self._release_stream(grads)
        gi = b["gi"]
        F.step_range(self._lists[gi], self.kind, b["lo"], grads, self._hp(self.param_groups[gi]),
                     b["t"], stream)

    # -- checkpoints -------------------------------------------------------------
    def _sync_steps(self) -> None:
        """capturable: the step counts live in the device schedules."""
        for group, sched in zip(self.param_groups, self._sched):
            if sched is not None:
                t = sched.read().t
                for p in group["params"]:
                    self.state[p]["step"] = t

    def state_dict(self) -> dict:
        self._join_release()             # an open release bucket belongs to this state
        if self.capturable:
            self._sync_steps()
        sd = {"kind": self.kind, "codes_layout": CODES_LAYOUT, "param_groups": [], "state": {}}
        index = 0
        for group in self.param_groups:
            g = {k: v for k, v in group.items() if k != "params"}
            g["params"] = []
            for p in group["params"]:
                st = self.state[p]["flash"]
                sd["state"][index] = {"numel": st.numel, "codes": st.codes.clone(),
                                      "scales": st.scales.clone(),
                                      "step": self.state[p]["step"]}
                g["params"].append(index)
                index += 1
            sd["param_groups"].append(g)
        return sd

    def load_state_dict(self, sd: dict) -> None:
        self._join_release()             # stepped and finished, then overwritten below
        if sd.get("kind") != self.kind:
            raise ValueError(f"checkpoint is for {sd.get('kind')}, not {self.kind}")
        if sd.get("codes_layout") != CODES_LAYOUT:
            # same byte counts can hold differently placed codes: refuse, do not reinterpret
            raise ValueError(f"checkpoint codes layout {sd.get('codes_layout')!r} is not "
                             f"{CODES_LAYOUT!r}")
        saved = sd["param_groups"]
        if len(saved) != len(self.param_groups) or any(
                len(a["params"]) != len(b["params"]) for a, b in zip(saved, self.param_groups)):
            raise ValueError("checkpoint has a different parameter layout")
        for group, sgroup in zip(self.param_groups, saved):
            if self._state_kind(sgroup) != self._state_kind(group):
                raise ValueError("checkpoint has a different state layout for a parameter group")
            for k, v in sgroup.items():
                if k != "params":
                    group[k] = v
            for p, idx in zip(group["params"], sgroup["params"]):
                src = sd["state"][idx]
                st = self.state[p]["flash"]
                if src["numel"] != st.numel:
                    raise ValueError("checkpoint tensor size differs")
                st.codes.copy_(src["codes"])
                st.scales.copy_(src["scales"])
                self.state[p]["step"] = int(src["step"])
        if self.capturable:
            for i, (group, sched) in enumerate(zip(self.param_groups, self._sched)):
                if sched is None:
                    continue
                steps = {self.state[p]["step"] for p in group["params"]}
                if len(steps) != 1:
                    raise ValueError("capturable: a group's parameters need equal step counts")
                self._sched[i] = F.DeviceSchedule(self._hp(group), t=steps.pop(),
                                                  optimizer=self.kind)
                self._sched_hp[i] = self._hp(group)

    def export_fp32(self, p: torch.Tensor):
        """(theta_hat, m, v) of one parameter in FP32 (v None unless AdamW)."""
        self._join_release()
        st = self.state[p]["flash"]
        th = torch.empty(st.numel, dtype=torch.float32, device=st.theta.device)
        m = torch.empty_like(th)
        v = torch.empty_like(th) if self.kind == "adamw" else None
        F.flashopt_tensor_export(st, th, m, v)
        return th, m, v


class FlashAdamW(_FlashOptimizer):
    """AdamW (decoupled weight decay, bias correction) with FlashOptim's
    compressed weight and moments."""
    kind = "adamw"

    def __init__(self, params: Iterable, lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 1e-2, gradient_release: bool = False,
                 release_streams: int = 1, release_bucket_bytes: int = 0,
                 compress: bool = True, capturable: bool = False):
        super().__init__(params, dict(lr=lr, betas=tuple(betas), eps=eps,
                                      weight_decay=weight_decay, compress=compress),
                         gradient_release, release_streams, release_bucket_bytes, capturable)

    def _hp(self, group) -> dict:
        return dict(lr=group["lr"], beta1=group["betas"][0], beta2=group["betas"][1],
                    eps=group["eps"], weight_decay=group["weight_decay"])


class FlashSGD(_FlashOptimizer):
    """SGD with momentum (L2 weight decay, no dampening, no Nesterov) with a
    compressed momentum buffer."""
    kind = "sgd"

    def __init__(self, params: Iterable, lr: float = 0.1, momentum: float = 0.9,
                 weight_decay: float = 0.0, gradient_release: bool = False,
                 release_streams: int = 1, release_bucket_bytes: int = 0,
                 compress: bool = True, capturable: bool = False):
        super().__init__(params, dict(lr=lr, momentum=momentum, weight_decay=weight_decay,
                                      compress=compress), gradient_release, release_streams,
                         release_bucket_bytes, capturable)

    def _hp(self, group) -> dict:
        return dict(lr=group["lr"], momentum=group["momentum"],
                    weight_decay=group["weight_decay"])


class FlashLion(_FlashOptimizer):
    """Lion (sign update, decoupled weight decay) with a compressed momentum."""
    kind = "lion"

    def __init__(self, params: Iterable, lr: float = 1e-4, betas=(0.9, 0.99),
                 weight_decay: float = 0.0, gradient_release: bool = False,
                 release_streams: int = 1, release_bucket_bytes: int = 0,
                 compress: bool = True, capturable: bool = False):
        super().__init__(params, dict(lr=lr, betas=tuple(betas), weight_decay=weight_decay,
                                      compress=compress), gradient_release, release_streams,
                         release_bucket_bytes, capturable)

    def _hp(self, group) -> dict:
        return dict(lr=group["lr"], beta1=group["betas"][0], beta2=group["betas"][1],
                    weight_decay=group["weight_decay"])
