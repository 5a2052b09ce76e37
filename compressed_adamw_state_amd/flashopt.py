"""Thin Python binding of libflashopt.so (include/flashopt.h).

Argument marshalling only: each function below forwards to the C entry point
of the same name; every step of the optimizer runs in the HIP kernels.  torch
is used for device memory and streams: tensors are passed by data pointer,
streams by their HIP handle.  There is no fallback: if the HIP library is
missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflashopt.so")
GROUP = 32

STATUS = {0: "ok", -1: "null pointer", -2: "size", -3: "alignment", -4: "argument",
          -5: "step", -6: "workspace", -7: "HIP error", -8: "index", -9: "host memory"}


class FlashoptError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status} ({STATUS.get(status, '?')})")
        self.status = status


# flashopt_kind; "<opt>_fp32" is the optimizer with compression switched off
# (FP32 master weight and moments, no scales); "adamw_linv" the ablation with
# linear variance codes (experiments only)
KIND = {"adamw": 0, "sgd": 1, "lion": 2, "adamw_fp32": 3, "sgd_fp32": 4, "lion_fp32": 5,
        "adamw_linv": 6}
SCALES = {"adamw": 2, "sgd": 1, "lion": 1,        # FP16 scales per 32-element group
          "adamw_linv": 2}
FP32_FIELDS = {"adamw_fp32": 3, "sgd_fp32": 2, "lion_fp32": 2}   # per 512-element block


def base_optimizer(kind: str) -> str:
    """The optimizer of a state kind: "adamw_fp32", "adamw_linv" -> "adamw"."""
    return kind.split("_")[0]


class Tensor(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("theta", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("grad", ctypes.c_void_p)]


class AdamWHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class SGDHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("momentum", ctypes.c_double),
                ("weight_decay", ctypes.c_double)]


class LionHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("weight_decay", ctypes.c_double)]


class AdamWSchedule(ctypes.Structure):
    """flashopt_adamw_schedule (lives in device memory; see DeviceSchedule)."""
    _fields_ = [("lr", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("t", ctypes.c_int64), ("p1", ctypes.c_double),
                ("p2", ctypes.c_double), ("scalars", ctypes.c_uint32 * 10),
                ("pad", ctypes.c_uint32 * 2)]


class SGDSchedule(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("momentum", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("t", ctypes.c_int64),
                ("scalars", ctypes.c_uint32 * 4)]


class LionSchedule(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("t", ctypes.c_int64),
                ("scalars", ctypes.c_uint32 * 6)]


_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = {
    "flashopt_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "flashopt_split": (ctypes.c_int, [_P, _I64, _P, _P, _P]),
    "flashopt_unsplit": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "flashopt_quantize_m": (ctypes.c_int, [_P, _I64, _P, _P, _P]),
    "flashopt_dequantize_m": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "flashopt_quantize_v": (ctypes.c_int, [_P, _I64, _P, _P, _P]),
    "flashopt_dequantize_v": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "flashopt_list_workspace_bytes": (_SZ, [_I32]),
    "flashopt_split_ex": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "flashopt_unsplit_ex": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _P, _P]),
    "flashopt_quantize_lin_m": (ctypes.c_int, [_P, _I64, _P, _P, _P]),
    "flashopt_dequantize_lin_m": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "flashopt_quantize_lin_v": (ctypes.c_int, [_P, _I64, _P, _P, _P]),
    "flashopt_dequantize_lin_v": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "flashopt_codes_bytes": (_SZ, [_I32, _I64]),
    "flashopt_scales_bytes": (_SZ, [_I32, _I64]),
    "flashopt_tensor_init": (ctypes.c_int, [ctypes.POINTER(Tensor), _I32, _P, _P]),
    "flashopt_tensor_export": (ctypes.c_int, [ctypes.POINTER(Tensor), _I32, _P, _P, _P, _P]),
    "flashopt_list_create": (ctypes.c_int, [ctypes.POINTER(Tensor), _I32, _I32, _P, _SZ, _P,
                                            ctypes.POINTER(_P)]),
    "flashopt_list_destroy": (ctypes.c_int, [_P]),
    "flashopt_list_numel": (_I64, [_P]),
    "flashopt_list_set_grads": (ctypes.c_int, [_P, ctypes.POINTER(_P), _P]),
    "flashopt_state_zero": (ctypes.c_int, [_P, _P]),
    "flashopt_adamw_step": (ctypes.c_int, [_P, ctypes.POINTER(AdamWHparams), _I64, _P]),
    "flashopt_sgd_step": (ctypes.c_int, [_P, ctypes.POINTER(SGDHparams), _I64, _P]),
    "flashopt_adamw_step_one": (ctypes.c_int, [_P, _I32, _P, ctypes.POINTER(AdamWHparams),
                                               _I64, _P]),
    "flashopt_sgd_step_one": (ctypes.c_int, [_P, _I32, _P, ctypes.POINTER(SGDHparams), _I64,
                                             _P]),
    "flashopt_stream_probe": (ctypes.c_int, [_P, _P]),
    "flashopt_mix_ceiling": (ctypes.c_int, [_P, _P, _P, _P, _I64, _P]),
    "flashopt_pattern_probe": (ctypes.c_int, [_I32, _P, _P, _P, _P, _I64, _P]),
    "flashopt_adamw_step_noalloc": (ctypes.c_int, [ctypes.POINTER(Tensor), _I32,
                                                   ctypes.POINTER(AdamWHparams), _I64, _P]),
    "flashopt_stream_sweep": (ctypes.c_int, [_I32, _I32, ctypes.POINTER(_P), ctypes.POINTER(_P),
                                             _I32, _I64, _P]),
    "flashopt_lion_step": (ctypes.c_int, [_P, ctypes.POINTER(LionHparams), _I64, _P]),
    "flashopt_adamw_schedule_init": (ctypes.c_int, [_P, ctypes.POINTER(AdamWHparams), _I64, _P]),
    "flashopt_adamw_step_scheduled": (ctypes.c_int, [_P, _P, _P]),
    "flashopt_sgd_schedule_init": (ctypes.c_int, [_P, ctypes.POINTER(SGDHparams), _I64, _P]),
    "flashopt_sgd_step_scheduled": (ctypes.c_int, [_P, _P, _P]),
    "flashopt_lion_schedule_init": (ctypes.c_int, [_P, ctypes.POINTER(LionHparams), _I64, _P]),
    "flashopt_lion_step_scheduled": (ctypes.c_int, [_P, _P, _P]),
    "flashopt_lion_step_one": (ctypes.c_int, [_P, _I32, _P, ctypes.POINTER(LionHparams),
                                              _I64, _P]),
    "flashopt_adamw_step_range": (ctypes.c_int, [_P, _I32, _I32, ctypes.POINTER(_P),
                                                 ctypes.POINTER(AdamWHparams), _I64, _P]),
    "flashopt_sgd_step_range": (ctypes.c_int, [_P, _I32, _I32, ctypes.POINTER(_P),
                                               ctypes.POINTER(SGDHparams), _I64, _P]),
    "flashopt_lion_step_range": (ctypes.c_int, [_P, _I32, _I32, ctypes.POINTER(_P),
                                                ctypes.POINTER(LionHparams), _I64, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree HIP library (building it only if it is absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise FlashoptError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def groups(n: int) -> int:
    return (n + GROUP - 1) // GROUP


# ---- flat buffers ---------------------------------------------------------

def flashopt_split(theta, theta_bf16, rho, stream=None) -> None:
    _check("flashopt_split", lib().flashopt_split(_ptr(theta), theta.numel(), _ptr(theta_bf16),
                                                  _ptr(rho), _stream(stream)))


def flashopt_unsplit(theta_bf16, rho, theta_out, stream=None) -> None:
    _check("flashopt_unsplit", lib().flashopt_unsplit(_ptr(theta_bf16), _ptr(rho),
                                                      theta_bf16.numel(), _ptr(theta_out),
                                                      _stream(stream)))


def flashopt_quantize_m(m, q, scale, stream=None) -> None:
    _check("flashopt_quantize_m", lib().flashopt_quantize_m(_ptr(m), m.numel(), _ptr(q),
                                                            _ptr(scale), _stream(stream)))


def flashopt_dequantize_m(q, scale, m_out, stream=None) -> None:
    _check("flashopt_dequantize_m", lib().flashopt_dequantize_m(_ptr(q), _ptr(scale), q.numel(),
                                                                _ptr(m_out), _stream(stream)))


def flashopt_quantize_v(v, q, scale, stream=None) -> None:
    _check("flashopt_quantize_v", lib().flashopt_quantize_v(_ptr(v), v.numel(), _ptr(q),
                                                            _ptr(scale), _stream(stream)))


def flashopt_dequantize_v(q, scale, v_out, stream=None) -> None:
    _check("flashopt_dequantize_v", lib().flashopt_dequantize_v(_ptr(q), _ptr(scale), q.numel(),
                                                                _ptr(v_out), _stream(stream)))


# ---- codec ablations (not used by the step) ---------------------------------

BASE = {"bf16": 0, "fp16": 1}


def flashopt_split_ex(theta, base: str, qmax: int, theta_base, rho, stream=None) -> None:
    _check("flashopt_split_ex",
           lib().flashopt_split_ex(_ptr(theta), theta.numel(), BASE[base], qmax, _ptr(theta_base),
                                   _ptr(rho), _stream(stream)))


def flashopt_unsplit_ex(theta_base, rho, base: str, qmax: int, theta_out, stream=None) -> None:
    _check("flashopt_unsplit_ex",
           lib().flashopt_unsplit_ex(_ptr(theta_base), _ptr(rho), theta_base.numel(), BASE[base],
                                     qmax, _ptr(theta_out), _stream(stream)))


def flashopt_quantize_lin_m(m, q, scale, stream=None) -> None:
    _check("flashopt_quantize_lin_m", lib().flashopt_quantize_lin_m(
        _ptr(m), m.numel(), _ptr(q), _ptr(scale), _stream(stream)))


def flashopt_dequantize_lin_m(q, scale, m_out, stream=None) -> None:
    _check("flashopt_dequantize_lin_m", lib().flashopt_dequantize_lin_m(
        _ptr(q), _ptr(scale), q.numel(), _ptr(m_out), _stream(stream)))


def flashopt_quantize_lin_v(v, q, scale, stream=None) -> None:
    _check("flashopt_quantize_lin_v", lib().flashopt_quantize_lin_v(
        _ptr(v), v.numel(), _ptr(q), _ptr(scale), _stream(stream)))


def flashopt_dequantize_lin_v(q, scale, v_out, stream=None) -> None:
    _check("flashopt_dequantize_lin_v", lib().flashopt_dequantize_lin_v(
        _ptr(q), _ptr(scale), q.numel(), _ptr(v_out), _stream(stream)))


# ---- tensor lists -----------------------------------------------------------

class TensorState:
    """Device arrays of one tensor's state (allocated with torch): BF16
    theta', the codes (AdamW: 512-element blocks of rho, m and v code planes;
    SGD, Lion: 8-element records) and the FP16 scales in the layout of
    include/flashopt.h -- or, for the "_fp32" kinds, the blocks of FP32 fields
    and no scales."""

    def __init__(self, numel: int, optimizer: str, device, theta: Optional[torch.Tensor] = None,
                 codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
        """theta: an existing contiguous BF16 tensor of numel elements to use as
        theta' (e.g. a model parameter's data); allocated when None.  codes,
        scales: existing zeroed uint8 / int16 tensors of exactly the layout's
        sizes (e.g. slices of a StateArena); allocated when None."""
        self.numel = numel
        self.optimizer = optimizer
        self.kind = KIND[optimizer]
        if theta is None:
            theta = torch.empty(numel, dtype=torch.bfloat16, device=device)
        elif theta.dtype != torch.bfloat16 or theta.numel() != numel or not theta.is_contiguous():
            raise ValueError("theta must be a contiguous BF16 tensor of numel elements")
        self.theta = theta.view(-1)
        cb = lib().flashopt_codes_bytes(self.kind, numel)
        sn = lib().flashopt_scales_bytes(self.kind, numel) // 2
        if codes is None:
            codes = torch.zeros(cb, dtype=torch.uint8, device=device)
        elif codes.dtype != torch.uint8 or codes.numel() != cb or not codes.is_contiguous():
            raise ValueError(f"codes must be a contiguous uint8 tensor of {cb} bytes")
        if scales is None:
            scales = torch.zeros(sn, dtype=torch.int16, device=device)
        elif scales.dtype != torch.int16 or scales.numel() != sn or not scales.is_contiguous():
            raise ValueError(f"scales must be a contiguous int16 tensor of {sn} entries")
        self.codes = codes
        self.scales = scales

    def descriptor(self, grad: Optional[torch.Tensor] = None) -> Tensor:
        scales = _ptr(self.scales) if self.scales.numel() else None
        return Tensor(self.numel, _ptr(self.theta), _ptr(self.codes), scales, _ptr(grad))


class StateArena:
    """The state of a list of tensors in one device buffer with one region per
    stream the fused step reads or writes: optionally theta' (theta=True),
    optionally `grad_sets` sets of BF16 gradients, then the codes, then the
    FP16 scales.  Each region starts on a 2 MiB boundary and each tensor's
    slice within it on a 4096-byte boundary; codes and scales are zeroed.
    state(i) builds tensor i's TensorState on its slices (theta' from the
    arena, or a given tensor such as a parameter's own storage); grad(j, i) is
    tensor i's gradient of set j.

    Why one buffer with a region per stream: one allocation for the whole
    state instead of four per tensor, and each stream the step reads or
    writes contiguous across the list's tensors.  The step's rate on MI355X
    does not depend on the layout inside the buffer so much as on where the
    allocation's physical pages land: the same byte mix over different
    allocations of the same buffers takes 16.2-19.0 ms at Llama-3.1-8B size,
    whatever the order of the tiles, and each array alone streams at the same
    rate in every allocation.

    candidates > 1 (a compressed kind, with theta' and at least one gradient
    set): a placement search.  Up to `candidates` allocations of the buffer
    are made, all alive at once (fewer if the device runs short of free
    memory); on each, the step's own loads and stores over the list
    (flashopt_stream_probe, best of three launches after one untimed) are
    timed, the fastest allocation is kept and the others are freed and
    handed back to the device (torch.cuda.empty_cache).  The probe's time on
    an allocation ranks the step's on it; `placement_ms` holds the probe
    times in allocation order and `placement_choice` the index kept.  The
    search needs `candidates` times the buffer's memory while it runs."""

    ALIGN = 4096
    REGION = 1 << 21
    HEADROOM = 1 << 30           # free memory left on the device by the search

    def __init__(self, numels: Sequence[int], optimizer: str, device, theta: bool = False,
                 grad_sets: int = 0, candidates: int = 1):
        self.numels = [int(n) for n in numels]
        self.optimizer = optimizer
        kind = KIND[optimizer]
        cb = [lib().flashopt_codes_bytes(kind, n) for n in self.numels]
        sb = [lib().flashopt_scales_bytes(kind, n) for n in self.numels]
        bb = [2 * n for n in self.numels]
        start = 0
        self._ts = None
        if theta:
            self._ts, start = self._slices(bb, start)
        self._gs = []
        for _ in range(grad_sets):
            gs, start = self._slices(bb, start)
            self._gs.append(gs)
        self._cs, start = self._slices(cb, start)
        self._ss, end = self._slices(sb, start)
        nbytes = max(end, 1)
        self.placement_ms, self.placement_choice = None, None
        if candidates > 1:
            if optimizer in FP32_FIELDS or not theta or grad_sets < 1:
                raise ValueError("the placement search needs a compressed arena with theta' "
                                 "and a gradient set")
            self._search(nbytes, device, candidates)
        else:
            self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.device = self.buffer.device
        c0 = min([o for o, _ in self._cs] + [end])
        self.buffer[c0:end].zero_()                            # codes and scales

    def _search(self, nbytes: int, device, candidates: int) -> None:
        dev = torch.device(device)
        if dev.type != "cuda":
            raise ValueError("the placement search needs a GPU arena")
        with torch.cuda.device(dev):
            self._search_on(nbytes, dev, candidates)

    def _search_on(self, nbytes: int, dev: torch.device, candidates: int) -> None:
        stream = torch.cuda.current_stream(dev)
        n = len(self.numels)
        bufs, times = [], []
        for c in range(candidates):
            if c and torch.cuda.mem_get_info(dev)[0] < nbytes + self.HEADROOM:
                break
            self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            self.device = self.buffer.device
            lst = FlashoptList([self.state(i) for i in range(n)],
                               [self.grad(0, i) for i in range(n)])
            flashopt_stream_probe(lst, stream)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record(stream)
            for k in range(3):
                flashopt_stream_probe(lst, stream)
                ev[k + 1].record(stream)
            torch.cuda.synchronize(dev)
            times.append(min(ev[k].elapsed_time(ev[k + 1]) for k in range(3)))
            bufs.append(self.buffer)
            del lst
        best = min(range(len(times)), key=times.__getitem__)
        self.buffer = bufs[best]
        self.placement_ms, self.placement_choice = times, best
        del bufs
        torch.cuda.empty_cache()

    @classmethod
    def _slices(cls, sizes, start):
        """slices of `sizes` bytes from the next region boundary at or after start"""
        o = -(-start // cls.REGION) * cls.REGION
        out = []
        for b in sizes:
            out.append((o, b))
            o += -(-b // cls.ALIGN) * cls.ALIGN
        return out, o

    def state(self, i: int, theta: Optional[torch.Tensor] = None) -> TensorState:
        co, cb = self._cs[i]
        so, sb = self._ss[i]
        if theta is None and self._ts is not None:
            to, tb = self._ts[i]
            theta = self.buffer[to:to + tb].view(torch.bfloat16)
        return TensorState(self.numels[i], self.optimizer, self.device, theta=theta,
                           codes=self.buffer[co:co + cb],
                           scales=self.buffer[so:so + sb].view(torch.int16))

    def grad(self, j: int, i: int) -> torch.Tensor:
        """Tensor i's BF16 gradient buffer of set j (contents undefined)."""
        go, gb = self._gs[j][i]
        return self.buffer[go:go + gb].view(torch.bfloat16)


def flashopt_tensor_init(st: TensorState, theta_fp32: torch.Tensor, stream=None) -> None:
    """theta', rho from FP32 weights (device [numel]); codes and scales zero."""
    d = st.descriptor()
    _check("flashopt_tensor_init", lib().flashopt_tensor_init(ctypes.byref(d), st.kind,
                                                              _ptr(theta_fp32), _stream(stream)))


def flashopt_tensor_export(st: TensorState, theta_out=None, m_out=None, v_out=None,
                           stream=None) -> None:
    """Rebuilt FP32 master weight and dequantised m, v (device [numel] each, any None)."""
    d = st.descriptor()
    _check("flashopt_tensor_export",
           lib().flashopt_tensor_export(ctypes.byref(d), st.kind, _ptr(theta_out), _ptr(m_out),
                                        _ptr(v_out), _stream(stream)))


class FlashoptList:
    """A flashopt_list handle over a list of TensorState of one optimizer kind
    (device workspace from torch)."""

    def __init__(self, states: Sequence[TensorState], grads: Sequence[Optional[torch.Tensor]],
                 stream=None, optimizer: Optional[str] = None):
        self.states = list(states)
        count = len(self.states)
        if optimizer is None:
            optimizer = self.states[0].optimizer if count else "adamw"
        if any(st.optimizer != optimizer for st in self.states):
            raise ValueError("every tensor of a list needs the list's optimizer layout")
        self.optimizer = optimizer
        arr = (Tensor * max(count, 1))()
        for i, (st, g) in enumerate(zip(self.states, grads)):
            arr[i] = st.descriptor(g)
        self.grads = list(grads)
        nbytes = lib().flashopt_list_workspace_bytes(count)
        dev = self.states[0].theta.device if count else torch.device("cuda")
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        h = ctypes.c_void_p()
        _check("flashopt_list_create",
               lib().flashopt_list_create(arr, count, KIND[optimizer], _ptr(self.workspace),
                                          nbytes, _stream(stream), ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.flashopt_list_destroy(h)
            self.handle = None

    def numel(self) -> int:
        return lib().flashopt_list_numel(self.handle)


def flashopt_list_set_grads(lst: FlashoptList, grads: Sequence[Optional[torch.Tensor]],
                            stream=None) -> None:
    arr = (ctypes.c_void_p * max(len(grads), 1))(*[_ptr(g) for g in grads])
    _check("flashopt_list_set_grads", lib().flashopt_list_set_grads(lst.handle, arr,
                                                                    _stream(stream)))
    lst.grads = list(grads)


def flashopt_state_zero(lst: FlashoptList, stream=None) -> None:
    _check("flashopt_state_zero", lib().flashopt_state_zero(lst.handle, _stream(stream)))


def flashopt_stream_probe(lst: FlashoptList, stream=None) -> None:
    """Bandwidth probe (include/flashopt_probe.h): the list's step's exact
    loads and stores (AdamW, SGD or Lion) with one XOR per word instead of
    the update.  Overwrites the state."""
    _check("flashopt_stream_probe", lib().flashopt_stream_probe(lst.handle, _stream(stream)))


NOALLOC_MAX_TENSORS = 4096


def flashopt_adamw_step_noalloc(states: Sequence[TensorState], grads: Sequence[torch.Tensor],
                                hp: dict, step: int, stream=None) -> None:
    """The whole-list AdamW step without a handle or workspace
    (include/flashopt.h): the descriptor table lives in the library's own
    device array, so the call allocates nothing on the device."""
    arr = (Tensor * max(len(states), 1))()
    for i, (st, g) in enumerate(zip(states, grads)):
        arr[i] = st.descriptor(g)
    h = _adam(hp)
    _check("flashopt_adamw_step_noalloc", lib().flashopt_adamw_step_noalloc(
        arr, len(states), ctypes.byref(h), step, _stream(stream)))


def flashopt_mix_ceiling(theta: torch.Tensor, grad: torch.Tensor, codes: torch.Tensor,
                         scales: torch.Tensor, n: int, stream=None) -> None:
    """Ceiling of the step's byte mix (include/flashopt_probe.h) over flat
    buffers of n parameters: theta, grad 2n bytes, codes 3n, scales n/8.
    Overwrites theta, codes and scales."""
    for t, need in ((theta, 2 * n), (grad, 2 * n), (codes, 3 * n), (scales, n // 8)):
        assert t.is_contiguous() and t.numel() * t.element_size() >= need
    _check("flashopt_mix_ceiling", lib().flashopt_mix_ceiling(
        _ptr(theta), _ptr(grad), _ptr(codes), _ptr(scales), n, _stream(stream)))


def flashopt_pattern_probe(variant: int, theta: torch.Tensor, grad: torch.Tensor,
                           codes: torch.Tensor, scales: torch.Tensor, n: int, stream=None) -> None:
    """The step's traffic with access pattern `variant` (include/flashopt_probe.h)
    over the flat buffers of flashopt_mix_ceiling.  Overwrites theta, codes and
    scales."""
    for t, need in ((theta, 2 * n), (grad, 2 * n), (codes, 3 * n), (scales, n // 8)):
        assert t.is_contiguous() and t.numel() * t.element_size() >= need
    _check("flashopt_pattern_probe", lib().flashopt_pattern_probe(
        variant, _ptr(theta), _ptr(grad), _ptr(codes), _ptr(scales), n, _stream(stream)))


def flashopt_stream_sweep(reads: Sequence[torch.Tensor], writes: Sequence[torch.Tensor],
                          nbytes: int, in_place: bool = False, stream=None) -> None:
    """Stream-count sweep (include/flashopt_probe.h): len(reads) buffers read,
    len(writes) written, nbytes each; in place, `writes` must be the first
    len(writes) of `reads`."""
    if in_place and any(a is not b for a, b in zip(writes, reads[:len(writes)])):
        raise ValueError("in place: writes must be reads[:len(writes)]")
    for t in list(reads) + list(writes):
        assert t.is_contiguous() and t.numel() * t.element_size() >= nbytes
    r = (ctypes.c_void_p * max(len(reads), 1))(*[_ptr(t) for t in reads])
    w = (ctypes.c_void_p * max(len(writes), 1))(*[_ptr(t) for t in writes])
    _check("flashopt_stream_sweep", lib().flashopt_stream_sweep(
        len(reads), len(writes), r, w, int(in_place), nbytes, _stream(stream)))


def _adam(hp: dict) -> AdamWHparams:
    return AdamWHparams(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])


def _sgd(hp: dict) -> SGDHparams:
    return SGDHparams(hp["lr"], hp["momentum"], hp["weight_decay"])


def flashopt_adamw_step(lst: FlashoptList, hp: dict, step: int, stream=None) -> None:
    h = _adam(hp)
    _check("flashopt_adamw_step", lib().flashopt_adamw_step(lst.handle, ctypes.byref(h), step,
                                                            _stream(stream)))


def flashopt_sgd_step(lst: FlashoptList, hp: dict, step: int, stream=None) -> None:
    h = _sgd(hp)
    _check("flashopt_sgd_step", lib().flashopt_sgd_step(lst.handle, ctypes.byref(h), step,
                                                        _stream(stream)))


def flashopt_adamw_step_one(lst: FlashoptList, index: int, grad, hp: dict, step: int,
                            stream=None) -> None:
    h = _adam(hp)
    _check("flashopt_adamw_step_one",
           lib().flashopt_adamw_step_one(lst.handle, index, _ptr(grad), ctypes.byref(h), step,
                                         _stream(stream)))


def flashopt_sgd_step_one(lst: FlashoptList, index: int, grad, hp: dict, step: int,
                          stream=None) -> None:
    h = _sgd(hp)
    _check("flashopt_sgd_step_one",
           lib().flashopt_sgd_step_one(lst.handle, index, _ptr(grad), ctypes.byref(h), step,
                                       _stream(stream)))


def _lion(hp: dict) -> LionHparams:
    return LionHparams(hp["lr"], hp["beta1"], hp["beta2"], hp["weight_decay"])


def flashopt_lion_step(lst: FlashoptList, hp: dict, step: int, stream=None) -> None:
    h = _lion(hp)
    _check("flashopt_lion_step", lib().flashopt_lion_step(lst.handle, ctypes.byref(h), step,
                                                          _stream(stream)))


def flashopt_lion_step_one(lst: FlashoptList, index: int, grad, hp: dict, step: int,
                           stream=None) -> None:
    h = _lion(hp)
    _check("flashopt_lion_step_one",
           lib().flashopt_lion_step_one(lst.handle, index, _ptr(grad), ctypes.byref(h), step,
                                        _stream(stream)))


def step_range(lst: FlashoptList, optimizer: str, first: int,
               grads: Sequence[Optional[torch.Tensor]], hp: dict, t: int, stream=None) -> None:
    """Bucketed gradient release: one launch over the list's tensors
    [first, first + len(grads)) with these gradients (flashopt_*_step_range).
    The gradients serve this launch only: the list keeps no reference to
    them (so released gradients are freed), and holds no gradient for these
    tensors afterwards."""
    base = base_optimizer(optimizer)
    fn = "flashopt_%s_step_range" % base
    h = {"adamw": _adam, "sgd": _sgd, "lion": _lion}[base](hp)
    arr = (ctypes.c_void_p * max(len(grads), 1))(*[_ptr(g) for g in grads])
    _check(fn, getattr(lib(), fn)(lst.handle, first, len(grads), arr, ctypes.byref(h), t,
                                  _stream(stream)))
    lst.grads[first:first + len(grads)] = [None] * len(grads)


class DeviceSchedule:
    """A flashopt_{adamw,sgd,lion}_schedule in device memory (a torch byte
    tensor): the step counter (and, for AdamW, the bias-correction powers)
    and the schedulable hyper-parameters of the *_step_scheduled calls,
    which a captured HIP graph can replay."""

    _STRUCT = {"adamw": AdamWSchedule, "sgd": SGDSchedule, "lion": LionSchedule}
    _HP = {"adamw": lambda hp: _adam(hp), "sgd": lambda hp: _sgd(hp),
           "lion": lambda hp: _lion(hp)}
    # the hyper-parameters each call reads on the device (AdamW's betas are
    # fixed at init because the powers depend on them)
    SETTABLE = {"adamw": ("lr", "eps", "weight_decay"),
                "sgd": ("lr", "momentum", "weight_decay"),
                "lion": ("lr", "beta1", "beta2", "weight_decay")}

    def __init__(self, hp: dict, t: int = 0, device="cuda", stream=None,
                 optimizer: str = "adamw"):
        self.optimizer = optimizer
        self.struct = self._STRUCT[optimizer]
        self.buf = torch.zeros(ctypes.sizeof(self.struct), dtype=torch.uint8, device=device)
        h = self._HP[optimizer](hp)
        fn = "flashopt_%s_schedule_init" % optimizer
        _check(fn, getattr(lib(), fn)(_ptr(self.buf), ctypes.byref(h), t, _stream(stream)))

    def set(self, name: str, value: float) -> None:
        """Write one of SETTABLE on the device (stream-ordered: takes effect
        from the next step call or replay).  The device does not validate
        what it reads, so the value is checked here against the ranges of the
        hyper-parameter structs (include/flashopt.h)."""
        if name not in self.SETTABLE[self.optimizer]:
            raise ValueError(f"{name} is not settable on a {self.optimizer} schedule")
        value = float(value)
        if name in ("momentum", "beta1", "beta2"):
            ok = 0.0 <= value < 1.0
        elif name == "eps":
            ok = math.isfinite(value) and float(np.float32(value)) > 0.0
        else:                                    # lr, weight_decay
            ok = math.isfinite(value) and value >= 0.0
        if not ok:
            raise ValueError(f"{name} = {value} is outside its range")
        o = getattr(self.struct, name).offset
        self.buf[o:o + 8].view(torch.float64).fill_(value)

    def read(self):
        return self.struct.from_buffer_copy(self.buf.cpu().numpy().tobytes())


def flashopt_adamw_step_scheduled(lst: FlashoptList, schedule: DeviceSchedule,
                                  stream=None) -> None:
    _check("flashopt_adamw_step_scheduled",
           lib().flashopt_adamw_step_scheduled(lst.handle, _ptr(schedule.buf), _stream(stream)))


def flashopt_sgd_step_scheduled(lst: FlashoptList, schedule: DeviceSchedule,
                                stream=None) -> None:
    _check("flashopt_sgd_step_scheduled",
           lib().flashopt_sgd_step_scheduled(lst.handle, _ptr(schedule.buf), _stream(stream)))


def flashopt_lion_step_scheduled(lst: FlashoptList, schedule: DeviceSchedule,
                                 stream=None) -> None:
    _check("flashopt_lion_step_scheduled",
           lib().flashopt_lion_step_scheduled(lst.handle, _ptr(schedule.buf), _stream(stream)))


def step_scheduled(lst: FlashoptList, schedule: DeviceSchedule, stream=None) -> None:
    {"adamw": flashopt_adamw_step_scheduled, "sgd": flashopt_sgd_step_scheduled,
     "lion": flashopt_lion_step_scheduled}[schedule.optimizer](lst, schedule, stream)


def step(lst: FlashoptList, optimizer: str, hp: dict, t: int, stream=None) -> None:
    """optimizer: "adamw", "sgd", "lion" (either state kind of that optimizer)."""
    {"adamw": flashopt_adamw_step, "sgd": flashopt_sgd_step,
     "lion": flashopt_lion_step}[base_optimizer(optimizer)](lst, hp, t, stream)


def step_one(lst: FlashoptList, optimizer: str, index: int, grad, hp: dict, t: int,
             stream=None) -> None:
    {"adamw": flashopt_adamw_step_one, "sgd": flashopt_sgd_step_one,
     "lion": flashopt_lion_step_one}[base_optimizer(optimizer)](lst, index, grad, hp, t, stream)


def build_list(theta_fp32: List[torch.Tensor], optimizer: str,
               grads: Sequence[Optional[torch.Tensor]], stream=None):
    """Allocate compressed state for fp32 master weights, split them (zero
    optimizer state); returns (states, list handle)."""
    states = []
    arena = StateArena([th.numel() for th in theta_fp32], optimizer,
                       theta_fp32[0].device, theta=True) if theta_fp32 else None
    for i, th in enumerate(theta_fp32):
        st = arena.state(i)
        flashopt_tensor_init(st, th.reshape(-1).contiguous(), stream)
        states.append(st)
    lst = FlashoptList(states, grads, stream, optimizer)
    return states, lst
