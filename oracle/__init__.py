"""Python binding of the CPU oracle (oracle/flashopt_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg.  The library path never imports it.

Arrays are numpy; bf16 and fp16 values travel as their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "flashopt_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
GROUP = 32

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-builtin",
          "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_D = ctypes.c_double


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        sig = {
            "orc_env_ok": (ctypes.c_int, []),
            "orc_bf16_rne": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "orc_f16_rne": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "orc_split": (None, [_P, _I64, _P, _P]),
            "orc_unsplit": (None, [_P, _P, _I64, _P]),
            "orc_split_q": (None, [_P, _I64, ctypes.c_int32, _P, _P]),
            "orc_unsplit_q": (None, [_P, _P, _I64, ctypes.c_int32, _P]),
            "orc_split_f16_q": (None, [_P, _I64, ctypes.c_int32, _P, _P]),
            "orc_unsplit_f16_q": (None, [_P, _P, _I64, ctypes.c_int32, _P]),
            "orc_quant_lin_m": (None, [_P, _I64, _P, _P]),
            "orc_dequant_lin_m": (None, [_P, _P, _I64, _P]),
            "orc_quant_lin_v": (None, [_P, _I64, _P, _P]),
            "orc_dequant_lin_v": (None, [_P, _P, _I64, _P]),
            "orc_phi_m": (ctypes.c_float, [ctypes.c_float]),
            "orc_phi_m_inv": (ctypes.c_float, [ctypes.c_float]),
            "orc_phi_v": (ctypes.c_float, [ctypes.c_float]),
            "orc_phi_v_inv": (ctypes.c_float, [ctypes.c_float]),
            "orc_quant_m": (None, [_P, _I64, _P, _P]),
            "orc_dequant_m": (None, [_P, _P, _I64, _P]),
            "orc_quant_v": (None, [_P, _I64, _P, _P]),
            "orc_dequant_v": (None, [_P, _P, _I64, _P]),
            "orc_adamw_scalars": (None, [_D, _D, _D, _D, _D, _I64, _P]),
            "orc_adamw_step": (None, [_I64, _P, _P, _P, _P, _P, _P, _P,
                                      _D, _D, _D, _D, _D, _I64, _P, _P, _P]),
            "orc_sgd_step": (None, [_I64, _P, _P, _P, _P, _P, _D, _D, _D, _I64, _P, _P]),
            "orc_lion_step": (None, [_I64, _P, _P, _P, _P, _P, _D, _D, _D, _D, _P, _P]),
            "orc_adamw_step_fp32": (None, [_I64, _P, _P, _P, _P, _P, _D, _D, _D, _D, _D, _I64]),
            "orc_adamw_step_linv": (None, [_I64, _P, _P, _P, _P, _P, _P, _P,
                                           _D, _D, _D, _D, _D, _I64, _P, _P, _P]),
            "orc_sgd_step_fp32": (None, [_I64, _P, _P, _P, _P, _D, _D, _D]),
            "orc_lion_step_fp32": (None, [_I64, _P, _P, _P, _P, _D, _D, _D, _D]),
        }
        for name in ("bf16_rne_array", "f16_rne_array", "f16_to_f32_array", "phi_m_array",
                     "phi_m_inv_array", "phi_v_array", "phi_v_inv_array"):
            sig["orc_" + name] = (None, [_P, _I64, _P])
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        if L.orc_env_ok() != 1:
            raise RuntimeError("oracle: flush-to-zero or non-nearest rounding is in effect")
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def groups(n: int) -> int:
    return (n + GROUP - 1) // GROUP


# -- conversions ------------------------------------------------------------

def bf16_rne(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_rne_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(b) -> np.ndarray:
    b = _c(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f16_rne(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f16_rne_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32_array(_ptr(h), h.size, _ptr(out))
    return out


# -- split ------------------------------------------------------------------

def split(theta):
    theta = _c(theta, np.float32)
    tb = np.empty(theta.shape, np.uint16)
    rho = np.empty(theta.shape, np.int8)
    lib().orc_split(_ptr(theta), theta.size, _ptr(tb), _ptr(rho))
    return tb, rho


def unsplit(tb, rho) -> np.ndarray:
    tb = _c(tb, np.uint16)
    rho = _c(rho, np.int8)
    out = np.empty(tb.shape, np.float32)
    lib().orc_unsplit(_ptr(tb), _ptr(rho), tb.size, _ptr(out))
    return out


def split_q(theta, qmax: int):
    theta = _c(theta, np.float32)
    tb = np.empty(theta.shape, np.uint16)
    rho = np.empty(theta.shape, np.int32)
    lib().orc_split_q(_ptr(theta), theta.size, qmax, _ptr(tb), _ptr(rho))
    return tb, rho


def unsplit_q(tb, rho, qmax: int) -> np.ndarray:
    tb = _c(tb, np.uint16)
    rho = _c(rho, np.int32)
    out = np.empty(tb.shape, np.float32)
    lib().orc_unsplit_q(_ptr(tb), _ptr(rho), tb.size, qmax, _ptr(out))
    return out


def split_f16_q(theta, qmax: int):
    theta = _c(theta, np.float32)
    hb = np.empty(theta.shape, np.uint16)
    rho = np.empty(theta.shape, np.int32)
    lib().orc_split_f16_q(_ptr(theta), theta.size, qmax, _ptr(hb), _ptr(rho))
    return hb, rho


def unsplit_f16_q(hb, rho, qmax: int) -> np.ndarray:
    hb = _c(hb, np.uint16)
    rho = _c(rho, np.int32)
    out = np.empty(hb.shape, np.float32)
    lib().orc_unsplit_f16_q(_ptr(hb), _ptr(rho), hb.size, qmax, _ptr(out))
    return out


# -- companding and quantisers ----------------------------------------------

def _map(fname, x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.float32)
    getattr(lib(), fname)(_ptr(x), x.size, _ptr(out))
    return out


def phi_m(x): return _map("orc_phi_m_array", x)
def phi_m_inv(z): return _map("orc_phi_m_inv_array", z)
def phi_v(x): return _map("orc_phi_v_array", x)
def phi_v_inv(z): return _map("orc_phi_v_inv_array", z)


def quant_m(m):
    m = _c(m, np.float32)
    q = np.empty(m.shape, np.int8)
    s = np.empty(groups(m.size), np.uint16)
    lib().orc_quant_m(_ptr(m), m.size, _ptr(q), _ptr(s))
    return q, s


def dequant_m(q, s) -> np.ndarray:
    q = _c(q, np.int8)
    s = _c(s, np.uint16)
    assert s.size == groups(q.size)
    out = np.empty(q.shape, np.float32)
    lib().orc_dequant_m(_ptr(q), _ptr(s), q.size, _ptr(out))
    return out


def quant_v(v):
    v = _c(v, np.float32)
    q = np.empty(v.shape, np.uint8)
    s = np.empty(groups(v.size), np.uint16)
    lib().orc_quant_v(_ptr(v), v.size, _ptr(q), _ptr(s))
    return q, s


def dequant_v(q, s) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.uint16)
    assert s.size == groups(q.size)
    out = np.empty(q.shape, np.float32)
    lib().orc_dequant_v(_ptr(q), _ptr(s), q.size, _ptr(out))
    return out


def quant_lin_m(m):
    m = _c(m, np.float32)
    q = np.empty(m.shape, np.int8)
    s = np.empty(groups(m.size), np.uint16)
    lib().orc_quant_lin_m(_ptr(m), m.size, _ptr(q), _ptr(s))
    return q, s


def dequant_lin_m(q, s) -> np.ndarray:
    q = _c(q, np.int8)
    s = _c(s, np.uint16)
    out = np.empty(q.shape, np.float32)
    lib().orc_dequant_lin_m(_ptr(q), _ptr(s), q.size, _ptr(out))
    return out


def quant_lin_v(v):
    v = _c(v, np.float32)
    q = np.empty(v.shape, np.uint8)
    s = np.empty(groups(v.size), np.uint16)
    lib().orc_quant_lin_v(_ptr(v), v.size, _ptr(q), _ptr(s))
    return q, s


def dequant_lin_v(q, s) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.uint16)
    out = np.empty(q.shape, np.float32)
    lib().orc_dequant_lin_v(_ptr(q), _ptr(s), q.size, _ptr(out))
    return out


# -- steps ------------------------------------------------------------------

def adamw_scalars(lr, beta1, beta2, eps, weight_decay, t) -> np.ndarray:
    out = np.empty(8, np.float32)
    lib().orc_adamw_scalars(lr, beta1, beta2, eps, weight_decay, t, _ptr(out))
    return out


class State:
    """Compressed state of one tensor (host arrays, updated in place)."""

    def __init__(self, theta_fp32, optimizer="adamw"):
        n = int(np.asarray(theta_fp32).size)
        self.n = n
        self.optimizer = optimizer
        self.tb, self.rho = split(np.asarray(theta_fp32, np.float32).reshape(-1))
        self.qm = np.zeros(n, np.int8)
        self.sm = np.zeros(groups(n), np.uint16)
        if optimizer in ("adamw", "adamw_linv"):
            self.qv = np.zeros(n, np.uint8)
            self.sv = np.zeros(groups(n), np.uint16)
        else:
            self.qv = self.sv = None

    def copy(self) -> "State":
        c = State.__new__(State)
        c.n, c.optimizer = self.n, self.optimizer
        for k in ("tb", "rho", "qm", "sm", "qv", "sv"):
            v = getattr(self, k)
            setattr(c, k, None if v is None else v.copy())
        return c


def adamw_step(st: State, grad_bits, t: int, lr, beta1, beta2, eps, weight_decay,
               want_fp32: bool = False):
    """The AdamW step; for a State of optimizer "adamw_linv", the ablation
    with linearly quantised variance."""
    g = _c(grad_bits, np.uint16).reshape(-1)
    assert g.size == st.n
    outs = [np.empty(st.n, np.float32) for _ in range(3)] if want_fp32 else [None] * 3
    ptrs = [None if o is None else _ptr(o) for o in outs]
    fn = lib().orc_adamw_step_linv if st.optimizer == "adamw_linv" else lib().orc_adamw_step
    fn(st.n, _ptr(st.tb), _ptr(st.rho), _ptr(st.qm), _ptr(st.sm), _ptr(st.qv), _ptr(st.sv),
       _ptr(g), lr, beta1, beta2, eps, weight_decay, t, *ptrs)
    return outs if want_fp32 else None


def sgd_step(st: State, grad_bits, t: int, lr, momentum, weight_decay, want_fp32=False):
    g = _c(grad_bits, np.uint16).reshape(-1)
    assert g.size == st.n
    outs = [np.empty(st.n, np.float32) for _ in range(2)] if want_fp32 else [None] * 2
    ptrs = [None if o is None else _ptr(o) for o in outs]
    lib().orc_sgd_step(st.n, _ptr(st.tb), _ptr(st.rho), _ptr(st.qm), _ptr(st.sm), _ptr(g),
                       lr, momentum, weight_decay, t, *ptrs)
    return outs if want_fp32 else None


def lion_step(st: State, grad_bits, lr, beta1, beta2, weight_decay, want_fp32=False):
    g = _c(grad_bits, np.uint16).reshape(-1)
    assert g.size == st.n
    outs = [np.empty(st.n, np.float32) for _ in range(2)] if want_fp32 else [None] * 2
    ptrs = [None if o is None else _ptr(o) for o in outs]
    lib().orc_lion_step(st.n, _ptr(st.tb), _ptr(st.rho), _ptr(st.qm), _ptr(st.sm), _ptr(g),
                        lr, beta1, beta2, weight_decay, *ptrs)
    return outs if want_fp32 else None


def step(st: State, grad_bits, t: int, hp: dict, want_fp32=False):
    if st.optimizer in ("adamw", "adamw_linv"):
        return adamw_step(st, grad_bits, t, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                          hp["weight_decay"], want_fp32)
    if st.optimizer == "lion":
        return lion_step(st, grad_bits, hp["lr"], hp["beta1"], hp["beta2"], hp["weight_decay"],
                         want_fp32)
    return sgd_step(st, grad_bits, t, hp["lr"], hp["momentum"], hp["weight_decay"], want_fp32)


# -- compression disabled: FP32 master weight and moments --------------------

class StateFP32:
    """Uncompressed state of one tensor: FP32 theta, m, v (AdamW) and the
    BF16 theta' the model computes with (host arrays, updated in place)."""

    def __init__(self, theta_fp32, optimizer="adamw"):
        self.theta = np.array(theta_fp32, np.float32).reshape(-1)
        self.n = self.theta.size
        self.optimizer = optimizer
        self.m = np.zeros(self.n, np.float32)
        self.v = np.zeros(self.n, np.float32) if optimizer == "adamw" else None
        self.tb = bf16_rne(self.theta)

    def copy(self) -> "StateFP32":
        c = StateFP32.__new__(StateFP32)
        c.n, c.optimizer = self.n, self.optimizer
        for k in ("theta", "m", "v", "tb"):
            v = getattr(self, k)
            setattr(c, k, None if v is None else v.copy())
        return c


def step_fp32(st: StateFP32, grad_bits, t: int, hp: dict) -> None:
    g = _c(grad_bits, np.uint16).reshape(-1)
    assert g.size == st.n
    if st.optimizer == "adamw":
        lib().orc_adamw_step_fp32(st.n, _ptr(st.theta), _ptr(st.m), _ptr(st.v), _ptr(st.tb),
                                  _ptr(g), hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                  hp["weight_decay"], t)
    elif st.optimizer == "lion":
        lib().orc_lion_step_fp32(st.n, _ptr(st.theta), _ptr(st.m), _ptr(st.tb), _ptr(g),
                                 hp["lr"], hp["beta1"], hp["beta2"], hp["weight_decay"])
    else:
        lib().orc_sgd_step_fp32(st.n, _ptr(st.theta), _ptr(st.m), _ptr(st.tb), _ptr(g),
                                hp["lr"], hp["momentum"], hp["weight_decay"])


# -- threading helper (the oracle itself stays single-threaded) -------------

def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def chunked(fn, arrays_in, arrays_out, n: int, align: int = 1, nthreads: int | None = None):
    """Run fn(slice) over [0, n) in chunks on threads; ctypes drops the GIL.

    `fn(lo, hi)` must only touch elements [lo, hi).  Chunk edges are multiples
    of `align` (32 for the group-wise step functions), so every chunk is a
    whole number of groups and the result is the same for any thread count.
    """
    from concurrent.futures import ThreadPoolExecutor
    nt = nthreads or threads()
    per = -(-n // nt)
    per = -(-per // align) * align
    edges = [(lo, min(n, lo + per)) for lo in range(0, n, per)] if n else []
    if len(edges) <= 1:
        for lo, hi in edges:
            fn(lo, hi)
        return
    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(lambda e: fn(*e), edges))


def view(st: State, lo: int, hi: int) -> State:
    """State of elements [lo, hi) as views; lo must start a group."""
    assert lo % GROUP == 0
    c = State.__new__(State)
    c.n, c.optimizer = hi - lo, st.optimizer
    g0, g1 = lo // GROUP, groups(hi)
    c.tb, c.rho, c.qm, c.sm = st.tb[lo:hi], st.rho[lo:hi], st.qm[lo:hi], st.sm[g0:g1]
    c.qv = None if st.qv is None else st.qv[lo:hi]
    c.sv = None if st.sv is None else st.sv[g0:g1]
    return c


def step_chunked(st: State, grad_bits, t: int, hp: dict, nthreads: int | None = None):
    """`step` over whole groups on several threads; identical bytes to `step`."""
    g = _c(grad_bits, np.uint16).reshape(-1)
    chunked(lambda lo, hi: step(view(st, lo, hi), g[lo:hi], t, hp), None, None, st.n,
            align=GROUP, nthreads=nthreads)
