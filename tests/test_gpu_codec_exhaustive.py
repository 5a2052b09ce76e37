"""Exhaustive device check of the fused kernel's short exactly rounded
sequences (tests/hip/codec_exhaustive.hip): over all 2^32 binary32 inputs
and all 2^16 FP16 scales, each must equal the general sequence it replaces
wherever the kernel uses it.  This is what licenses the fast path; the
oracle parity tests then check the whole step."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
NAMES = ["phi_m", "phi_m_inverse", "sqrt", "split", "split_flag", "variance_code", "sqrt_flag",
         "momentum_code", "reciprocal", "quotient_window", "phi_m_half", "unsplit_fma"]


def _lib():
    path = os.path.join(HERE, "hip", "libcodec_exhaustive.so")
    if not os.path.exists(path):
        from compressed_adamw_state_amd import build
        build.build_test_lib()
    return ctypes.CDLL(path)


def test_short_sequences_match_general_sequences_on_every_input():
    L = _lib()
    k = L.codec_exhaustive_checks()
    blocks = 2048
    nth = blocks * 256
    count = torch.zeros(nth * k, dtype=torch.int32, device="cuda")
    example = torch.zeros(nth * k, dtype=torch.int32, device="cuda")
    scale_bad = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    rc = L.codec_exhaustive_run(ctypes.c_void_p(count.data_ptr()),
                                ctypes.c_void_p(example.data_ptr()), blocks,
                                ctypes.c_void_p(scale_bad.data_ptr()))
    assert rc == 0
    c = count.view(nth, k).cpu().numpy().astype(np.int64).sum(axis=0)
    ex = example.view(nth, k).cpu().numpy().view(np.uint32)
    report = {NAMES[i]: int(c[i]) for i in range(k)}
    print("mismatches per check:", report, flush=True)
    for i in range(k):
        assert c[i] == 0, (NAMES[i], int(c[i]), [hex(v) for v in ex[ex[:, i] != 0, i][:5]])
    sb = scale_bad.cpu().numpy()
    assert not (sb & 1).any(), "127/s differs for some FP16 scale"
    assert not (sb & 2).any(), "255/s differs for some FP16 scale"
    assert not (sb & 4).any(), "254/s is not 2 * 127/s for some FP16 scale"


def test_adam_quotient_on_every_significand_pair():
    # div_rn against the IEEE division for all 2^46 pairs (a, b) in [1, 2)^2,
    # in 16 slices of 2^19 numerators
    L = _lib()
    bad = torch.zeros(1 << 23, dtype=torch.int32, device="cuda")
    for k in range(16):
        rc = L.codec_quotient_slice(ctypes.c_uint32(k << 19), ctypes.c_uint32(1 << 19),
                                    ctypes.c_void_p(bad.data_ptr()))
        assert rc == 0
        print(f"quotient slice {k}: {int(bad.sum())} mismatches so far", flush=True)
    b = bad.cpu().numpy()
    assert not b.any(), [hex(0x3F800000 | int(j)) for j in np.nonzero(b)[0][:5]]
