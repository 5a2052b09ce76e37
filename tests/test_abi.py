"""The C-ABI library loads, exports every symbol include/*.h declares,
and validates arguments on the host (no GPU call is made by these tests:
every case fails validation before any HIP call)."""
import ctypes
import os
import re

import pytest
import torch


from compressed_adamw_state_amd import flashopt as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(flashopt_\w+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol():
    lib = F.lib()
    names = declared_symbols()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(F.SIGNATURES), set(names) ^ set(F.SIGNATURES)


def test_status_strings():
    lib = F.lib()
    for s in range(-9, 1):
        assert lib.flashopt_status_string(s) != b"unknown status"
        assert s in F.STATUS
    assert lib.flashopt_status_string(0) == b"ok"
    assert lib.flashopt_status_string(-10) == b"unknown status"


def test_host_validation_without_gpu():
    lib = F.lib()
    P = ctypes.c_void_p
    fake = P(0x10000)                                  # never dereferenced: validation fails first
    mis = P(0x10001)
    assert lib.flashopt_split(None, 10, fake, fake, None) == -1
    assert lib.flashopt_split(fake, -1, fake, fake, None) == -2
    assert lib.flashopt_split(mis, 10, fake, fake, None) == -3
    assert lib.flashopt_split(fake, 0, None, None, None) == 0   # empty: nothing to do
    assert lib.flashopt_unsplit(fake, fake, 5, mis, None) == -3
    assert lib.flashopt_quantize_m(fake, 5, None, fake, None) == -1
    assert lib.flashopt_dequantize_v(fake, P(0x10003), 5, fake, None) == -3
    assert lib.flashopt_split_ex(fake, 10, 2, 127, fake, fake, None) == -4      # base
    assert lib.flashopt_split_ex(fake, 10, 1, 0, fake, fake, None) == -4       # qmax
    assert lib.flashopt_split_ex(fake, 10, 1, 32768, fake, fake, None) == -4
    assert lib.flashopt_split_ex(None, 10, 1, 127, fake, fake, None) == -1
    # the step that allocates nothing: count range, NULL array, hyper-parameters,
    # and the list checks of every descriptor, all before any HIP call
    hp = F.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    one = (F.Tensor * 1)(F.Tensor(10, fake, fake, fake, fake))
    noalloc = lib.flashopt_adamw_step_noalloc
    assert noalloc(one, F.NOALLOC_MAX_TENSORS + 1, ctypes.byref(hp), 1, None) == -2
    assert noalloc(one, -1, ctypes.byref(hp), 1, None) == -2
    assert noalloc(None, 3, ctypes.byref(hp), 1, None) == -1
    assert noalloc(one, 1, ctypes.byref(hp), 0, None) == -5
    bad = F.AdamWHparams(1e-3, 1.0, 0.999, 1e-8, 0.01)
    assert noalloc(one, 1, ctypes.byref(bad), 1, None) == -4
    assert noalloc((F.Tensor * 1)(F.Tensor(10, fake, fake, fake, None)), 1, ctypes.byref(hp), 1,
                   None) == -1                                  # a gradient is required
    assert noalloc((F.Tensor * 1)(F.Tensor(10, mis, fake, fake, fake)), 1, ctypes.byref(hp), 1,
                   None) == -3
    assert noalloc((F.Tensor * 1)(F.Tensor(-1, fake, fake, fake, fake)), 1, ctypes.byref(hp), 1,
                   None) == -2
    assert lib.flashopt_unsplit_ex(fake, P(0x10001), 10, 0, 127, fake, None) == -3
    assert lib.flashopt_quantize_lin_v(fake, 5, None, fake, None) == -1
    assert lib.flashopt_dequantize_lin_m(fake, fake, -1, fake, None) == -2
    assert lib.flashopt_list_workspace_bytes(0) >= 8
    assert lib.flashopt_list_workspace_bytes(291) >= 291 * 64
    out = P()
    A, S = 0, 1                                        # flashopt_kind
    # AdamW: whole 1536-byte blocks of 512 elements; SGD: 16-byte records of 8
    assert lib.flashopt_codes_bytes(A, 17) == 1536 and lib.flashopt_codes_bytes(S, 17) == 3 * 16
    assert lib.flashopt_codes_bytes(A, 513) == 2 * 1536 and lib.flashopt_codes_bytes(A, 0) == 0
    assert lib.flashopt_scales_bytes(A, 33) == 2 * 4 and lib.flashopt_scales_bytes(S, 33) == 2 * 2
    assert lib.flashopt_codes_bytes(7, 17) == 0 and lib.flashopt_scales_bytes(A, -1) == 0
    arr = (F.Tensor * 1)(F.Tensor(10, fake, fake, fake, fake))
    ws = P(0x100000)
    need = lib.flashopt_list_workspace_bytes(1)
    assert lib.flashopt_list_create(arr, 1, A, ws, need - 1, None, ctypes.byref(out)) == -6
    assert lib.flashopt_list_create(arr, 1, A, P(0x100010), need, None, ctypes.byref(out)) == -6
    assert lib.flashopt_list_create(arr, -1, A, ws, need, None, ctypes.byref(out)) == -2
    assert lib.flashopt_list_create(arr, 1, 7, ws, need, None, ctypes.byref(out)) == -4
    nul = (F.Tensor * 1)(F.Tensor(10, fake, None, fake, fake))
    assert lib.flashopt_list_create(nul, 1, A, ws, need, None, ctypes.byref(out)) == -1
    mis_t = (F.Tensor * 1)(F.Tensor(10, P(0x10008), fake, fake, fake))
    assert lib.flashopt_list_create(mis_t, 1, A, ws, need, None, ctypes.byref(out)) == -3
    for k in (A, S, 2):                                # codes: 16 B for every compressed kind
        mis_c = (F.Tensor * 1)(F.Tensor(10, fake, P(0x10008), fake, fake))
        assert lib.flashopt_list_create(mis_c, 1, k, ws, need, None, ctypes.byref(out)) == -3
    mis_s = (F.Tensor * 1)(F.Tensor(10, fake, fake, P(0x10002), fake))  # AdamW scales need 4 B
    assert lib.flashopt_list_create(mis_s, 1, A, ws, need, None, ctypes.byref(out)) == -3
    assert lib.flashopt_list_create(mis_s, 1, 6, ws, need, None, ctypes.byref(out)) == -3
    # the linear-variance ablation kind has the AdamW layout
    assert lib.flashopt_codes_bytes(6, 17) == 1536 and lib.flashopt_scales_bytes(6, 33) == 8
    neg = (F.Tensor * 1)(F.Tensor(-5, fake, fake, fake, fake))
    assert lib.flashopt_list_create(neg, 1, A, ws, need, None, ctypes.byref(out)) == -2
    assert lib.flashopt_tensor_init(arr, 7, fake, None) == -4
    assert lib.flashopt_tensor_init(arr, A, None, None) == -1
    assert lib.flashopt_tensor_init(mis_t, A, fake, None) == -3
    assert lib.flashopt_tensor_export(None, A, fake, None, None, None) == -1
    assert lib.flashopt_tensor_export(arr, A, None, None, None, None) == 0   # nothing requested
    hp = F.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    assert lib.flashopt_adamw_step(None, ctypes.byref(hp), 1, None) == -1
    assert lib.flashopt_stream_probe(None, None) == -1
    # an empty list is created without touching the device
    assert lib.flashopt_list_create(None, 0, A, None, 0, None, ctypes.byref(out)) == 0
    L = out
    assert lib.flashopt_list_numel(L) == 0
    assert lib.flashopt_adamw_step(L, ctypes.byref(hp), 0, None) == -5
    for bad_hp in (F.AdamWHparams(-1, 0.9, 0.999, 1e-8, 0), F.AdamWHparams(1e-3, 1.0, 0.999, 1e-8, 0),
                   F.AdamWHparams(1e-3, 0.9, 0.999, 0.0, 0), F.AdamWHparams(1e-3, 0.9, 0.999, 1e-46, 0),
                   F.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, -1),
                   F.AdamWHparams(float("nan"), 0.9, 0.999, 1e-8, 0)):
        assert lib.flashopt_adamw_step(L, ctypes.byref(bad_hp), 1, None) == -4
    assert lib.flashopt_adamw_step(L, ctypes.byref(hp), 1, None) == 0    # nothing to launch
    # bucketed release over an empty list: only the empty range is valid
    assert lib.flashopt_adamw_step_range(None, 0, 0, None, ctypes.byref(hp), 1, None) == -1
    assert lib.flashopt_adamw_step_range(L, 0, 0, None, ctypes.byref(hp), 1, None) == 0
    assert lib.flashopt_adamw_step_range(L, 0, 1, None, ctypes.byref(hp), 1, None) == -8
    assert lib.flashopt_adamw_step_range(L, -1, 0, None, ctypes.byref(hp), 1, None) == -8
    assert lib.flashopt_adamw_step_range(L, 0, 0, None, ctypes.byref(hp), 0, None) == -5
    assert lib.flashopt_sgd_step_range(L, 0, 0, None, ctypes.byref(F.SGDHparams(0.1, 0.9, 0.0)),
                                       1, None) == -4                     # an AdamW list
    sgd = F.SGDHparams(0.1, 1.0, 0.0)
    assert lib.flashopt_sgd_step(L, ctypes.byref(sgd), 1, None) == -4
    sgd = F.SGDHparams(0.1, 0.9, 0.0)
    assert lib.flashopt_sgd_step(L, ctypes.byref(sgd), 1, None) == -4   # AdamW list
    assert lib.flashopt_adamw_step_one(L, 0, fake, ctypes.byref(hp), 1, None) == -8
    lion = F.LionHparams(1e-4, 0.9, 0.99, 0.1)
    assert lib.flashopt_lion_step(None, ctypes.byref(lion), 1, None) == -1
    assert lib.flashopt_lion_step(L, ctypes.byref(lion), 1, None) == -4     # AdamW list
    assert lib.flashopt_lion_step_one(L, 0, fake, ctypes.byref(lion), 1, None) == -8
    assert lib.flashopt_state_zero(L, None) == 0
    # the device schedule: validated on the host, nothing launched on failure
    assert ctypes.sizeof(F.AdamWSchedule) == 112
    assert lib.flashopt_adamw_schedule_init(None, ctypes.byref(hp), 0, None) == -1
    assert lib.flashopt_adamw_schedule_init(P(0x10004), ctypes.byref(hp), 0, None) == -3
    assert lib.flashopt_adamw_schedule_init(fake, ctypes.byref(hp), -1, None) == -5
    bad = F.AdamWHparams(1e-3, 1.0, 0.999, 1e-8, 0)
    assert lib.flashopt_adamw_schedule_init(fake, ctypes.byref(bad), 0, None) == -4
    assert lib.flashopt_adamw_step_scheduled(L, None, None) == -1
    assert lib.flashopt_adamw_step_scheduled(None, fake, None) == -1
    assert lib.flashopt_adamw_step_scheduled(L, P(0x10004), None) == -3
    assert lib.flashopt_list_destroy(L) == 0
    # an empty Lion list: hyper-parameter and step checks
    assert lib.flashopt_list_create(None, 0, 2, None, 0, None, ctypes.byref(out)) == 0
    L = out
    assert lib.flashopt_lion_step(L, ctypes.byref(lion), 0, None) == -5
    for bad_l in (F.LionHparams(-1, 0.9, 0.99, 0), F.LionHparams(1e-4, 1.0, 0.99, 0),
                  F.LionHparams(1e-4, 0.9, -0.1, 0), F.LionHparams(1e-4, 0.9, 0.99, -1),
                  F.LionHparams(float("inf"), 0.9, 0.99, 0)):
        assert lib.flashopt_lion_step(L, ctypes.byref(bad_l), 1, None) == -4
    assert lib.flashopt_lion_step(L, ctypes.byref(lion), 1, None) == 0      # nothing to launch
    assert lib.flashopt_adamw_step(L, ctypes.byref(hp), 1, None) == -4      # Lion list
    assert lib.flashopt_adamw_step_scheduled(L, fake, None) == -4           # Lion list
    assert lib.flashopt_sgd_step_scheduled(L, fake, None) == -4             # Lion list
    assert ctypes.sizeof(F.SGDSchedule) == 48 and ctypes.sizeof(F.LionSchedule) == 64
    assert lib.flashopt_lion_schedule_init(None, ctypes.byref(lion), 0, None) == -1
    assert lib.flashopt_lion_schedule_init(fake, ctypes.byref(lion), -2, None) == -5
    assert lib.flashopt_lion_schedule_init(P(0x10002), ctypes.byref(lion), 0, None) == -3
    bad_sgd = F.SGDHparams(0.1, 1.5, 0.0)
    assert lib.flashopt_sgd_schedule_init(fake, ctypes.byref(bad_sgd), 0, None) == -4
    assert lib.flashopt_lion_step_scheduled(None, fake, None) == -1
    assert lib.flashopt_codes_bytes(2, 17) == 3 * 16 and lib.flashopt_scales_bytes(2, 33) == 4
    assert lib.flashopt_list_destroy(L) == 0
    # uncompressed kinds: 512-element blocks of 3 (AdamW) or 2 FP32 fields, no scales
    AF, SF, LF = 3, 4, 5
    assert lib.flashopt_codes_bytes(AF, 17) == 6144 and lib.flashopt_codes_bytes(SF, 513) == 8192
    assert lib.flashopt_codes_bytes(LF, 512) == 4096 and lib.flashopt_codes_bytes(AF, 0) == 0
    assert all(lib.flashopt_scales_bytes(k, 33) == 0 for k in (AF, SF, LF))
    no_codes = (F.Tensor * 1)(F.Tensor(10, fake, None, None, fake))
    assert lib.flashopt_list_create(no_codes, 1, AF, ws, need, None, ctypes.byref(out)) == -1
    mis_c = (F.Tensor * 1)(F.Tensor(10, fake, P(0x10008), None, fake))   # records need 16 B
    assert lib.flashopt_list_create(mis_c, 1, AF, ws, need, None, ctypes.byref(out)) == -3
    assert lib.flashopt_tensor_init(mis_c, LF, fake, None) == -3
    assert lib.flashopt_list_create(None, 0, AF, None, 0, None, ctypes.byref(out)) == 0
    L = out
    assert lib.flashopt_adamw_step(L, ctypes.byref(hp), 1, None) == 0       # nothing to launch
    assert lib.flashopt_sgd_step(L, ctypes.byref(sgd), 1, None) == -4       # AdamW list
    assert lib.flashopt_stream_probe(L, None) == -4                         # compressed only
    assert lib.flashopt_state_zero(L, None) == 0
    assert lib.flashopt_list_destroy(L) == 0


def test_schedule_set_checks_ranges_on_the_host():
    """DeviceSchedule.set writes device memory that no kernel validates, so it
    checks each value first (a host buffer stands in for the device one)."""
    for opt, good, bad in (("adamw", [("lr", 0.0), ("eps", 1e-45), ("weight_decay", 0.1)],
                            [("lr", -1.0), ("lr", float("inf")), ("eps", 0.0), ("eps", 1e-46),
                             ("eps", float("nan")), ("weight_decay", -0.1), ("beta1", 0.5)]),
                           ("sgd", [("momentum", 0.0), ("lr", 0.1)],
                            [("momentum", 1.0), ("momentum", -0.1), ("lr", float("nan"))]),
                           ("lion", [("beta1", 0.99), ("beta2", 0.0)],
                            [("beta2", 1.0), ("weight_decay", float("inf"))])):
        s = F.DeviceSchedule.__new__(F.DeviceSchedule)
        s.optimizer = opt
        s.struct = F.DeviceSchedule._STRUCT[opt]
        s.buf = torch.zeros(ctypes.sizeof(s.struct), dtype=torch.uint8)
        for name, v in good:
            s.set(name, v)
            assert getattr(s.read(), name) == v
        for name, v in bad:
            with pytest.raises(ValueError):
                s.set(name, v)
