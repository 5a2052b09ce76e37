"""StateArena's slicing on the host (CPU tensors; no GPU call): each tensor's
code records and scales are views of the two shared buffers, of exactly the
layout's sizes, starting on 4096-byte boundaries, in order and disjoint."""
import pytest
import torch

from compressed_adamw_state_amd import flashopt as F

SIZES = [4097, 0, 33, 2048 * 3, 1, (1 << 17) + 5, 32]


@pytest.mark.parametrize("opt", ["adamw", "sgd", "lion", "adamw_linv", "adamw_fp32", "sgd_fp32"])
def test_slices(opt):
    arena = F.StateArena(SIZES, opt, "cpu")
    lib = F.lib()
    kind = F.KIND[opt]
    cbase = arena.codes.data_ptr()
    sbase = arena.scales.data_ptr()
    prev_c = prev_s = 0
    for i, n in enumerate(SIZES):
        st = arena.state(i)
        assert st.numel == n and st.theta.numel() == n and st.theta.dtype == torch.bfloat16
        assert st.codes.numel() == lib.flashopt_codes_bytes(kind, n)
        assert 2 * st.scales.numel() == lib.flashopt_scales_bytes(kind, n)
        assert st.codes.untyped_storage().data_ptr() == cbase          # views, not copies
        assert st.scales.untyped_storage().data_ptr() == sbase
        if n == 0:
            continue                      # an empty view's data_ptr is 0, as for any empty tensor
        co = st.codes.data_ptr() - cbase
        assert co % F.StateArena.ALIGN == 0 and co >= prev_c           # aligned, in order, disjoint
        prev_c = co + st.codes.numel()
        if st.scales.numel():                                           # the FP32 kinds have none
            so = st.scales.data_ptr() - sbase
            assert so % F.StateArena.ALIGN == 0 and so >= prev_s
            prev_s = so + 2 * st.scales.numel()
        assert not st.codes.any() and not st.scales.any()               # zeroed
    assert prev_c <= arena.codes.numel() and prev_s <= 2 * arena.scales.numel()


def test_theta_taken_and_checked():
    arena = F.StateArena([10, 20], "adamw", "cpu")
    th = torch.zeros(20, dtype=torch.bfloat16)
    st = arena.state(1, theta=th)
    assert st.theta.data_ptr() == th.data_ptr()
    with pytest.raises(ValueError):
        arena.state(0, theta=torch.zeros(11, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        F.TensorState(10, "adamw", "cpu", codes=torch.zeros(7, dtype=torch.uint8))
    with pytest.raises(ValueError):
        F.TensorState(10, "adamw", "cpu", scales=torch.zeros(3, dtype=torch.int32))


def test_empty_list():
    arena = F.StateArena([], "adamw", "cpu")
    assert arena.codes.numel() >= 1 and arena.scales.numel() >= 1
