"""StateArena's slicing on the host (CPU tensors; no GPU call): each tensor's
codes, scales and (when asked) theta' and gradient buffers are views
of the one shared buffer, of exactly the layout's sizes, starting on
4096-byte boundaries, disjoint, one region per stream in a fixed order."""
import pytest
import torch

from compressed_adamw_state_amd import flashopt as F

SIZES = [4097, 0, 33, 2048 * 3, 1, (1 << 17) + 5, 32]


@pytest.mark.parametrize("opt", ["adamw", "sgd", "lion", "adamw_linv", "adamw_fp32", "sgd_fp32"])
@pytest.mark.parametrize("theta,grad_sets", [(False, 0), (True, 2)])
def test_slices(opt, theta, grad_sets):
    arena = F.StateArena(SIZES, opt, "cpu", theta=theta, grad_sets=grad_sets)
    lib = F.lib()
    kind = F.KIND[opt]
    base = arena.buffer.data_ptr()
    end = base + arena.buffer.numel()
    views = []                                    # (stream, start, bytes)
    for i, n in enumerate(SIZES):
        st = arena.state(i)
        assert st.numel == n and st.theta.numel() == n and st.theta.dtype == torch.bfloat16
        assert st.codes.numel() == lib.flashopt_codes_bytes(kind, n)
        assert 2 * st.scales.numel() == lib.flashopt_scales_bytes(kind, n)
        for t in [st.codes, st.scales] + ([st.theta] if theta else []):
            assert t.untyped_storage().data_ptr() == base            # views, not copies
        if n == 0:
            continue                      # an empty view's data_ptr is 0, as for any empty tensor
        arrays = [("codes", st.codes)] + ([("scales", st.scales)] if st.scales.numel() else [])
        if theta:
            arrays.append(("theta", st.theta))
        for j in range(grad_sets):
            g = arena.grad(j, i)
            assert g.dtype == torch.bfloat16 and g.numel() == n
            assert g.untyped_storage().data_ptr() == base
            arrays.append((f"grad{j}", g))
        for name, t in arrays:
            views.append((name, t.data_ptr(), t.numel() * t.element_size()))
        assert not st.codes.any() and not st.scales.any()               # zeroed
    # aligned, inside the buffer, disjoint; each stream's slices in tensor order
    # within one region, regions in the order theta, grads, codes, scales
    for name, p, b in views:
        assert (p - base) % F.StateArena.ALIGN == 0 and base <= p and p + b <= end
    iv = sorted((p, p + b) for _, p, b in views)
    assert all(a[1] <= c[0] for a, c in zip(iv, iv[1:]))
    order = ["theta"] + [f"grad{j}" for j in range(grad_sets)] + ["codes", "scales"]
    first = {}
    for name, p, b in views:
        first.setdefault(name, p)
        assert p >= first[name]
    present = [o for o in order if o in first]
    assert [first[o] for o in present] == sorted(first[o] for o in present)
    for o in present:
        assert (first[o] - base) % F.StateArena.REGION == 0


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
    arena = F.StateArena([], "adamw", "cpu", theta=True, grad_sets=1)
    assert arena.buffer.numel() >= 1


@pytest.mark.parametrize("opt,theta,grad_sets", [("adamw_fp32", True, 1), ("lion_fp32", True, 1),
                                                 ("adamw", False, 1), ("sgd", True, 0)])
def test_placement_search_needs_a_compressed_arena_with_theta_and_grads(opt, theta, grad_sets):
    # refused on the host, before any allocation: the search times the step's
    # own probe (compressed kinds only), which reads theta' and a gradient
    with pytest.raises(ValueError, match="placement search"):
        F.StateArena(SIZES, opt, "cpu", theta=theta, grad_sets=grad_sets, candidates=2)


def test_placement_search_needs_a_gpu_arena():
    with pytest.raises(ValueError, match="GPU arena"):
        F.StateArena(SIZES, "adamw", "cpu", theta=True, grad_sets=1, candidates=2)
