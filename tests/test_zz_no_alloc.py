"""flashopt_adamw_step_noalloc (include/flashopt.h), the whole-list AdamW step
for callers that cannot allocate device memory: its descriptor table lives in
the library's own device array.  Against the list-handle step
(flashopt_list_create + flashopt_adamw_step) on identical copies of the
state: every byte of theta', the code records and the scales is equal, on two
calls in a row, the second over a smaller list (the array keeps the first
call's larger table; the second must use only its own entries)."""
import numpy as np
import pytest
import torch

from compressed_adamw_state_amd import flashopt as F

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _pair(sizes, seed):
    """Two identical compressed states over `sizes` and one gradient set."""
    gen = torch.Generator().manual_seed(seed)
    a, b, grads = [], [], []
    for n in sizes:
        theta = (torch.randn(n, generator=gen) * 0.02).cuda()
        sa, sb = F.TensorState(n, "adamw", "cuda"), F.TensorState(n, "adamw", "cuda")
        F.flashopt_tensor_init(sa, theta)
        F.flashopt_tensor_init(sb, theta)
        a.append(sa)
        b.append(sb)
        grads.append((torch.randn(n, generator=gen) * 1e-3).to(torch.bfloat16).cuda())
    return a, b, grads


def _assert_equal(a, b, label):
    for i, (sa, sb) in enumerate(zip(a, b)):
        assert torch.equal(sa.theta.view(torch.int16), sb.theta.view(torch.int16)), (label, i)
        assert torch.equal(sa.codes, sb.codes), (label, i)
        assert torch.equal(sa.scales, sb.scales), (label, i)


def test_noalloc_step_equals_the_list_step_on_two_calls():
    rng = np.random.default_rng(21)
    # call 1: 300 tensors (six fill launches of 56 descriptors), ragged sizes,
    # empty tensors, and one tensor large enough for several tiles
    sizes1 = [int(x) for x in rng.integers(0, 5000, 300)] + [0, 1, 31, 33, 2048 * 9 + 5]
    sizes2 = [100, 2048, 7, 4097, 0, 65, 3000]                 # call 2: smaller
    a1, b1, g1 = _pair(sizes1, 22)
    a2, b2, g2 = _pair(sizes2, 23)
    lst1 = F.FlashoptList(b1, g1)
    lst2 = F.FlashoptList(b2, g2)
    for t in (1, 2):
        if t == 2:                    # after one round of the same calls: nothing allocated
            torch.cuda.synchronize()
            free0, reserved0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_reserved()
        F.flashopt_adamw_step_noalloc(a1, g1, HP, t)
        F.flashopt_adamw_step_noalloc(a2, g2, HP, t)
        if t == 2:
            torch.cuda.synchronize()
            assert torch.cuda.mem_get_info()[0] == free0
            assert torch.cuda.memory_reserved() == reserved0
        F.step(lst1, "adamw", HP, t)
        F.step(lst2, "adamw", HP, t)
        torch.cuda.synchronize()
        _assert_equal(a1, b1, f"first list, step {t}")
        _assert_equal(a2, b2, f"second list, step {t}")


def test_noalloc_step_with_the_largest_list():
    """FLASHOPT_NOALLOC_MAX_TENSORS tensors (the array's full size), then one
    tensor: both equal to the list step."""
    sizes = [64 + (i % 7) * 33 for i in range(F.NOALLOC_MAX_TENSORS)]
    a, b, g = _pair(sizes, 24)
    lst = F.FlashoptList(b, g)
    F.flashopt_adamw_step_noalloc(a, g, HP, 1)
    F.step(lst, "adamw", HP, 1)
    torch.cuda.synchronize()
    _assert_equal(a, b, "largest list")
    a, b, g = _pair([5000], 25)
    lst = F.FlashoptList(b, g)
    F.flashopt_adamw_step_noalloc(a, g, HP, 3)
    F.step(lst, "adamw", HP, 3)
    torch.cuda.synchronize()
    _assert_equal(a, b, "one tensor after the largest list")
