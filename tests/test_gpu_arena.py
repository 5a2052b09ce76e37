"""StateArena's placement search on the device: the kept allocation is the
one whose probe was fastest, its codes and scales are zero, and the state
built on it steps bit for bit as on a plain arena."""
import numpy as np
import pytest
import torch

from compressed_adamw_state_amd import flashopt as F

SIZES = [4101, 33, 2048 * 5, 70000, 1]
HP = {"adamw": dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
      "sgd": dict(lr=0.1, momentum=0.9, weight_decay=1e-4),
      "lion": dict(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.1)}
STEP = {"adamw": F.flashopt_adamw_step, "sgd": F.flashopt_sgd_step, "lion": F.flashopt_lion_step}


def _build(kind, candidates):
    arena = F.StateArena(SIZES, kind, "cuda", theta=True, grad_sets=1, candidates=candidates)
    gen = torch.Generator(device="cuda").manual_seed(3)
    states, grads = [], []
    for i, n in enumerate(SIZES):
        assert not arena.state(i).codes.any() and not arena.state(i).scales.any()
        st = arena.state(i)
        F.flashopt_tensor_init(st, torch.randn(n, device="cuda", generator=gen) * 0.02)
        states.append(st)
        grads.append(arena.grad(0, i).copy_(
            (torch.randn(n, device="cuda", generator=gen) * 1e-3).to(torch.bfloat16)))
    return arena, states, F.FlashoptList(states, grads)


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["adamw", "sgd", "lion"])
def test_placement_search_keeps_the_fastest_and_steps_identically(kind):
    plain, sp, lp = _build(kind, 1)
    assert plain.placement_ms is None and plain.placement_choice is None
    searched, ss, ls = _build(kind, 3)
    ms = searched.placement_ms
    assert len(ms) == 3 and all(m > 0 for m in ms)
    assert searched.placement_choice == int(np.argmin(ms))
    for t in (1, 2, 3):
        STEP[kind](lp, HP[kind], t)
        STEP[kind](ls, HP[kind], t)
    torch.cuda.synchronize()
    for a, b in zip(sp, ss):
        assert torch.equal(a.theta.view(torch.int16), b.theta.view(torch.int16))
        assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
