"""Parity at full size, every element: the fused step over the GPT-2-small
(124 M parameters), Llama-3.1-8B (8.03 B; AdamW and Lion) and Llama-2-13B
(13.0 B, gradient release) workloads, in the launch configuration the
benchmark times, against
the oracle ("FlashOptim: Optimizers for Memory Efficient Training", digest
page, "Core method > Fused optimizer step", Alg. 4).

Each workload runs its whole trajectory on the GPU.  At the checked steps
every element is compared: the device state before the step is copied aside,
the oracle steps every tensor from that copy with the step's gradient (host
threads over whole 32-element groups), and every byte of theta', rho, the
momentum and variance codes and both FP16 scales must equal the device state
after the step.  The other steps keep the sampled comparison (the first, the
last and random groups of every tensor, stepped by the oracle through the
whole trajectory).  One test per checked step (each one advances the shared
run to the step before), so that no test runs for minutes without output."""
import pytest
import torch

from compressed_adamw_state_amd import workloads as W

from parity import Run, log

pytestmark = pytest.mark.gpu


def _run(name, samples):
    r = Run(W.WORKLOADS[name], "sampled", samples_per_tensor=samples)
    log(f"{name}: state built ({r.w.numel} parameters, {len(r.w.tensors)} tensors)")
    return r


def _check(r, t, label, compare_every):
    r.advance_to(t - 1, compare_every, label)
    n = r.step(t, every_element=True)
    log(f"{label} step {t}: {n} of {r.w.numel} elements compared, all equal")
    assert n == r.w.numel
    n = r.compare(f"{label} step {t}")                 # the sampled trajectory too


def _free(r):
    del r
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class TestGPT2Small:
    """GPT-2 small, AdamW, 100 steps: every element at steps 1, 50 and 100."""

    @pytest.fixture(scope="class")
    def run(self):
        r = _run("gpt2_small", 6)
        yield r
        _free(r)

    @pytest.mark.parametrize("t", [1, 50, 100])
    def test_every_element(self, run, t):
        _check(run, t, "gpt2", 25)


class TestLlama31_8B:
    """Llama-3.1-8B, AdamW, 20 steps in the benchmark's launch (one launch
    over the whole list): every element at steps 1 and 20."""

    @pytest.fixture(scope="class")
    def run(self):
        r = _run("llama31_8b", 4)
        yield r
        _free(r)

    @pytest.mark.parametrize("t", [1, 20])
    def test_every_element(self, run, t):
        _check(run, t, "llama8b", 5)


class TestLlama31_8B_Lion:
    """Llama-3.1-8B, Lion (the 16-byte code records), in the benchmark's
    launch: every element at the first and the last step."""

    @pytest.fixture(scope="class")
    def run(self):
        r = _run("llama31_8b_lion", 4)
        yield r
        _free(r)

    @pytest.mark.parametrize("t", [1, W.WORKLOADS["llama31_8b_lion"].steps])
    def test_every_element(self, run, t):
        _check(run, t, "llama8b lion", 5)


class TestLlama2_13B_Release:
    """Llama-2-13B, AdamW in gradient-release mode (one launch per tensor,
    backward order), with special weights and mixed gradients, 10 steps:
    every element at steps 1 and 10."""

    @pytest.fixture(scope="class")
    def run(self):
        r = _run("llama2_13b", 4)
        yield r
        _free(r)

    @pytest.mark.parametrize("t", [1, 10])
    def test_every_element(self, run, t):
        _check(run, t, "llama13b release", 3)
