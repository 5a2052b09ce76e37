"""Synthetic workloads: tensor-list shapes and seeded input generators.

This module holds no arithmetic of the optimizer method.  It only knows the
shapes of the model parameter lists the FlashOptim digest ("FlashOptim:
Optimizers for Memory Efficient Training", experiments section: ResNet-50,
GPT-2, Llama-3.1-8B; Table 4) trains, plus a Llama-2-13B list, and draws
seeded random inputs of the stated distributions with plain torch ops.  Both
the CPU oracle side and the GPU side receive the *same* bits from here.

Every draw is keyed by (workload seed, purpose, step, tensor index) so any
tensor's inputs can be regenerated independently, on any device.  The same
key gives bit-identical values on one device type; across device types the
bits differ (torch's CPU and GPU generators differ), so a parity test that
generates on the GPU copies the sampled inputs back to the host.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence

import torch

GROUP = 32  # elements per quantisation group (companding section: G = 32)


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: tuple
    init: str  # "normal" (N(0, 0.02)), "ones", "zeros"

    @property
    def numel(self) -> int:
        n = 1
        for d in self.shape:
            n *= d
        return n


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tensors: tuple
    optimizer: str          # state kind: "adamw" | "sgd" | "lion", or "<one of them>_fp32"
    steps: int
    seed: int
    grad_dist: str          # see draw_grad
    grad_scale: float
    hparams: dict
    release: bool = False   # gradient-release mode: one step call per tensor
    special_theta: bool = False

    @property
    def numel(self) -> int:
        return sum(t.numel for t in self.tensors)

    @property
    def groups(self) -> int:
        return sum((t.numel + GROUP - 1) // GROUP for t in self.tensors)


ADAMW_HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
SGD_HP = dict(lr=0.1, momentum=0.9, weight_decay=1e-4)
# Lion: the published rule's usual setting (a smaller lr and a larger decay than AdamW)
LION_HP = dict(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.1)
HPARAMS = {"adamw": ADAMW_HP, "sgd": SGD_HP, "lion": LION_HP, "adamw_linv": ADAMW_HP}


def gpt2_small() -> List[TensorSpec]:
    d, v, ctx, ff = 768, 50257, 1024, 3072
    t = [TensorSpec("wte", (v, d), "normal"), TensorSpec("wpe", (ctx, d), "normal")]
    for i in range(12):
        p = f"h{i}."
        t += [
            TensorSpec(p + "ln_1.weight", (d,), "ones"),
            TensorSpec(p + "ln_1.bias", (d,), "zeros"),
            TensorSpec(p + "attn.c_attn.weight", (d, 3 * d), "normal"),
            TensorSpec(p + "attn.c_attn.bias", (3 * d,), "zeros"),
            TensorSpec(p + "attn.c_proj.weight", (d, d), "normal"),
            TensorSpec(p + "attn.c_proj.bias", (d,), "zeros"),
            TensorSpec(p + "ln_2.weight", (d,), "ones"),
            TensorSpec(p + "ln_2.bias", (d,), "zeros"),
            TensorSpec(p + "mlp.c_fc.weight", (d, ff), "normal"),
            TensorSpec(p + "mlp.c_fc.bias", (ff,), "zeros"),
            TensorSpec(p + "mlp.c_proj.weight", (ff, d), "normal"),
            TensorSpec(p + "mlp.c_proj.bias", (d,), "zeros"),
        ]
    t += [TensorSpec("ln_f.weight", (d,), "ones"), TensorSpec("ln_f.bias", (d,), "zeros")]
    return t


def resnet50() -> List[TensorSpec]:
    t = [TensorSpec("conv1.weight", (64, 3, 7, 7), "normal")]
    t += [TensorSpec("bn1.weight", (64,), "ones"), TensorSpec("bn1.bias", (64,), "zeros")]
    cin = 64
    for li, (blocks, width) in enumerate(zip((3, 4, 6, 3), (64, 128, 256, 512))):
        for b in range(blocks):
            p = f"layer{li + 1}.{b}."
            cout = 4 * width
            t += [TensorSpec(p + "conv1.weight", (width, cin, 1, 1), "normal"),
                  TensorSpec(p + "bn1.weight", (width,), "ones"),
                  TensorSpec(p + "bn1.bias", (width,), "zeros"),
                  TensorSpec(p + "conv2.weight", (width, width, 3, 3), "normal"),
                  TensorSpec(p + "bn2.weight", (width,), "ones"),
                  TensorSpec(p + "bn2.bias", (width,), "zeros"),
                  TensorSpec(p + "conv3.weight", (cout, width, 1, 1), "normal"),
                  TensorSpec(p + "bn3.weight", (cout,), "ones"),
                  TensorSpec(p + "bn3.bias", (cout,), "zeros")]
            if b == 0:
                t += [TensorSpec(p + "downsample.0.weight", (cout, cin, 1, 1), "normal"),
                      TensorSpec(p + "downsample.1.weight", (cout,), "ones"),
                      TensorSpec(p + "downsample.1.bias", (cout,), "zeros")]
            cin = cout
    t += [TensorSpec("fc.weight", (1000, 2048), "normal"), TensorSpec("fc.bias", (1000,), "zeros")]
    return t


def llama(layers: int, d: int, kv: int, ff: int, vocab: int) -> List[TensorSpec]:
    t = [TensorSpec("embed_tokens.weight", (vocab, d), "normal")]
    for i in range(layers):
        p = f"layers.{i}."
        t += [TensorSpec(p + "input_layernorm.weight", (d,), "ones"),
              TensorSpec(p + "self_attn.q_proj.weight", (d, d), "normal"),
              TensorSpec(p + "self_attn.k_proj.weight", (kv, d), "normal"),
              TensorSpec(p + "self_attn.v_proj.weight", (kv, d), "normal"),
              TensorSpec(p + "self_attn.o_proj.weight", (d, d), "normal"),
              TensorSpec(p + "post_attention_layernorm.weight", (d,), "ones"),
              TensorSpec(p + "mlp.gate_proj.weight", (ff, d), "normal"),
              TensorSpec(p + "mlp.up_proj.weight", (ff, d), "normal"),
              TensorSpec(p + "mlp.down_proj.weight", (d, ff), "normal")]
    t += [TensorSpec("norm.weight", (d,), "ones"), TensorSpec("lm_head.weight", (vocab, d), "normal")]
    return t


def llama31_8b() -> List[TensorSpec]:
    return llama(32, 4096, 1024, 14336, 128256)


def llama2_13b() -> List[TensorSpec]:
    return llama(40, 5120, 5120, 13824, 32000)


WORKLOADS = {
    "flat1m": Workload("flat1m", (TensorSpec("flat", (1 << 20,), "normal"),), "adamw", 10, 0,
                       "normal", 1e-3, ADAMW_HP),
    "gpt2_small": Workload("gpt2_small", tuple(gpt2_small()), "adamw", 100, 1,
                           "student_t3", 1e-3, ADAMW_HP),
    "resnet50": Workload("resnet50", tuple(resnet50()), "sgd", 20, 2, "normal", 1e-2, SGD_HP),
    "llama31_8b": Workload("llama31_8b", tuple(llama31_8b()), "adamw", 20, 3, "normal", 1e-4,
                           ADAMW_HP),
    "llama2_13b": Workload("llama2_13b", tuple(llama2_13b()), "adamw", 10, 4, "mixed", 1e-4,
                           ADAMW_HP, release=True, special_theta=True),
    # FlashLion at the Llama-3.1-8B shapes (the one-momentum layout, 10.125 B/param)
    "llama31_8b_lion": Workload("llama31_8b_lion", tuple(llama31_8b()), "lion", 20, 5, "normal",
                                1e-4, LION_HP),
    # compression switched off for every layer: FP32 master weight and moments
    "llama31_8b_adamw_fp32": Workload("llama31_8b_adamw_fp32", tuple(llama31_8b()), "adamw_fp32",
                                      20, 6, "normal", 1e-3, ADAMW_HP),
}


def ragged(sizes: Sequence[int], seed: int = 7, steps: int = 3, optimizer: str = "adamw",
           grad_scale: float = 1e-3) -> Workload:
    """A list of 1-D tensors of arbitrary sizes (tail-group coverage)."""
    t = tuple(TensorSpec(f"t{i}", (n,), "normal") for i, n in enumerate(sizes))
    return Workload(f"ragged{len(sizes)}", t, optimizer, steps, seed, "normal", grad_scale,
                    HPARAMS[optimizer])


# ---------------------------------------------------------------------------
# seeded draws

_PURPOSE = {"theta": 1, "grad": 2, "special": 3, "weights": 4, "moments": 5}


def _gen(seed: int, purpose: str, step: int, index: int, device) -> torch.Generator:
    key = (((seed * 1000003 + _PURPOSE[purpose]) * 1000003 + step) * 1000003 + index)
    key &= (1 << 63) - 1
    g = torch.Generator(device=device)
    g.manual_seed(key)
    return g


def draw_theta(w: Workload, index: int, device="cpu") -> torch.Tensor:
    """Initial fp32 master weight of tensor `index` (flattened)."""
    spec = w.tensors[index]
    n = spec.numel
    if spec.init == "ones":
        x = torch.ones(n, dtype=torch.float32, device=device)
    elif spec.init == "zeros":
        x = torch.zeros(n, dtype=torch.float32, device=device)
    else:
        g = _gen(w.seed, "theta", 0, index, device)
        x = torch.randn(n, generator=g, dtype=torch.float32, device=device) * 0.02
    if w.special_theta and n > 0:
        g = _gen(w.seed, "special", 0, index, device)
        u = torch.rand(n, generator=g, device=device)
        bits = x.view(torch.int32)
        # 0.1%: exactly on a bf16 half-ULP boundary (lower 16 bits = 0x8000)
        tie = u < 1e-3
        bits = torch.where(tie, (bits & ~0xFFFF) | 0x8000, bits)
        # 0.1%: an fp32 subnormal (exponent field 0, random mantissa and sign)
        sub = (u >= 1e-3) & (u < 2e-3)
        mant = (torch.randint(1, 1 << 23, (n,), generator=g, device=device, dtype=torch.int32))
        sbits = (bits & (-0x80000000)) | mant
        bits = torch.where(sub, sbits, bits)
        x = bits.view(torch.float32)
    return x


def draw_grad(w: Workload, index: int, step: int, device="cpu") -> torch.Tensor:
    """bf16 gradient of tensor `index` at 1-based `step` (flattened)."""
    n = w.tensors[index].numel
    g = _gen(w.seed, "grad", step, index, device)
    if w.grad_dist == "normal":
        x = torch.randn(n, generator=g, dtype=torch.float32, device=device) * w.grad_scale
    elif w.grad_dist == "student_t3":
        z = torch.randn(n, generator=g, dtype=torch.float32, device=device)
        c = torch.randn(3, n, generator=g, dtype=torch.float32, device=device)
        chi2 = (c * c).sum(0)
        x = z / torch.sqrt(chi2 / 3.0) * w.grad_scale
    elif w.grad_dist == "mixed":
        x = torch.randn(n, generator=g, dtype=torch.float32, device=device) * w.grad_scale
        u = torch.rand(n, generator=g, device=device)
        x = torch.where(u < 1e-3, x * 1e3, x)                      # 0.1% outliers x1e3
        x = torch.where((u >= 1e-3) & (u < 1.1e-2), torch.zeros_like(x), x)  # 1% exact zeros
        sub = (u >= 1.1e-2) & (u < 1.2e-2)                         # 0.1% bf16 subnormals
        mant = torch.randint(1, 1 << 7, (n,), generator=g, device=device, dtype=torch.int32)
        sbits = (x.view(torch.int32) & (-0x80000000)) | (mant << 16)
        x = torch.where(sub, sbits.view(torch.float32), x)
    else:
        raise ValueError(w.grad_dist)
    return x.to(torch.bfloat16)


def draw_weights(n: int, seed: int, device="cpu") -> torch.Tensor:
    """fp32 weights N(0, 0.02), the initialisation of the transformer lists."""
    g = _gen(seed, "weights", 0, 0, device)
    return torch.randn(n, generator=g, dtype=torch.float32, device=device) * 0.02


def draw_moments(n: int, seed: int, scale: float, spread: float, device="cpu"):
    """(m, v) fp32 of the kind an AdamW run holds, drawn directly.

    Each element has its own gradient scale s = scale * exp(spread * z),
    z ~ N(0, 1) (log-normal, so one group of 32 mixes scales); the first
    moment is 0.23 * s * N(0, 1) (an exponential average with decay 0.9 of
    white noise has 0.23 of the noise's standard deviation) and the second
    s^2 * chi2_8 / 8 (an average of squares that still fluctuates)."""
    g = _gen(seed, "moments", 0, 0, device)
    s = scale * torch.exp(spread * torch.randn(n, generator=g, dtype=torch.float64, device=device))
    m = 0.23 * s * torch.randn(n, generator=g, dtype=torch.float64, device=device)
    c = torch.randn(8, n, generator=g, dtype=torch.float64, device=device)
    v = s * s * (c * c).sum(0) / 8.0
    return m.float(), v.float()


def state_bytes(numel: int, optimizer: str = "adamw") -> dict:
    """Byte accounting of the compressed layout for one tensor (Table 4 pins)."""
    groups = (numel + GROUP - 1) // GROUP
    out = {"theta_bf16": 2 * numel, "rho": numel, "m_code": numel, "m_scale": 2 * groups}
    if optimizer == "adamw":
        out.update(v_code=numel, v_scale=2 * groups)
    return out
