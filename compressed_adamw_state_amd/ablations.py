"""Codec ablations of FlashOptim ("FlashOptim: Optimizers for Memory Efficient
Training"), measured on the GPU through the C ABI.

* Weight splitting (Core method > Weight splitting, Eq. 1-2; Sec. 4.4 and
  Fig. 3): the rebuild error of theta' + rho for a BF16 or FP16 base weight
  and a correction of b = 0, 4, 8, 12 or 16 bits (qmax = 2^(b-1) - 1; b = 0
  keeps theta' alone), over N(0, 0.02) weights and exhaustively over every
  FP32 value of each binade from 2^-24 to 2^16, beside the BF16 + BF16 scheme
  the figure compares with (theta' plus theta - theta' rounded to BF16).
* Optimizer-state quantisation (Companding, Fig. 4-5): the error of 8-bit
  group quantisation of m and v with the softsign / square-root companding
  the step uses and without it (linear codes over the same FP16 group
  scale), over moments drawn with log-normal per-element scales: the NMSE,
  its distribution over groups of 32, and the share of nonzero values that
  come back as 0.

* Training without companding (Fig. 5): a small MLP on a synthetic
  regression task trained with torch's AdamW on FP32 weights (the
  reference), with FlashAdamW, and with FlashAdamW whose variance is stored
  by linear codes (the fused step's ablation kind); the page reports that
  the last diverges.

Every codec operation runs in the library's kernels; the error statistics
are plain torch reductions over their outputs, and the BF16 + BF16 baseline
is two torch casts.  python -m compressed_adamw_state_amd.ablations prints
the study as JSON.
"""
from __future__ import annotations

import argparse
import json

import torch

from . import flashopt as F
from . import workloads as W

QMAX = (0, 7, 127, 2047, 32767)          # b = 0, 4, 8, 12, 16 correction bits
BASES = ("bf16", "fp16")
BINADES = range(103, 143)                # exponent fields: [2^-24, 2^16)
FP16_MIN_NORMAL = 2.0 ** -14
GROUP = 32


def rebuild(x: torch.Tensor, base: str, qmax: int) -> torch.Tensor:
    """theta_hat from split_ex then unsplit_ex of fp32 x (qmax 0: rho = 0)."""
    n = x.numel()
    tb = torch.empty(n, dtype=torch.int16, device=x.device)
    rho = torch.empty(n, dtype=torch.int16, device=x.device)
    F.flashopt_split_ex(x, base, max(qmax, 1), tb, rho)
    if qmax == 0:
        rho.zero_()
    y = torch.empty_like(x)
    F.flashopt_unsplit_ex(tb, rho, base, max(qmax, 1), y)
    return y


def rebuild_bf16_bf16(x: torch.Tensor) -> torch.Tensor:
    """The baseline: BF16 weight plus the residual stored as BF16."""
    tb = x.to(torch.bfloat16)
    r = (x - tb.float()).to(torch.bfloat16)
    return tb.float() + r.float()


def split_errors(x: torch.Tensor, y: torch.Tensor) -> dict:
    """Mean and max relative error over the x != 0 rebuilt as finite values,
    the share rebuilt bit for bit, and the share whose base overflowed (an
    FP16 base rounds |x| >= 65520 to Inf and keeps no correction)."""
    x64 = x.double()
    ok = (x64 != 0) & torch.isfinite(y)
    d = (y.double() - x64).abs()
    rel = d[ok] / x64[ok].abs()
    return {"mean_rel": rel.mean().item(), "max_rel": rel.max().item(),
            "bit_exact": (y.view(torch.int32) == x.view(torch.int32)).double().mean().item(),
            "overflow": (~torch.isfinite(y)).double().mean().item()}


def quant_errors(x: torch.Tensor, back: torch.Tensor) -> dict:
    """NMSE, quantiles of the per-group NMSE, share of nonzeros sent to 0."""
    x64, b64 = x.double(), back.double()
    e2 = (b64 - x64) ** 2
    ng = x.numel() // GROUP
    ge = e2[: ng * GROUP].view(ng, GROUP).sum(1)
    gx = (x64[: ng * GROUP] ** 2).view(ng, GROUP).sum(1)
    gn = (ge[gx > 0] / gx[gx > 0]).float()
    qs = torch.quantile(gn, torch.tensor([0.5, 0.9, 0.99], device=gn.device)).tolist()
    nz = x64 != 0
    return {"nmse": (e2.sum() / (x64 ** 2).sum()).item(),
            "group_nmse_p50": qs[0], "group_nmse_p90": qs[1], "group_nmse_p99": qs[2],
            "zeroed": ((b64 == 0) & nz).sum().item() / max(nz.sum().item(), 1)}


def _quant_roundtrip(x: torch.Tensor, which: str, companded: bool) -> torch.Tensor:
    n = x.numel()
    q = torch.empty(n, dtype=torch.int8 if which == "m" else torch.uint8, device=x.device)
    s = torch.empty((n + GROUP - 1) // GROUP, dtype=torch.int16, device=x.device)
    back = torch.empty_like(x)
    if which == "m":
        quant, dequant = ((F.flashopt_quantize_m, F.flashopt_dequantize_m) if companded else
                          (F.flashopt_quantize_lin_m, F.flashopt_dequantize_lin_m))
    else:
        quant, dequant = ((F.flashopt_quantize_v, F.flashopt_dequantize_v) if companded else
                          (F.flashopt_quantize_lin_v, F.flashopt_dequantize_lin_v))
    quant(x, q, s)
    dequant(q, s, back)
    return back


# moment cases: (state, gradient scale, log-normal spread).  "m_unit" holds
# momenta near 0.2, where the softsign is no longer linear; "v_small" holds the
# variances of gradients near 1e-5, below the FP16 scale's reach when stored
# linearly
QUANT_CASES = {"m": ("m", 1e-3, 0.5), "m_unit": ("m", 1.0, 0.5), "v": ("v", 1e-3, 0.5),
               "v_wide": ("v", 1e-3, 1.0), "v_small": ("v", 1e-5, 0.5)}


def run(n: int = 1 << 22, seed: int = 0, device: str = "cuda", binades=BINADES) -> dict:
    """The whole study.  Inputs are drawn on the host (seeded) and copied."""
    out = {"n": n, "seed": seed}
    w = W.draw_weights(n, seed).to(device)
    w = w[w.abs() >= FP16_MIN_NORMAL].contiguous()       # both bases hold these as normals
    out["split"] = {b: {str(q): split_errors(w, rebuild(w, b, q)) for q in QMAX} for b in BASES}
    out["bf16_bf16"] = split_errors(w, rebuild_bf16_bf16(w))
    sweep = {}
    mant = torch.arange(1 << 23, dtype=torch.int32, device=device)
    for e in binades:
        x = (mant | (e << 23)).view(torch.float32)
        row = {f"{b}/{q}": split_errors(x, rebuild(x, b, q)) for b in BASES for q in QMAX[1:]}
        row["bf16_bf16"] = split_errors(x, rebuild_bf16_bf16(x))
        sweep[str(e - 127)] = row
    out["split_by_binade"] = sweep
    quant = {}
    for name, (which, scale, spread) in QUANT_CASES.items():
        m, v = W.draw_moments(n, seed, scale, spread)
        x = (m if which == "m" else v).to(device)
        quant[name] = {"scale": scale, "spread": spread,
                       "companded": quant_errors(x, _quant_roundtrip(x, which, True)),
                       "linear": quant_errors(x, _quant_roundtrip(x, which, False))}
    out["quant"] = quant
    return out


def _mlp_task(seed: int, device: str):
    """Synthetic regression: y = sin(3 x.a) + noise, x in R^64, 4096 samples;
    a 64-256-1 ReLU MLP.  Drawn on the host (seeded) and copied."""
    g = torch.Generator().manual_seed(seed)
    n, d, h = 4096, 64, 256
    X = torch.randn(n, d, generator=g)
    a = torch.randn(d, generator=g) / d ** 0.5
    y = (torch.sin(3 * X @ a) + 0.1 * torch.randn(n, generator=g)).unsqueeze(1)
    init = [torch.randn(h, d, generator=g) / d ** 0.5, torch.zeros(h),
            torch.randn(1, h, generator=g) / h ** 0.5, torch.zeros(1)]
    return X.to(device), y.to(device), init


def training_study(steps: int = 300, seed: int = 7, device: str = "cuda",
                   every: int = 10) -> dict:
    """Loss curves (every `every` steps; None once non-finite) of the three
    runs.  The model computes in FP32 (the BF16 weights theta' are upcast)."""
    from . import optim as O
    X, y, init = _mlp_task(seed, device)
    hp = dict(lr=3e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)

    def loss_of(ps):
        w1, b1, w2, b2 = (p.float() for p in ps)
        return ((torch.relu(X @ w1.t() + b1) @ w2.t() + b2 - y) ** 2).mean()

    runs = {}
    for name in ("reference", "companded", "linear"):
        ps = [torch.nn.Parameter(t.clone().to(device)) for t in init]
        if name == "reference":
            opt = torch.optim.AdamW(ps, **hp)
        else:
            opt = O.FlashAdamW([{"params": ps, "linear_variance": name == "linear"}], **hp)
        curve = []
        for it in range(steps):
            loss = loss_of(ps)
            val = loss.item()
            finite = val == val and abs(val) != float("inf")
            if it % every == 0 or it == steps - 1 or not finite:
                curve.append(val if finite else None)
            if not finite:                               # diverged: stop feeding NaN back
                break
            opt.zero_grad()
            loss.backward()
            opt.step()
        runs[name] = curve
    return {"steps": steps, "every": every, "hparams": {k: list(v) if isinstance(v, tuple) else v
                                                         for k, v in hp.items()}, "loss": runs}


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--n", type=int, default=1 << 22)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out", default=None, help="write the JSON here as well")
    a = ap.parse_args()
    r = run(a.n, a.seed)
    r["training"] = training_study()
    text = json.dumps(r, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    main()
