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


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--n", type=int, default=1 << 22)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out", default=None, help="write the JSON here as well")
    a = ap.parse_args()
    r = run(a.n, a.seed)
    text = json.dumps(r, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    main()
