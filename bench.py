"""Benchmark: FlashOptim fused compressed AdamW step on one MI355X.

A step is one pass of the fused kernel over the whole Llama-3.1-8B-shaped
parameter list (291 tensors, 8,030,261,248 parameters): rebuild the master
weight from BF16 + INT8, dequantise INT8 / UINT8 moments (FP16 scale per 32),
AdamW, requantise, re-split -- one launch of flashopt_adamw_step.  All state
and gradients are resident in HBM before timing starts; two gradient sets are
drawn up front and the steps alternate between them (two list handles over
the same state).

Prints one JSON line (rank 0).  --gpus N > 1 is refused: the step is measured
on one GPU (it shards with no exchange inside the step; no multi-GPU run is
provided).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from compressed_adamw_state_amd import flashopt as F          # noqa: E402
from compressed_adamw_state_amd import workloads as W          # noqa: E402

METRIC = "fused AdamW step params/s + achieved HBM GB/s (% peak) at Llama-3.1-8B shapes"
HBM_PEAK_GBS = 8000.0
KERNEL = "step_kernel<0, false, false>"   # the fused AdamW step kernel, one wave per tile
# the fused step kernel's sources (a committed profile applies while their hash is unchanged)
PEAK_CLOCK_GHZ = 2.4        # MI355X peak engine clock (256 CUs x 4 SIMDs)
SOURCES = ["compressed_adamw_state_amd/csrc/step.hip",
           "compressed_adamw_state_amd/csrc/device.hpp",
           "compressed_adamw_state_amd/csrc/host.hpp",
           "compressed_adamw_state_amd/csrc/codec.hpp"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for s in SOURCES:
        h.update(open(os.path.join(ROOT, s), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w: W.Workload) -> int:
    """Bytes the method must move per step: read theta', rho, m, v codes, both
    scales and the BF16 grad; write everything but the grad.  Uncompressed
    (_fp32) state: read the FP32 master weight and moments and the grad, write
    them back and theta'."""
    total = 0
    if w.optimizer.endswith("_fp32"):
        per = 14 if w.optimizer == "adamw_fp32" else 10       # bytes read = bytes written
        return sum(2 * per * t.numel for t in w.tensors)
    for t in w.tensors:
        n, g = t.numel, (t.numel + 31) // 32
        rd = 2 * n + n + n + 2 * g + 2 * n
        wr = 2 * n + n + n + 2 * g
        if w.optimizer == "adamw":
            rd += n + 2 * g
            wr += n + 2 * g
        total += rd + wr
    return total


def read_profile(kind: str, workload: str, kernel_hash: str) -> dict:
    """key: value lines of a committed rocprofv3 summary (profiles/), if it was
    taken on the current kernel source; else {}."""
    path = os.path.join(ROOT, "profiles", f"{kind}_adamw_{workload}.txt")
    if not os.path.exists(path):
        return {}
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv if kv.get("source_sha256_16") == kernel_hash else {}


def build_state(w: W.Workload, grad_sets: int, candidates: int = 1, placement: dict = None):
    """The workload's state and `grad_sets` gradient sets, all in one
    StateArena (theta', gradients, codes and scales each in a region of their
    own), and one list handle per gradient set.  candidates > 1: the arena's
    placement search (StateArena) picks the allocation; its probe times go
    into `placement`."""
    dev = torch.device("cuda")
    states = []
    arena = F.StateArena([spec.numel for spec in w.tensors], w.optimizer, dev, theta=True,
                         grad_sets=grad_sets, candidates=candidates)
    if placement is not None and arena.placement_ms is not None:
        placement.update({"candidates": candidates, "allocations": len(arena.placement_ms),
                          "probe_ms": arena.placement_ms, "chosen": arena.placement_choice})
    for i, spec in enumerate(w.tensors):
        theta = W.draw_theta(w, i, dev)
        st = arena.state(i)
        F.flashopt_tensor_init(st, theta)
        del theta
        states.append(st)
    grads = []
    for k in range(grad_sets):
        grads.append([arena.grad(k, i).copy_(W.draw_grad(w, i, k + 1, dev))
                      for i in range(len(w.tensors))])
    lists = [F.FlashoptList(states, g) for g in grads]
    F.flashopt_state_zero(lists[0])
    torch.cuda.synchronize()
    return states, grads, lists


def copy_ceiling(nbytes: int, stream, reps: int = 5):
    """A plain streaming copy of known size (torch's elementwise bitwise_not on
    int32: reads nbytes, writes nbytes) -- the practical HBM ceiling for a
    pure stream, and the reference the rocprofv3 HBM counters are scaled by."""
    n = nbytes // 4
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for r in range(reps):
        torch.bitwise_not(src, out=dst)
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    best = min(ev[r].elapsed_time(ev[r + 1]) for r in range(reps)) / 1e3
    return {"kernel": "torch bitwise_not int32", "bytes_read": 4 * n, "bytes_written": 4 * n,
            "best_ms": best * 1e3, "gb_s": 8 * n / best / 1e9}


def release_buckets(sizes, bucket_bytes: int):
    """Gradient-release buckets in backward order: (first, count) ranges of
    consecutive tensors, each closed once its BF16 gradients reach
    bucket_bytes (one tensor per bucket when bucket_bytes is 0)."""
    out, hi = [], len(sizes) - 1
    while hi >= 0:
        lo, b = hi, 2 * sizes[hi]
        while b < bucket_bytes and lo > 0:
            lo -= 1
            b += 2 * sizes[lo]
        out.append((lo, hi - lo + 1))
        hi = lo - 1
    return out


def other_optimizer(name: str, steps: int, stream, release_streams: int = 1,
                    bucket_bytes: int = 0, release: bool = False, candidates: int = 3) -> dict:
    """Time `steps` list steps of another optimizer's workload (after warm-up);
    state built fresh, freed on return.  In gradient-release mode (the
    workload's own, or `release`) the tensors are stepped in backward order,
    one launch per tensor or, with bucket_bytes > 0, one range launch per
    bucket of consecutive tensors (release_buckets); the launches go
    round-robin over `release_streams` streams (tensors are independent, so
    one launch's tail can overlap the next); each step is bracketed on
    `stream`.  The state's arena is placed by the placement search over
    `candidates` allocations (compressed kinds; the _fp32 kinds take the
    first allocation)."""
    w = W.WORKLOADS[name]
    release = release or w.release
    placement = {}
    states, grads, lists = build_state(
        w, grad_sets=2, candidates=1 if w.optimizer in F.FP32_FIELDS else candidates,
        placement=placement)
    side = [stream] + [torch.cuda.Stream() for _ in range(release_streams - 1)]
    buckets = release_buckets([t.numel for t in w.tensors], bucket_bytes)

    def one_step(k, t):
        if release:              # gradient release, backward order
            start = torch.cuda.Event()
            start.record(stream)
            for s in side[1:]:
                s.wait_event(start)
            for j, (first, count) in enumerate(buckets):
                if bucket_bytes > 0:
                    F.step_range(lists[k % 2], w.optimizer, first,
                                 grads[k % 2][first:first + count], w.hparams, t,
                                 side[j % len(side)])
                else:
                    F.step_one(lists[k % 2], w.optimizer, first, grads[k % 2][first],
                               w.hparams, t, side[j % len(side)])
            for s in side[1:]:
                done = torch.cuda.Event()
                done.record(s)
                stream.wait_event(done)
        else:
            F.step(lists[k % 2], w.optimizer, w.hparams, t, stream)

    for t in (1, 2):
        one_step(t, t)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for k in range(steps):
        one_step(k, k + 3)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)])    # ms
    del states, grads, lists
    torch.cuda.synchronize()
    ms = float(np.median(per))
    gbs = algorithmic_bytes(w) / (ms * 1e-3) / 1e9
    return {"workload": name, "optimizer": w.optimizer, "params": w.numel,
            "gradient_release": release, "bucket_bytes": bucket_bytes if release else None,
            "launches_per_step": (len(buckets) * (2 if bucket_bytes > 0 else 1)) if release else 1,
            "streams": len(side) if release else 1,
            "bytes_per_param": algorithmic_bytes(w) / w.numel, "step_ms_median": ms,
            "step_ms_min": float(per.min()), "params_s": w.numel / (ms * 1e-3),
            "algorithmic_gb_s": gbs, "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
            "placement_search": placement or None}


def wrapper_adamw(steps: int, stream) -> dict:
    """FlashAdamW.step() through the torch.optim API on the Llama-3.1-8B list:
    FP32 parameters split at construction, one BF16 gradient set, `steps`
    timed steps (GPU events and host wall time, so the host-side marshalling
    shows)."""
    from compressed_adamw_state_amd import optim as O
    w = W.WORKLOADS["llama31_8b"]
    dev = torch.device("cuda")
    params = []
    for i in range(len(w.tensors)):
        params.append(torch.nn.Parameter(W.draw_theta(w, i, dev)))
    opt = O.FlashAdamW(params, lr=w.hparams["lr"], betas=(w.hparams["beta1"], w.hparams["beta2"]),
                       eps=w.hparams["eps"], weight_decay=w.hparams["weight_decay"])
    for i, p in enumerate(params):
        p.grad = W.draw_grad(w, i, 1, dev).view(p.shape)
    for _ in range(2):
        opt.step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for k in range(steps):
        opt.step()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) / steps * 1e3
    per = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)])
    del opt, params
    torch.cuda.synchronize()
    ms = float(np.median(per))
    return {"workload": "llama31_8b", "optimizer": "FlashAdamW (torch.optim API)",
            "params": w.numel, "step_ms_median": ms, "step_ms_min": float(per.min()),
            "wall_ms_per_step": wall, "params_s": w.numel / (ms * 1e-3),
            "algorithmic_gb_s": algorithmic_bytes(w) / (ms * 1e-3) / 1e9}


def graph_replay_adamw(steps: int) -> dict:
    """The scheduled AdamW step (step counter and scalars in a device
    schedule) captured once in a HIP graph and replayed `steps` times on the
    Llama-3.1-8B list: the path a graph-captured training loop takes."""
    w = W.WORKLOADS["llama31_8b"]
    states, grads, lists = build_state(w, grad_sets=1)
    sched = F.DeviceSchedule(w.hparams, t=0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            F.flashopt_adamw_step_scheduled(lists[0], sched)
    torch.cuda.synchronize()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for k in range(steps):
        graph.replay()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)])
    t_dev = sched.read().t
    del graph, sched, states, grads, lists
    torch.cuda.synchronize()
    ms = float(np.median(per))
    return {"workload": "llama31_8b", "optimizer": "adamw, scheduled step replayed from a HIP graph",
            "params": w.numel, "replays": steps, "device_step_count": t_dev,
            "step_ms_median": ms, "step_ms_min": float(per.min()),
            "params_s": w.numel / (ms * 1e-3),
            "algorithmic_gb_s": algorithmic_bytes(w) / (ms * 1e-3) / 1e9}


def release_memory(iters: int, stream, layers: int = 32, width: int = 4096,
                   batch: int = 8) -> dict:
    """Gradient release end to end: forward + backward + FlashAdamW step of
    a stack of `layers` BF16 linear layers (width x width, no bias; a small
    batch, so the gradients are most of an iteration's transient memory),
    with the step after backward, with gradient release on one and two
    side streams, and with release in 64 MiB buckets.  Reports the peak of allocated memory during an iteration
    above what stays resident (model + state), the saving per parameter, the
    median time per iteration, and whether the weights after the timed
    iterations are bit-identical across the three modes."""
    from compressed_adamw_state_amd import optim as O
    n = layers * width * width
    x = torch.randn(batch, width, device="cuda", dtype=torch.bfloat16,
                    generator=torch.Generator("cuda").manual_seed(11))
    modes = {}
    ref = None
    for name, release, streams, bucket in (("step after backward", False, 1, 0),
                                           ("gradient release", True, 1, 0),
                                           ("gradient release, 2 streams", True, 2, 0),
                                           ("gradient release, 64 MiB buckets", True, 1, 64 << 20)):
        torch.cuda.manual_seed(12)
        model = torch.nn.Sequential(*[torch.nn.Linear(width, width, bias=False, device="cuda",
                                                      dtype=torch.bfloat16)
                                      for _ in range(layers)])
        opt = O.FlashAdamW(model.parameters(), lr=1e-3, gradient_release=release,
                           release_streams=streams, release_bucket_bytes=bucket)

        def iteration():
            model(x).float().pow(2).mean().backward()
            opt.step()
            opt.zero_grad(set_to_none=True)

        iteration()
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        ev[0].record(stream)
        for k in range(iters):
            iteration()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        per = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(iters)])
        w = torch.cat([p.detach().view(torch.int16).reshape(-1) for p in model.parameters()])
        same = None if ref is None else bool(torch.equal(w, ref))
        if ref is None:
            ref = w
        modes[name] = {"peak_transient_bytes": int(peak), "iteration_ms_median": float(np.median(per)),
                       "weights_equal_step_after_backward": same}
        del opt, model, w
        torch.cuda.empty_cache()
    base_peak = modes["step after backward"]["peak_transient_bytes"]
    for name, m in modes.items():
        m["saving_bytes_per_param"] = (base_peak - m["peak_transient_bytes"]) / n
    del ref
    torch.cuda.empty_cache()
    return {"workload": f"{layers} x Linear({width}, {width}) BF16, batch {batch}",
            "optimizer": "FlashAdamW, gradient release end to end", "params": n,
            "iterations": iters, "modes": modes,
            "step_ms_median": modes["gradient release"]["iteration_ms_median"]}


def stream_probe(lst, stream, bytes_step: int, reps: int = 5):
    """The step's exact loads and stores with no arithmetic (flashopt_stream_probe):
    the practical floor of its access pattern.  Overwrites the state."""
    F.flashopt_stream_probe(lst, stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for r in range(reps):
        F.flashopt_stream_probe(lst, stream)
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    best = min(ev[r].elapsed_time(ev[r + 1]) for r in range(reps)) / 1e3
    return {"kernel": "probe_kernel (flashopt_stream_probe)", "best_ms": best * 1e3,
            "gb_s": bytes_step / best / 1e9}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_single_thread_flat1m(seconds: float = 3.0) -> float:
    """One-thread oracle params/s on the flat 1M-parameter AdamW workload."""
    import oracle
    w = W.WORKLOADS["flat1m"]
    n = w.numel
    st = oracle.State(W.draw_theta(w, 0).numpy(), "adamw")
    grads = [W.draw_grad(w, 0, t).view(torch.int16).numpy().view(np.uint16) for t in (1, 2)]
    steps = 0
    t0 = time.perf_counter()
    while True:
        oracle.step(st, grads[steps % 2], steps + 1, w.hparams)
        steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    return n * steps / (time.perf_counter() - t0)


def cpu_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, at most
    16 (the CPU share of one GPU on the benchmark's hosts)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return max(1, min(16, avail))


def host_fields(st: F.TensorState) -> dict:
    """theta', rho, momentum and variance codes, both scales of one AdamW
    tensor as contiguous host arrays (the code planes of each 512-element
    block, include/flashopt.h, unpacked on the device, then copied)."""
    n = st.numel
    nblk, ng = (n + 511) // 512, (n + 31) // 32
    pl = st.codes[:nblk * 1536].view(nblk, 3, 512)
    sc = st.scales[:ng * 2].view(ng, 2)
    host = lambda t: t.contiguous().cpu().numpy()
    return {"tb": host(st.theta.view(torch.int16)).view(np.uint16),
            "rho": host(pl[:, 0].reshape(-1)[:n]).view(np.int8),
            "qm": host(pl[:, 1].reshape(-1)[:n]).view(np.int8),
            "qv": host(pl[:, 2].reshape(-1)[:n]),
            "sm": host(sc[:, 0]).view(np.uint16), "sv": host(sc[:, 1]).view(np.uint16)}


def cpu_baseline(states, grads, t: int, hp: dict, threads: int) -> dict:
    """The oracle as it stands, timed on one full step of the benchmark's
    workload: every tensor of the list, from the state the GPU holds after
    the timed steps and with the gradient set of step t, copied to the host
    tensor by tensor (the copies and unpacking are not timed) and stepped by
    the oracle on `threads` host threads over whole 32-element groups."""
    import oracle
    spent, n = 0.0, 0
    for st, g in zip(states, grads):
        f = host_fields(st)
        o = oracle.State.__new__(oracle.State)
        o.n, o.optimizer = st.numel, "adamw"
        for k, v in f.items():
            setattr(o, k, v)
        gb = g.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        oracle.step_chunked(o, gb, t, hp, nthreads=threads)
        spent += time.perf_counter() - t0
        n += st.numel
        del f, o, gb
    return {"value": n / spent, "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": f"one full AdamW step of the benchmark's list ({len(states)} tensors, {n} "
                      f"params) from the GPU's state after the timed steps, tensor by tensor, "
                      f"host copies not timed; {threads} threads over whole 32-element groups, "
                      f"{spent:.1f} s",
            "oracle_seconds": spent, "params": n,
            "host_cpus": os.cpu_count(), "host_cpus_available": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(),
            "single_thread_flat1m_params_s": cpu_single_thread_flat1m()}


def mix_ceiling(n: int, stream, reps: int = 5) -> dict:
    """flashopt_mix_ceiling over flat buffers of n parameters: the step's own
    byte mix (7.125 B read, 5.125 B written per parameter, four streams read
    and three written, in place) with every access a coalesced 16 bytes per
    lane -- the practical ceiling for the step's traffic."""
    th = torch.randint(-2 ** 15, 2 ** 15 - 1, (n,), dtype=torch.int16, device="cuda")
    gr = torch.randint(-2 ** 15, 2 ** 15 - 1, (n,), dtype=torch.int16, device="cuda")
    cd = torch.randint(0, 255, (3 * n,), dtype=torch.uint8, device="cuda")
    sc = torch.randint(-2 ** 15, 2 ** 15 - 1, (n // 16,), dtype=torch.int16, device="cuda")
    F.flashopt_mix_ceiling(th, gr, cd, sc, n, stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for r in range(reps):
        F.flashopt_mix_ceiling(th, gr, cd, sc, n, stream)
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    best = min(ev[r].elapsed_time(ev[r + 1]) for r in range(reps)) / 1e3
    nbytes = int(12.25 * n)
    del th, gr, cd, sc
    torch.cuda.empty_cache()
    return {"kernel": "mix_ceiling_kernel (flashopt_mix_ceiling)", "params": n,
            "bytes_read_per_param": 7.125, "bytes_written_per_param": 5.125,
            "best_ms": best * 1e3, "gb_s": nbytes / best / 1e9}


def best_of(f, reps: int, stream) -> float:
    """Best of `reps` launches of f (ms, HIP events on `stream`), after one
    untimed launch."""
    f()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for k in range(reps):
        f()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    return min(ev[k].elapsed_time(ev[k + 1]) for k in range(reps))


def placement(n: int, stream, sets: int = 3, rounds: int = 3, reps: int = 3) -> dict:
    """Where the buffers lie: `sets` allocations of the byte-mix buffers
    (theta', grad, codes, scales of n parameters) alive at once, each timed
    with flashopt_mix_ceiling in alternation over `rounds` rounds; every
    pattern variant (4: hashed tile order) on each; then set 0 with one array of
    set 1 swapped in at a time, and each array alone (read, write, in-place
    read+write over its whole size by flashopt_stream_sweep)."""
    def alloc():
        return [torch.empty(2 * n, dtype=torch.uint8, device="cuda"),
                torch.empty(2 * n, dtype=torch.uint8, device="cuda"),
                torch.empty(3 * n, dtype=torch.uint8, device="cuda"),
                torch.empty(n // 8, dtype=torch.uint8, device="cuda")]
    S = [alloc() for _ in range(sets)]
    for b in S:
        for t in b:
            t.zero_()
    mix = lambda b: (lambda: F.flashopt_mix_ceiling(b[0], b[1], b[2], b[3], n, stream))
    pat = lambda v, b: (lambda: F.flashopt_pattern_probe(v, b[0], b[1], b[2], b[3], n, stream))
    out = {"params": n, "mix_ms_by_round": [[best_of(mix(b), reps, stream) for b in S]
                                            for _ in range(rounds)],
           "variant_ms": {v: [best_of(pat(v, b), reps, stream) for b in S] for v in range(6)}}
    names = ["theta", "grad", "codes", "scales"]
    out["set0_with_one_array_of_set1_ms"] = {
        names[i]: best_of(mix([S[1][j] if j == i else S[0][j] for j in range(4)]), reps, stream)
        for i in range(4)}
    single = {}
    for k, b in enumerate(S):
        for i in range(3):
            t, nb = b[i], b[i].numel() // 16 * 16
            rd = best_of(lambda: F.flashopt_stream_sweep([t], [], nb, False, stream), reps, stream)
            wr = best_of(lambda: F.flashopt_stream_sweep([], [t], nb, False, stream), reps, stream)
            rw = best_of(lambda: F.flashopt_stream_sweep([t], [t], nb, True, stream), reps, stream)
            single[f"set{k} {names[i]}"] = {"read_gb_s": nb / rd / 1e6, "write_gb_s": nb / wr / 1e6,
                                            "rw_in_place_gb_s": 2 * nb / rw / 1e6}
    out["single_array"] = single
    del S
    torch.cuda.empty_cache()
    return out


def pattern_variants(n: int, stream, reps: int = 5, rounds: int = 2) -> list:
    """flashopt_pattern_probe variants 0-5 and flashopt_mix_ceiling over the
    same flat buffers of n parameters, alternating, best of `reps` launches
    per round: the step's traffic under each access pattern."""
    th = torch.randint(-2 ** 15, 2 ** 15 - 1, (n,), dtype=torch.int16, device="cuda")
    gr = torch.randint(-2 ** 15, 2 ** 15 - 1, (n,), dtype=torch.int16, device="cuda")
    cd = torch.randint(0, 255, (3 * n,), dtype=torch.uint8, device="cuda")
    sc = torch.randint(-2 ** 15, 2 ** 15 - 1, (n // 16,), dtype=torch.int16, device="cuda")
    names = {0: "codes as 3 x 8-B plane runs, hinted, 2 buffers (the fused kernel's)",
             1: "codes as 16-B units", 2: "16-B units by global-to-LDS DMA",
             3: "as 0, 3 buffers (loads before stores)",
             4: "as 0, tiles in a hashed order",
             5: "codes as interleaved 24-B records, 3 x 8 B unhinted (the earlier layout)",
             "mix": "mix ceiling (all 16-B, flat)"}
    rows = {}
    for _ in range(rounds):
        for v in names:
            f = (lambda: F.flashopt_mix_ceiling(th, gr, cd, sc, n, stream)) if v == "mix" else \
                (lambda v=v: F.flashopt_pattern_probe(v, th, gr, cd, sc, n, stream))
            rows.setdefault(v, []).append(best_of(f, reps, stream))
    del th, gr, cd, sc
    torch.cuda.empty_cache()
    return [{"variant": v, "pattern": names[v], "best_ms": min(t),
             "gb_s": 12.25 * n / (min(t) * 1e-3) / 1e9} for v, t in rows.items()]


def layouts(w: W.Workload, stream, steps: int = 10) -> list:
    """The fused step and its probe over the workload in two placements: the
    StateArena with theta', the gradients, the codes and the scales each in a
    region of their own (build_state), and theta' and the gradients allocated
    tensor by tensor beside an arena of codes and scales."""
    out = []
    for name in ("arena regions", "theta' and gradients per tensor"):
        if name == "arena regions":
            states, grads, lists = build_state(w, grad_sets=1)
            lst = lists[0]
        else:
            dev = torch.device("cuda")
            arena = F.StateArena([t.numel for t in w.tensors], w.optimizer, dev)
            states = []
            for i in range(len(w.tensors)):
                theta = W.draw_theta(w, i, dev)
                st = arena.state(i)
                F.flashopt_tensor_init(st, theta)
                del theta
                states.append(st)
            grads = [[W.draw_grad(w, i, 1, dev) for i in range(len(w.tensors))]]
            lst = F.FlashoptList(states, grads[0])
            lists = [lst]
        t = 0
        for _ in range(2):
            t += 1
            F.flashopt_adamw_step(lst, w.hparams, t, stream)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for k in range(steps):
            t += 1
            F.flashopt_adamw_step(lst, w.hparams, t, stream)
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]
        probe = stream_probe(lst, stream, algorithmic_bytes(w))
        out.append({"layout": name, "step_ms_median": float(np.median(per)),
                    "probe_ms": probe["best_ms"], "probe_gb_s": probe["gb_s"]})
        del states, grads, lists, lst
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


SWEEP = [(1, 0, False), (0, 1, False), (4, 0, False), (0, 4, False), (1, 1, False),
         (1, 1, True), (2, 1, False), (2, 1, True), (1, 2, False), (2, 2, False), (2, 2, True),
         (3, 2, False), (3, 2, True), (4, 3, False), (4, 3, True), (7, 5, False)]


def stream_sweep(nbytes: int, stream, reps: int = 5, rounds: int = 2) -> list:
    """flashopt_stream_sweep: plain 16-byte-per-lane streams over separate
    buffers of nbytes each, R read and W written (in place: the written
    buffers are read ones), best of `reps` launches, `rounds` rounds."""
    bufs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
            for _ in range(12)]
    rows = {}
    for _ in range(rounds):
        for r, w, ip in SWEEP:
            reads = bufs[:r]
            writes = bufs[:w] if ip else bufs[r:r + w]
            F.flashopt_stream_sweep(reads, writes, nbytes, ip, stream)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            ev[0].record(stream)
            for k in range(reps):
                F.flashopt_stream_sweep(reads, writes, nbytes, ip, stream)
                ev[k + 1].record(stream)
            torch.cuda.synchronize()
            best = min(ev[k].elapsed_time(ev[k + 1]) for k in range(reps)) / 1e3
            rows.setdefault((r, w, ip), []).append((r + w) * nbytes / best / 1e9)
    del bufs
    torch.cuda.empty_cache()
    return [{"read": r, "written": w, "in_place": ip, "gb_s": v}
            for (r, w, ip), v in rows.items()]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama31_8b")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle threads for cpu_baseline (0: the CPUs available, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=1 << 32,
                    help="size of the plain copy kernel timed after the steps (0: skip)")
    ap.add_argument("--no-other-optimizers", action="store_true",
                    help="skip the FlashLion (Llama-3.1-8B) and FlashSGD (ResNet-50) lines")
    ap.add_argument("--access-patterns", action="store_true",
                    help="time only the access-pattern evidence and print it as JSON: the plain "
                         "stream-count sweep (12 buffers of 2 GiB), the step's traffic over flat "
                         "buffers under each pattern variant and the byte-mix ceiling, and the "
                         "step and its probe in two placements")
    ap.add_argument("--placement", action="store_true",
                    help="time only the placement study and print it as JSON: three allocations "
                         "of the byte-mix buffers at Llama-3.1-8B size, timed in alternation, "
                         "in two tile orders, with arrays swapped between them and alone")
    ap.add_argument("--placement-candidates", type=int, default=3,
                    help="allocations of each benchmark state tried by the arena's placement "
                         "search (the fastest under the step's own access probe is kept; 1: "
                         "the first allocation, no search; the _fp32 kinds never search)")
    ap.add_argument("--secondary", default=None, metavar="WORKLOAD",
                    help="time only this secondary workload (--steps steps) and print its "
                         "record: a profiling aid, not the benchmark line")
    ap.add_argument("--release", action="store_true",
                    help="with --secondary: step the workload in gradient-release mode (one "
                         "launch per tensor, backward order)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the fused step is measured on one GPU only; --gpus must be 1 "
              "(the step shards with no exchange inside it, but no multi-GPU run is "
              "provided)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    F.lib()

    if args.secondary:
        r = other_optimizer(args.secondary, args.steps, torch.cuda.current_stream(),
                            release=args.release, candidates=args.placement_candidates)
        print(json.dumps(r), flush=True)
        return
    if args.access_patterns:
        stream = torch.cuda.current_stream()
        w = W.WORKLOADS["llama31_8b"]
        r = {"stream_sweep_2GiB": stream_sweep(2 << 30, stream),
             "flat_patterns": pattern_variants(w.numel, stream),
             "layouts": layouts(w, stream)}
        print(json.dumps(r), flush=True)
        return
    if args.placement:
        n = W.WORKLOADS["llama31_8b"].numel // 2048 * 2048
        print(json.dumps(placement(n, torch.cuda.current_stream())), flush=True)
        return

    w = W.WORKLOADS[args.workload]
    assert w.optimizer == "adamw" and not w.release
    log(f"bench: building {w.name} state ({w.numel} params, {len(w.tensors)} tensors)")
    t0 = time.perf_counter()
    placement_search = {}
    states, grads, lists = build_state(w, grad_sets=2, candidates=args.placement_candidates,
                                       placement=placement_search)
    log(f"bench: state ready in {time.perf_counter() - t0:.1f} s"
        + (f"; placement search: probe {placement_search['probe_ms']} ms, kept allocation "
           f"{placement_search['chosen']}" if placement_search else ""))
    hp = w.hparams
    stream = torch.cuda.current_stream()

    t = 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for k in range(args.warmup):
        t += 1
        if k == 0:
            e0.record(stream)
        F.flashopt_adamw_step(lists[t % 2], hp, t, stream)
        if k == 0:
            e1.record(stream)
    torch.cuda.synchronize()
    step1_ms = e0.elapsed_time(e1) if args.warmup > 0 else None
    log(f"bench: {args.warmup} warmup steps done")

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(args.steps):
        t += 1
        starts[k].record(stream)
        F.flashopt_adamw_step(lists[t % 2], hp, t, stream)
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]) / 1e3   # seconds
    total = float(per.sum())
    log(f"bench: {args.steps} timed steps, wall {wall * 1e3:.1f} ms, kernel sum {total * 1e3:.1f} ms")

    nparams = w.numel
    bytes_step = algorithmic_bytes(w)
    avg = total / args.steps
    achieved = bytes_step / avg / 1e9
    khash = source_hash()
    traffic_kv = read_profile("traffic", w.name, khash)
    traffic = float(traffic_kv["hbm_bytes_per_launch"]) if "hbm_bytes_per_launch" in traffic_kv \
        else None
    sq = read_profile("sq", w.name, khash)
    valu_cycles = float(sq["SQ_INSTS_VALU"]) * 4 / 1024 if "SQ_INSTS_VALU" in sq else None
    out = {
        "metric": METRIC,
        "value": nparams * args.steps / wall,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: Llama-3.1-8B-shaped list, {len(w.tensors)} tensors, "
                               f"{nparams} params, AdamW lr 1e-3 betas (0.9, 0.999) eps 1e-8 "
                               f"wd 0.01, bf16 grads N(0, 1e-4)",
                   "state": "theta' bf16 + int8 rho, int8 m and uint8 v code planes per 512-element block + fp16 scale pair per 32",
                   "launches_per_step": 1,
                   "placement": (f"best of {placement_search['allocations']} arena allocations "
                                 f"by the step's own access probe" if placement_search
                                 else "first allocation")},
        "placement_search": placement_search or None,
        "hbm_gb_s": achieved,
        "pct_hbm_peak": 100.0 * achieved / HBM_PEAK_GBS,
        "step_ms_median": float(np.median(per) * 1e3),
        "step_ms_min": float(per.min() * 1e3),
        "step1_ms": step1_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel": KERNEL,
                     "algorithmic_bytes_per_launch": bytes_step,
                     "avg_launch_ms": avg * 1e3, "source_sha256_16": khash,
                     "valu_instructions_per_param":
                         float(sq["valu_instructions_per_param"]) if sq else None,
                     # VALU issue cycles per SIMD per launch (SQ_INSTS_VALU of the profiled
                     # run, one wave64 instruction per SIMD every 4 cycles on 1024 SIMDs), and
                     # the shader clock at which that issue alone fills this run's launch
                     "valu_cycles_per_simd": valu_cycles,
                     "valu_bound_clock_ghz": (valu_cycles / (avg * 1e9)) if valu_cycles else None,
                     # the same issue time over this launch at the part's peak engine clock
                     # (2.4 GHz): the fraction of VALU issue capacity the launch uses
                     "valu_issue_frac_at_peak_clock":
                         (valu_cycles / (avg * PEAK_CLOCK_GHZ * 1e9)) if valu_cycles else None,
                     "shader_clock_ghz_in_profiled_run":
                         float(sq["shader_clock_ghz"]) if "shader_clock_ghz" in sq else None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or cpu_threads()
        log(f"bench: timing the CPU oracle on one full step ({threads} threads)")
        out["cpu_baseline"] = cpu_baseline(states, grads[(t + 1) % 2], t + 1, hp, threads)
        log(f"bench: oracle {out['cpu_baseline']['value'] / 1e9:.3f} G params/s")
    out["stream_probe"] = stream_probe(lists[0], stream, bytes_step)
    out["stream_probe"]["step_over_probe"] = avg * 1e3 / out["stream_probe"]["best_ms"]
    log(f"bench: stream probe {out['stream_probe']['gb_s']:.0f} GB/s")
    del states, grads, lists
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    out["mix_ceiling"] = mix_ceiling(nparams, stream)
    out["mix_ceiling"]["step_over_ceiling"] = avg * 1e3 / out["mix_ceiling"]["best_ms"]
    log(f"bench: byte-mix ceiling {out['mix_ceiling']['gb_s']:.0f} GB/s")
    if not args.no_other_optimizers:
        oo = lambda *a, **k: other_optimizer(*a, candidates=args.placement_candidates, **k)
        out["other_optimizers"] = [oo("llama31_8b_lion", 10, stream),
                                   oo("llama31_8b_adamw_fp32", 5, stream),
                                   oo("resnet50", 10, stream),
                                   oo("flat1m", 10, stream),
                                   oo("gpt2_small", 10, stream),
                                   oo("llama2_13b", 5, stream),
                                   oo("llama2_13b", 5, stream, release_streams=2),
                                   oo("llama2_13b", 5, stream, bucket_bytes=64 << 20),
                                   oo("llama2_13b", 5, stream, release_streams=2,
                                      bucket_bytes=64 << 20),
                                   oo("gpt2_small", 10, stream, release=True),
                                   oo("gpt2_small", 10, stream, release=True,
                                      bucket_bytes=16 << 20),
                                   wrapper_adamw(10, stream),
                                   graph_replay_adamw(10),
                                   release_memory(5, stream)]
        for o in out["other_optimizers"]:
            log(f"bench: {o['optimizer']} {o['workload']}: {o['step_ms_median']:.3f} ms/step")
    if args.copy_bytes:
        out["copy_ceiling"] = copy_ceiling(args.copy_bytes, stream)
        log(f"bench: plain copy {out['copy_ceiling']['gb_s']:.0f} GB/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
