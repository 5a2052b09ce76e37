"""MI355X (gfx950) implementation of FlashOptim's fused compressed optimizer
step ("FlashOptim: Optimizers for Memory Efficient Training").

* flashopt.py  -- the thin ctypes binding of the C-ABI HIP library
  (include/flashopt.h; kernels in csrc/, built in-tree by build.py);
* optim.py     -- drop-in FlashAdamW / FlashSGD / FlashLion (torch.optim API,
  compressed checkpoints, gradient release, per-group compression switch,
  HIP-graph capture);
* ablations.py -- the codec studies (weight rebuild error, companding,
  training without companding) run through the library;
* workloads.py -- synthetic parameter-list shapes and seeded input draws for
  the tests and the benchmark.
"""
