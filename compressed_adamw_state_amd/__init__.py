"""MI355X (gfx950) implementation of FlashOptim's fused compressed optimizer
step: a C-ABI HIP library (include/flashopt.h, csrc/) and its thin binding
(flashopt.py).  workloads.py holds the synthetic parameter-list shapes and
seeded input draws used by tests and the benchmark."""
