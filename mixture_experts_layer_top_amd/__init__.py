"""Fused MoE layer for one MI355X (gfx950): hand-written HIP kernels behind a C ABI.

Submodules:
  moe     ctypes binding of libmoe_mi355x.so (loaded on first use; raises if it is not built)
  inputs  seeded synthetic inputs (shared by tests and the benchmark)
  build   compiles the HIP library in-tree with hipcc for gfx950
"""
