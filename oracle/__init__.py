"""CPU fp64 oracle for the fused MoE layer.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
bench.py may import or call anything here.  The product path (the HIP library and its Python
binding) never imports it, and this package imports nothing from the product path.  The only
code both sides draw on is the seeded input generator (mixture_experts_layer_top_amd.inputs),
which holds no arithmetic of the layer.

Modules:
  fp8_e4m3   OCP E4M3FN codec written from the format definition.
  mxfp4      OCP MXFP4 (E2M1 elements, E8M0 scales per 32) written from the format definitions.
  moe_oracle the layer, step by step, in float64.
"""
