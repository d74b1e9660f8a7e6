"""Trellis-quantized routed MoE layer for MI355X (gfx950): HIP kernels behind a C ABI.

Import `trellis_quantized_moe_tmoe_amd.layer` for the torch-facing wrapper (it loads libtmoe.so and
fails if the library is not built) and `trellis_quantized_moe_tmoe_amd.workloads` for seeded inputs.
"""
__all__ = ["layer", "native", "workloads"]
