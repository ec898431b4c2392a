"""sparse_moe_ffn_amd: MI355X-native (gfx950, hand-written HIP) MobileMoE
MoE-FFN layer forward, exposed through the C-ABI library ``libmobmoe``.

Submodules are imported on demand so that importing the package does not load
the GPU library:
  - ``sparse_moe_ffn_amd.binding``   thin ctypes binding of include/mobmoe.h
  - ``sparse_moe_ffn_amd.layer``     a layer object that owns device buffers
                                     and issues the seven calls in order
  - ``sparse_moe_ffn_amd.workloads`` workload shapes and seeded inputs
  - ``sparse_moe_ffn_amd.build``     hipcc build of libmobmoe.so
"""
__all__ = ["binding", "layer", "workloads", "build"]
