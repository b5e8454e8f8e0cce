"""MI355X-native fused Mixture-of-Experts layer.

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI of
include/moe_layer.h; `moe_layer_router_amd.lib` is its Python binding and
`moe_layer_router_amd.layer` a small convenience wrapper that allocates the
outputs and the workspace with PyTorch.
"""
