"""W4A16 routed-expert MoE layer for one MI355X (gfx950).

The layer's work runs in the HIP library libmoe_w4a16.so (C ABI in
include/moe_w4a16.h); `binding` marshals arguments to it, `layer` owns device
buffers, `synth` makes seeded synthetic inputs.
"""
__all__ = ["binding", "layer", "synth", "build"]
