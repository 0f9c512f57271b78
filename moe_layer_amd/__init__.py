"""moe_layer_amd: a fused Mixture-of-Experts layer for AMD MI355X (gfx950).

The layer (router softmax + top-k, token-to-expert alignment, grouped gate/up
GEMM with a fused SiLU-mul (+fp8 re-quant) epilogue, grouped down GEMM and the
router-weighted combine) runs in hand-written HIP kernels behind the C ABI of
``libmoe_mi355x.so`` (declared in ``include/moe.h``).  ``moe_layer_amd.ops``
is the thin Python binding with the same entry-point names; importing this
package does not load the library.
"""

__all__ = ["ops", "workloads"]
