"""Routed mixture-of-experts FFN execution on AMD Instinct MI355X (gfx950).

The library is libmoe.so (C ABI in include/moe.h: HIP kernels plus the host
slot manager); routed_expert_execution_amd.moe is its Python binding.  Importing
the binding fails loudly when the library has not been built.
"""
