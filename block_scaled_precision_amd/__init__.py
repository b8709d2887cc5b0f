"""Fused microscaling (MX) mixture-of-experts layer for AMD MI355X (gfx950).

The compute lives in ``libmoe_mx.so`` (HIP kernels behind the C ABI of
``include/moe_mx.h``); ``block_scaled_precision_amd.moe_mx`` is its ctypes
binding, ``block_scaled_precision_amd.inputs`` the seeded synthetic inputs and
``block_scaled_precision_amd.build`` the in-tree build.  Importing the package
loads nothing; the library is opened on first use.
"""
__all__ = ["moe_mx", "inputs", "build"]
