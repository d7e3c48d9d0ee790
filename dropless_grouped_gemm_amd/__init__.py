"""Dropless MoE layer forward pass on MI355X (gfx950).

The compute path lives in the HIP shared library ``libmoe.so`` built from
``csrc/``; ``dropless_grouped_gemm_amd.binding`` marshals torch tensors into its
C-ABI.  Importing this package does not load the library (so the pure-Python
ledger stays usable without a GPU); ``binding.lib()`` does, and raises if it is
missing.
"""
__all__ = ["ledger"]
