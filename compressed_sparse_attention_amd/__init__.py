"""CSA2 sparse attention over a compressed global KV cache, for MI355X (gfx950).

The compute path is the C-ABI library ``libcsa2.so`` (hand-written HIP kernels);
``compressed_sparse_attention_amd.csa2`` is its Python binding (argument
marshalling only).  Importing this package does not load the library; the first
call into the binding does, and raises if the library was not built.
"""
from . import ledger  # noqa: F401

__all__ = ["ledger"]
