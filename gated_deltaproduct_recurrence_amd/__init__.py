"""MI355X-native chunked Gated DeltaProduct prefill.

The compute path is the HIP library ``libgdp.so`` (C ABI in include/gdp.h);
``binding`` marshals torch tensors into it.  Importing this package does not
load the library; ``from gated_deltaproduct_recurrence_amd import binding``
does, and fails loudly when it is not built.
"""
__all__ = ["binding", "workloads"]
