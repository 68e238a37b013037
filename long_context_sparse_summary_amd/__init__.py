"""MI355X-native coverage-rule sparse paged decode attention.

The compute path is the HIP library ``libmoira.so`` (gfx950) behind a C ABI;
``long_context_sparse_summary_amd.moira`` is its thin ctypes binding. Importing
this package does not load the library; the binding loads it on first use and
raises if it is missing.
"""
__all__ = ["moira", "workloads"]
