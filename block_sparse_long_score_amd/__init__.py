"""MiniMax Sparse Attention (MSA) hot path for MI355X (gfx950).

The compute lives in ``libmsa.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/msa.h``).  ``ops`` is a thin ctypes binding with the same
entry-point names; ``inputs`` draws seeded synthetic workloads.  Importing the
package loads nothing: the library is opened on the first call and a missing
library raises instead of falling back to anything else.
"""
__all__ = ["ops", "inputs"]
