"""libmsa: the Memory Sparse Attention hot path (block pooling, routing scan,
Top-k, context gather, sparse GQA decode) as hand-written HIP for MI355X.

`msa` is the ctypes binding of the C ABI declared in include/msa.h.
"""
from . import msa  # noqa: F401
