"""Ragged-paged decode attention for MI355X (gfx950).

A C ABI (include/tg.h, ``libtg.so``) with a host planner -- budget
reservation, clustering, tier split, ref-counted ragged page pools, block
tables, ahead-of-time split plan -- and HIP kernels for the cache fill, the
split-K decode with online softmax and in-register INT8 dequantisation, and
the log-sum-exp merge.  This package is the thin Python binding.
"""
from .api import *  # noqa: F401,F403
from .api import __all__  # noqa: F401
