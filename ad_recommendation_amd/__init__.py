"""mi355emb: one training step of a GPU-resident sparse embedding layer on MI355X.

The HIP library (libmi355emb.so, built in-tree) does the work; ``emb`` is its ctypes binding.
"""
from . import emb  # noqa: F401
