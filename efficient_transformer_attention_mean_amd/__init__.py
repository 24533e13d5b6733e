"""Nyström self-attention forward on MI355X (gfx950): HIP kernels behind a C ABI.

``_lib`` binds the C entry points of ``libnystrom.so`` (same names as
``include/nystrom.h``); ``api`` adds tensor-level checks; ``workloads`` draws
the seeded synthetic inputs.  Importing this package does not load the
library; the first call does, and fails loudly if it is not built.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads"]
