"""MI355X (gfx950) hot path of lookahead sparse-KV decode attention.

``ops`` marshals torch tensors into liboasis.so (HIP kernels behind the C ABI
of include/oasis.h); ``synth`` draws the seeded synthetic inputs.  Importing
the package loads nothing; the first ``ops`` call loads the library and fails
loudly if it is not built.
"""
from . import ops, synth  # noqa: F401

__all__ = ["ops", "synth"]
