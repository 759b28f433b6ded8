"""Deflated ASP NVFP4 W4A4 linear for MI355X (gfx950).

The compute path lives in the HIP/C++ shared library ``libasp.so`` built from
``csrc/``; ``binding`` marshals arguments to its C entry points.  The library is
loaded on first use; a missing build, one of another ABI revision, or one built
from other sources than those beside it (a digest of csrc/ and include/ is
compiled in) raises immediately: there is no CPU fallback.
"""

__all__ = ["binding", "synth"]
