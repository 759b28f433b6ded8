"""Deflated ASP NVFP4 W4A4 linear for MI355X (gfx950).

The compute path lives in the HIP/C++ shared library ``libasp.so`` built from
``csrc/``; ``binding`` marshals arguments to its C entry points.  The library is
loaded on first use and a missing or stale build raises immediately: there is
no CPU fallback.
"""

__all__ = ["binding", "synth"]
