"""Chunked gated linear recurrence (Gated DeltaNet / GLA) for AMD MI355X.

The layer runs as hand-written HIP kernels for gfx950 behind a C ABI
(``include/clr.h``); ``ops`` is a thin ctypes binding over it and
``stateflow`` chains sequence chunks through the boundary state.
Nothing here is imported eagerly, so ``inputs`` can be used without the
native library.
"""
__all__ = ["ops", "stateflow", "inputs"]
