"""libflarepp: the FLARE++ routing forward pass (seed encode -> encode ->
decode) as hand-written HIP kernels for gfx950 behind a C-ABI library.

Submodules are imported on demand: ``inputs`` (seeded synthetic problems,
no GPU needed) and ``flarepp`` (the ctypes binding of libflarepp.so).
"""
__all__ = ["inputs", "flarepp"]
