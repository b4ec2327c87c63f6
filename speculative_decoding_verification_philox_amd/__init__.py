"""DropMatch verify step on MI355X: hand-written HIP kernels behind a C ABI.

``binding`` holds the ctypes binding of libdmverify.so (same names as
include/dm_verify.h); ``workloads`` draws seeded synthetic inputs; ``build``
compiles the library with hipcc for gfx950.
"""
__all__ = ["binding", "workloads", "build"]
