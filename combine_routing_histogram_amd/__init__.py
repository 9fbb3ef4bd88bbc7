"""MI355X (gfx950) MoE expert-parallel dispatch/combine hot path.

``binding`` is the ctypes layer over libepdc.so (include/epdc.h); ``op`` holds
EpDispatchCombineConfig / EpDispatchCombineOp on top of it; ``workloads``
draws seeded synthetic inputs.  Submodules are imported on use so that the
input generator works without the HIP library.
"""
__all__ = ["binding", "op", "workloads", "build"]
