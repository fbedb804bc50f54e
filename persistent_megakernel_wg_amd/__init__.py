"""MI355X (gfx950) batch-1 decode megakernel: one persistent HIP kernel per
decode step, interpreting host-built per-CU instruction queues synchronised by
counters in global memory.

    binding  — ctypes marshalling of include/mk.h (mk_create, mk_build_plan,
               mk_decode_step, mk_destroy, ...)
    engine   — device buffers (torch tensors) around one context
    synth    — seeded synthetic weights / KV cache / tokens
    build    — compiles libmk.so in-tree for gfx950
"""
from . import synth  # noqa: F401

__all__ = ["synth", "binding", "engine", "build"]
