"""ctypes binding of include/mk.h: the same entry points, argument marshalling only.

Every step of the decode path runs inside libmk.so (HIP kernels for gfx950);
this module only converts Python values to the C structs and raises on errors.
Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK = 0
TRACE_WORDS = 16  # words per traced instruction
STATUS_NAMES = {0: "MK_OK", -1: "MK_ERR_INVALID_ARG", -2: "MK_ERR_HIP", -3: "MK_ERR_NO_PLAN",
                -4: "MK_ERR_UNSUPPORTED", -5: "MK_ERR_OOM", -6: "MK_ERR_TIMEOUT",
                -7: "MK_ERR_DEVICE"}


class MkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS_NAMES.get(status, "?"), status, msg))
        self.status = status


class MkConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "max_seq",
        "batch", "tied_embedding", "n_experts", "top_k", "expert_ffn", "parallel_block")] + [
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


WEIGHT_FIELDS = ("embed", "lm_head", "final_norm", "attn_norm", "wq", "wk", "wv", "wo",
                 "mlp_norm", "w_gate", "w_up", "w_down", "router", "e_gate", "e_up", "e_down",
                 "k_cache", "v_cache")


class MkWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class MkPlanOpts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_cus", "mlp_chunks", "attn_block", "watchdog_ms", "debug_corrupt_target",
        "generic_kernel", "attn_heads", "o_split", "mfma", "edn_queue", "egu_balance", "gu_all")]


class MkPlanSummary(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_cus", "n_instr", "max_queue", "n_counters", "lds_bytes", "n_pages", "page_bytes",
        "attn_block", "attn_tiles", "mlp_chunks")] + [
        (n, ctypes.c_int64) for n in ("weight_bytes", "max_cu_bytes", "min_cu_bytes")] + [
        ("kernel_variant", ctypes.c_int32), ("scratch_bytes", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


EXPORTS = ("mk_create", "mk_build_plan", "mk_decode_step", "mk_sync", "mk_destroy",
           "mk_last_error", "mk_plan_info", "mk_plan_check", "mk_trace_enable", "mk_trace_read",
           "mk_route_stats", "mk_decode_step_noalloc", "mk_stream_read", "mk_decode_steps")
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # MK_NOALLOC_SCRATCH_BYTES

_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmk.so (built by persistent_megakernel_wg_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmk.so is not built: run `python -m persistent_megakernel_wg_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    lib.mk_create.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(MkWeights), ctypes.c_int,
                              ctypes.POINTER(vp)]
    lib.mk_build_plan.argtypes = [vp, ctypes.POINTER(MkPlanOpts)]
    lib.mk_decode_step.argtypes = [vp, vp, i32, vp, vp, vp]
    lib.mk_decode_step_noalloc.argtypes = [vp, vp, i32, vp, vp, vp]
    lib.mk_decode_steps.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    lib.mk_sync.argtypes = [vp]
    lib.mk_destroy.argtypes = [vp]
    lib.mk_last_error.argtypes = [vp]
    lib.mk_last_error.restype = ctypes.c_char_p
    lib.mk_plan_info.argtypes = [vp, ctypes.POINTER(MkPlanSummary)]
    lib.mk_plan_check.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(MkPlanOpts), i32,
                                  ctypes.POINTER(MkPlanSummary), ctypes.c_char_p, ctypes.c_size_t]
    lib.mk_trace_enable.argtypes = [vp, ctypes.c_int]
    lib.mk_trace_read.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), ctypes.c_size_t,
                                  ctypes.POINTER(i32)]
    lib.mk_route_stats.argtypes = [vp, ctypes.POINTER(ctypes.c_int64), i32, ctypes.c_int]
    lib.mk_stream_read.argtypes = [vp, ctypes.c_size_t, vp, i32, vp]
    for name in ("mk_create", "mk_build_plan", "mk_decode_step", "mk_decode_step_noalloc", "mk_sync",
                 "mk_destroy",
                 "mk_plan_info", "mk_plan_check", "mk_trace_enable", "mk_trace_read",
                 "mk_route_stats", "mk_stream_read", "mk_decode_steps"):
        getattr(lib, name).restype = st
    _lib = lib
    return lib


def _check(status: int, ctx=None) -> None:
    if status != MK_OK:
        msg = load_library().mk_last_error(ctx)
        raise MkError(status, msg.decode() if msg else "")


def config_from_shape(shape) -> MkConfig:
    """MkConfig from any object with the ModelShape attributes."""
    return MkConfig(n_layers=shape.n_layers, hidden=shape.hidden, n_q_heads=shape.n_q_heads,
                    n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim, ffn=shape.ffn,
                    vocab=shape.vocab, max_seq=shape.max_seq, batch=shape.batch,
                    tied_embedding=int(shape.tied_embedding), n_experts=shape.n_experts,
                    top_k=shape.top_k, expert_ffn=shape.expert_ffn,
                    parallel_block=int(shape.parallel_block), rms_eps=shape.rms_eps,
                    rope_theta=shape.rope_theta)


def plan_opts(n_cus=0, mlp_chunks=0, attn_block=0, watchdog_ms=0, debug_corrupt_target=0,
              generic_kernel=0, attn_heads=0, o_split=0, mfma=0, edn_queue=0,
              egu_balance=0, gu_all=0):
    return MkPlanOpts(n_cus=n_cus, mlp_chunks=mlp_chunks, attn_block=attn_block,
                      watchdog_ms=watchdog_ms, debug_corrupt_target=debug_corrupt_target,
                      generic_kernel=generic_kernel, attn_heads=attn_heads, o_split=o_split,
                      mfma=mfma, edn_queue=edn_queue, egu_balance=egu_balance,
                      gu_all=gu_all)


# ------------------------------------------------------------ the C entry points
def mk_create(cfg: MkConfig, weights: MkWeights, device: int = 0) -> int:
    lib = load_library()
    out = ctypes.c_void_p()
    _check(lib.mk_create(ctypes.byref(cfg), ctypes.byref(weights), device, ctypes.byref(out)))
    return out.value


def mk_build_plan(ctx: int, opts: Optional[MkPlanOpts] = None) -> None:
    lib = load_library()
    _check(lib.mk_build_plan(ctx, ctypes.byref(opts) if opts is not None else None), ctx)


def mk_decode_step(ctx: int, d_tokens: int, pos: int, d_next: int, d_logits: int = 0,
                   stream: int = 0) -> None:
    lib = load_library()
    _check(lib.mk_decode_step(ctx, d_tokens, pos, d_next, d_logits or None, stream or None), ctx)


def mk_decode_step_noalloc(ctx: int, d_tokens: int, pos: int, d_next: int, d_logits: int = 0,
                           stream: int = 0) -> None:
    lib = load_library()
    _check(lib.mk_decode_step_noalloc(ctx, d_tokens, pos, d_next, d_logits or None, stream or None), ctx)


def mk_decode_steps(ctx: int, d_tokens: int, pos: int, n_steps: int, d_next: int, d_logits: int = 0,
                    stream: int = 0) -> None:
    lib = load_library()
    _check(lib.mk_decode_steps(ctx, d_tokens, pos, n_steps, d_next, d_logits or None, stream or None), ctx)


def mk_sync(ctx: int) -> None:
    _check(load_library().mk_sync(ctx), ctx)


def mk_destroy(ctx: Optional[int]) -> None:
    _check(load_library().mk_destroy(ctx))


def mk_last_error(ctx: Optional[int] = None) -> str:
    msg = load_library().mk_last_error(ctx)
    return msg.decode() if msg else ""


def mk_plan_info(ctx: int) -> dict:
    s = MkPlanSummary()
    _check(load_library().mk_plan_info(ctx, ctypes.byref(s)), ctx)
    return s.as_dict()


def mk_plan_check(cfg: MkConfig, n_cus: int, opts: Optional[MkPlanOpts] = None):
    """Host-only plan build + verification; returns (summary dict, report str)."""
    s = MkPlanSummary()
    buf = ctypes.create_string_buffer(1 << 16)
    _check(load_library().mk_plan_check(ctypes.byref(cfg),
                                         ctypes.byref(opts) if opts is not None else None,
                                         n_cus, ctypes.byref(s), buf, len(buf)))
    return s.as_dict(), buf.value.decode()


def mk_route_stats(ctx: int, n_layers: int, reset: bool = False):
    """Distinct experts selected per layer, summed over steps (list of ints)."""
    buf = (ctypes.c_int64 * n_layers)()
    _check(load_library().mk_route_stats(ctx, buf, n_layers, int(reset)), ctx)
    return list(buf)


def mk_trace_enable(ctx: int, on: bool = True) -> None:
    _check(load_library().mk_trace_enable(ctx, int(on)), ctx)


def mk_trace_read(ctx: int, n_cus: int, max_queue: int):
    """Trace of the last step as a uint32 array [n_cus, stride, 16]."""
    import numpy as np
    buf = np.zeros(n_cus * max_queue * TRACE_WORDS, dtype=np.uint32)
    stride = ctypes.c_int32()
    _check(load_library().mk_trace_read(
        ctx, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), buf.size,
        ctypes.byref(stride)), ctx)
    return buf[: n_cus * stride.value * TRACE_WORDS].reshape(n_cus, stride.value, TRACE_WORDS)


def mk_stream_read(d_src: int, nbytes: int, d_sink: int, blocks: int, stream: int = 0) -> None:
    """Enqueue one streaming read of nbytes at d_src (calibration kernel)."""
    _check(load_library().mk_stream_read(d_src, nbytes, d_sink, blocks, stream or None))
