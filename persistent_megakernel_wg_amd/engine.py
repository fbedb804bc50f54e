"""Engine: device buffers (PyTorch tensors) around one megakernel context.

PyTorch only allocates device memory and provides the stream; every step of
the decoder runs in libmk.so.  There is no fallback path: without a GPU or
without the built library the constructor raises.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import binding as B


def _device_bf16(arr: np.ndarray, torch, device):
    """Upload uint16 bf16 bit patterns as a torch.bfloat16 device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
    return t.to(device).view(torch.bfloat16)


class Engine:
    def __init__(self, shape, weights: Dict[str, np.ndarray], k_cache: np.ndarray,
                 v_cache: np.ndarray, device: int = 0, plan: Optional[B.MkPlanOpts] = None):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("Engine needs a GPU (the decode path has no CPU fallback)")
        B.load_library()
        self.torch = torch
        self.shape = shape
        self.dev = torch.device("cuda", device)
        self.tensors = {}
        for name, arr in weights.items():
            if name == "lm_head" and arr is weights.get("embed"):
                continue
            self.tensors[name] = _device_bf16(arr, torch, self.dev)
        self.k_cache = _device_bf16(k_cache, torch, self.dev)
        self.v_cache = _device_bf16(v_cache, torch, self.dev)
        w = B.MkWeights()
        for name in B.WEIGHT_FIELDS:
            t = self.tensors.get(name)
            if t is not None:
                setattr(w, name, t.data_ptr())
        if "lm_head" not in self.tensors:
            w.lm_head = self.tensors["embed"].data_ptr()
        w.k_cache = self.k_cache.data_ptr()
        w.v_cache = self.v_cache.data_ptr()
        self.cfg = B.config_from_shape(shape)
        torch.cuda.synchronize(self.dev)
        self.ctx = B.mk_create(self.cfg, w, device)
        B.mk_build_plan(self.ctx, plan)
        self.tokens = torch.zeros(shape.batch, dtype=torch.int32, device=self.dev)
        self.next = torch.zeros(shape.batch, dtype=torch.int32, device=self.dev)
        self.logits = torch.zeros(shape.batch, shape.vocab, dtype=torch.float32, device=self.dev)

    def plan_info(self) -> dict:
        return B.mk_plan_info(self.ctx)

    def rebuild_plan(self, plan: Optional[B.MkPlanOpts] = None) -> None:
        B.mk_build_plan(self.ctx, plan)

    def launch(self, pos: int, tokens=None, next_out=None, logits: bool = False, stream=None):
        """Enqueue one decode step (no synchronisation)."""
        t = self.tokens if tokens is None else tokens
        n = self.next if next_out is None else next_out
        s = (stream or self.torch.cuda.current_stream(self.dev)).cuda_stream
        B.mk_decode_step(self.ctx, t.data_ptr(), pos, n.data_ptr(),
                         self.logits.data_ptr() if logits else 0, s)

    def step(self, tokens: np.ndarray, pos: int, logits: bool = True):
        """One synchronous step from host tokens; returns (logits or None, next)."""
        self.tokens.copy_(self.torch.from_numpy(np.asarray(tokens, dtype=np.int32)))
        self.launch(pos, logits=logits)
        B.mk_sync(self.ctx)
        lg = self.logits.cpu().numpy().copy() if logits else None
        return lg, self.next.cpu().numpy().copy()

    def generate(self, tokens: np.ndarray, pos0: int, steps: int, logits: bool = False):
        """Greedy decode with the token chained on the device (one sync at the end
        unless logits are requested per step)."""
        torch = self.torch
        self.tokens.copy_(torch.from_numpy(np.asarray(tokens, dtype=np.int32)))
        bufs = [self.tokens] + [torch.zeros_like(self.next) for _ in range(steps)]
        out_logits = []
        for i in range(steps):
            self.launch(pos0 + i, tokens=bufs[i], next_out=bufs[i + 1], logits=logits)
            if logits:
                B.mk_sync(self.ctx)
                out_logits.append(self.logits.cpu().numpy().copy())
        B.mk_sync(self.ctx)
        toks = [b.cpu().numpy().copy() for b in bufs[1:]]
        return out_logits, toks

    def generate_resident(self, tokens: np.ndarray, pos0: int, steps: int, logits: bool = False,
                          stream=None):
        """Greedy decode of `steps` steps in one launch (mk_decode_steps);
        returns (logits [steps, B, V] or None, tokens [steps, B])."""
        torch = self.torch
        self.tokens.copy_(torch.from_numpy(np.asarray(tokens, dtype=np.int32)))
        out = torch.zeros(steps, self.shape.batch, dtype=torch.int32, device=self.dev)
        lg = (torch.zeros(steps, self.shape.batch, self.shape.vocab, dtype=torch.float32, device=self.dev)
              if logits else None)
        s = (stream or torch.cuda.current_stream(self.dev)).cuda_stream
        B.mk_decode_steps(self.ctx, self.tokens.data_ptr(), pos0, steps, out.data_ptr(),
                          lg.data_ptr() if logits else 0, s)
        B.mk_sync(self.ctx)
        return (lg.cpu().numpy() if logits else None), out.cpu().numpy()

    def read_kv(self):
        k = self.k_cache.view(self.torch.int16).cpu().numpy().view(np.uint16)
        v = self.v_cache.view(self.torch.int16).cpu().numpy().view(np.uint16)
        return k, v

    def sync(self):
        B.mk_sync(self.ctx)

    def close(self):
        if getattr(self, "ctx", None):
            try:
                self.torch.cuda.synchronize(self.dev)
            finally:
                B.mk_destroy(self.ctx)
                self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
