"""Seeded synthetic inputs for the decode megakernel: model shapes, bf16 weights,
a pre-filled bf16 KV cache and input tokens.

This module only draws random numbers and packs them as bf16 bit patterns; it
holds none of the decoder's arithmetic, so the CPU oracle and the HIP path can
both be fed from it without sharing any code of the method itself.

Recipe (the workloads described on the pages: a Llama-3.2-1B-shaped decoder at
batch 1 in the Hazy Research "megakernel" write-ups, and Cohere's batch-8 MoE
decode megakernel):
  * weights:  seed 0, N(0, 0.02) drawn in fp32, rounded to bf16 (round to
    nearest even); RMSNorm gains are exactly 1.0.
  * KV cache: seed 1, N(0, 1) -> bf16 for positions [0, prefill), zeros beyond.
  * tokens:   seed 2, uniform on [0, vocab).
Every tensor has its own stream ``default_rng([seed, tensor_id, chunk])`` over
fixed-size chunks, so the values do not depend on how many threads draw them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, Optional

import numpy as np

CHUNK = 1 << 22  # elements per independent random stream


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Shape of a Llama-style decoder (optionally a parallel-block MoE)."""

    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    prefill: int          # cached positions before the first decode step
    max_seq: int          # KV-cache capacity (positions)
    steps: int = 1        # greedy steps the workload runs
    batch: int = 1
    tied_embedding: bool = True
    n_experts: int = 0
    top_k: int = 0
    expert_ffn: int = 0
    parallel_block: bool = False
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0

    def replace(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny decoder, the Llama-3.2-1B shape at short and long
# context, the Llama-3-8B shape, and a synthetic batch-8 parallel-block MoE.
SHAPES: Dict[str, ModelShape] = {
    "tiny": ModelShape("tiny", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2,
                       head_dim=64, ffn=1024, vocab=4096, prefill=64, max_seq=128,
                       steps=1, rope_theta=10000.0),
    "llama1b_ctx128": ModelShape("llama1b_ctx128", n_layers=16, hidden=2048,
                                 n_q_heads=32, n_kv_heads=8, head_dim=64, ffn=8192,
                                 vocab=128256, prefill=128, max_seq=256, steps=32,
                                 rope_theta=500000.0),
    "llama1b_ctx8192": ModelShape("llama1b_ctx8192", n_layers=16, hidden=2048,
                                  n_q_heads=32, n_kv_heads=8, head_dim=64, ffn=8192,
                                  vocab=128256, prefill=8192, max_seq=8192 + 64,
                                  steps=32, rope_theta=500000.0),
    "llama8b_ctx2048": ModelShape("llama8b_ctx2048", n_layers=32, hidden=4096,
                                  n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
                                  vocab=128256, prefill=2048, max_seq=2048 + 64,
                                  steps=32, tied_embedding=False, rope_theta=500000.0),
    "moe_tiny": ModelShape("moe_tiny", n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2,
                           head_dim=128, ffn=0, vocab=4096, prefill=64, max_seq=128, steps=1,
                           batch=8, tied_embedding=False, n_experts=8, top_k=2, expert_ffn=512,
                           parallel_block=True, rope_theta=10000.0),
    "moe_b8_ctx2048": ModelShape("moe_b8_ctx2048", n_layers=24, hidden=2048,
                                 n_q_heads=16, n_kv_heads=4, head_dim=128, ffn=0,
                                 vocab=65536, prefill=2048, max_seq=2048 + 64, steps=32,
                                 batch=8, tied_embedding=False, n_experts=64, top_k=8,
                                 expert_ffn=1024, parallel_block=True,
                                 rope_theta=500000.0),
}

# Stable tensor ids: part of the recipe, never renumber.
TENSOR_IDS = {
    "embed": 1, "lm_head": 2, "final_norm": 3, "attn_norm": 4, "wq": 5, "wk": 6,
    "wv": 7, "wo": 8, "mlp_norm": 9, "w_gate": 10, "w_up": 11, "w_down": 12,
    "router": 13, "e_gate": 14, "e_up": 15, "e_down": 16,
    "k_cache": 101, "v_cache": 102, "tokens": 201,
}


def weight_shapes(s: ModelShape) -> Dict[str, tuple]:
    """bf16 tensors of the model, row-major [out, in], stacked over layers."""
    L, d, V = s.n_layers, s.hidden, s.vocab
    shapes = {
        "embed": (V, d),
        "final_norm": (d,),
        "attn_norm": (L, d),
        "wq": (L, s.q_dim, d),
        "wk": (L, s.kv_dim, d),
        "wv": (L, s.kv_dim, d),
        "wo": (L, d, s.q_dim),
    }
    if not s.tied_embedding:
        shapes["lm_head"] = (V, d)
    if s.is_moe:
        E, Fe = s.n_experts, s.expert_ffn
        shapes.update({"router": (L, E, d), "e_gate": (L, E, Fe, d),
                       "e_up": (L, E, Fe, d), "e_down": (L, E, d, Fe)})
    else:
        F = s.ffn
        shapes.update({"mlp_norm": (L, d), "w_gate": (L, F, d), "w_up": (L, F, d),
                       "w_down": (L, d, F)})
    return shapes


def _round_bf16_bits(f32: np.ndarray) -> np.ndarray:
    u = f32.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def _fill_normal_bf16(out: np.ndarray, seed: int, tid: int, std: float,
                      threads: int) -> None:
    flat = out.reshape(-1)
    n = flat.size
    n_chunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.default_rng([seed, tid, c])
        f = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            f *= np.float32(std)
        flat[lo:hi] = _round_bf16_bits(f)

    if n_chunks == 1 or threads <= 1:
        for c in range(n_chunks):
            work(c)
    else:
        with _cf.ThreadPoolExecutor(min(threads, n_chunks)) as ex:
            list(ex.map(work, range(n_chunks)))


def _default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


BF16_ONE = np.uint16(0x3F80)


def make_weights(s: ModelShape, seed: int = 0, std: float = 0.02,
                 threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All weights as uint16 arrays holding bf16 bit patterns.

    Norm gains are 1.0; when the embedding is tied, ``lm_head`` is the same
    array object as ``embed``.
    """
    threads = threads or _default_threads()
    out: Dict[str, np.ndarray] = {}
    for name, shape in weight_shapes(s).items():
        arr = np.empty(shape, dtype=np.uint16)
        if name.endswith("norm"):
            arr.fill(BF16_ONE)
        else:
            _fill_normal_bf16(arr, seed, TENSOR_IDS[name], std, threads)
        out[name] = arr
    if s.tied_embedding:
        out["lm_head"] = out["embed"]
    return out


def make_kv_cache(s: ModelShape, seed: int = 1, prefill: Optional[int] = None,
                  threads: Optional[int] = None):
    """(k_cache, v_cache), each uint16 bf16 [L, B, G, max_seq, Dh].

    Positions [0, prefill) hold N(0, 1) values taken as already-rotated keys;
    later positions are zero.
    """
    threads = threads or _default_threads()
    p = s.prefill if prefill is None else prefill
    if p > s.max_seq:
        raise ValueError("prefill exceeds max_seq")
    shape = (s.n_layers, s.batch, s.n_kv_heads, s.max_seq, s.head_dim)
    caches = []
    for name in ("k_cache", "v_cache"):
        c = np.zeros(shape, dtype=np.uint16)
        if p:
            body = np.empty((s.n_layers, s.batch, s.n_kv_heads, p, s.head_dim),
                            dtype=np.uint16)
            _fill_normal_bf16(body, seed, TENSOR_IDS[name], 1.0, threads)
            c[:, :, :, :p, :] = body
        caches.append(c)
    return caches[0], caches[1]


def make_tokens(s: ModelShape, seed: int = 2) -> np.ndarray:
    rng = np.random.default_rng([seed, TENSOR_IDS["tokens"]])
    return rng.integers(0, s.vocab, size=s.batch, dtype=np.int64).astype(np.int32)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (a storage conversion, not arithmetic)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def weight_bytes_per_step(s: ModelShape) -> int:
    """Bytes of weights one decode step streams (dense shapes): every layer
    matrix, the LM head, the norm gains and one embedding row per sequence."""
    if s.is_moe:
        raise ValueError("MoE weight bytes depend on routing")
    L, d = s.n_layers, s.hidden
    per_layer = 2 * (s.q_dim * d + 2 * s.kv_dim * d + d * s.q_dim + 3 * s.ffn * d + 2 * d)
    return L * per_layer + 2 * s.vocab * d + 2 * d + 2 * d * s.batch


def kv_bytes_per_step(s: ModelShape, pos: int) -> int:
    """KV-cache bytes one step reads (positions [0, pos)) and writes (pos)."""
    per_pos = 2 * 2 * s.n_layers * s.n_kv_heads * s.head_dim * s.batch
    return per_pos * pos + per_pos
