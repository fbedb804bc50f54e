"""CPU oracle: one greedy decode step of a Llama-style decoder, written plainly.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module; only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it. It shares no code with the HIP path.

What it computes (the plain definition the megakernel must reproduce):
  * Hazy Research's Llama-1B megakernel write-up (rocketrecap.com summary,
    "Fusing Operations with an On-GPU Interpreter"; javascript.cn article,
    section "Megakernel: 从零设计的融合思路") names the fused steps of one
    forward pass: RMSNorm + QKV projection + RoPE, attention, MLP.  The model is
    Llama-3.2-1B in bfloat16 at batch 1 ("Megakernel: The Core Solution").
  * Cohere's decode megakernel (airebao.com, «快在哪里» item 1) describes the
    parallel block: attention and the MoE both read one RMSNorm output and the
    branches meet in one residual add.
Everything is computed in float64 from bf16 weights widened exactly.  The two
places where floating point decides a discrete value take that decision on the
float32 rounding of the float64 value, the precision the GPU path works in:
  * the new key/value rows are rounded to bf16 (round to nearest even) when they
    are appended to the cache;
  * the greedy argmax (lowest index wins ties) and the MoE top-k selection
    (higher logit first, lower expert id wins ties).
Readings where the pages are silent (all standard Llama conventions):
  RMSNorm n = g * x / sqrt(mean(x^2) + eps); rotate-half RoPE with
  inv_freq_j = theta^(-2j/Dh) on pairs (j, j + Dh/2); query head h reads KV
  head h // (H/G); scores scaled by 1/sqrt(Dh); SwiGLU silu(Wg n) * (Wu n) with
  silu(z) = z / (1 + exp(-z)); pre-filled cache rows are already-rotated keys;
  MoE router: top-k of the raw logits, then a softmax over those k.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np


# ---------------------------------------------------------------- bf16 storage
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bf16 bit patterns; the decision is taken on the float32 value
    (float64 -> float32 nearest, then float32 -> bf16 nearest-even)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# ------------------------------------------------------------------ the pieces
def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """g * x / sqrt(mean(x^2) + eps) over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return gain * (x / np.sqrt(ms + eps))


def rope(v: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate-half RoPE of vectors v[..., Dh] at position pos.

    Dimension j (< Dh/2) and j + Dh/2 form a pair rotated by the angle
    pos * theta^(-2j/Dh)."""
    dh = v.shape[-1]
    half = dh // 2
    j = np.arange(half, dtype=np.float64)
    angle = float(pos) * np.power(float(theta), -2.0 * j / dh)
    c, s = np.cos(angle), np.sin(angle)
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - np.max(s))
    return e / np.sum(e)


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """One query head against P+1 cached rows: softmax(q K^T / sqrt(Dh)) V."""
    dh = q.shape[-1]
    scores = keys @ q / np.sqrt(dh)
    return softmax(scores) @ values


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def greedy(logits: np.ndarray) -> int:
    """Index of the largest float32 logit; the lowest index wins ties."""
    return int(np.argmax(np.asarray(logits, dtype=np.float64).astype(np.float32)))


def top_k_ids(logits: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest float32 logits, higher first, lower id on ties."""
    f = np.asarray(logits, dtype=np.float64).astype(np.float32)
    order = sorted(range(f.size), key=lambda e: (-float(f[e]), e))
    return np.array(order[:k], dtype=np.int64)


# --------------------------------------------------------------------- decoder
class DecoderOracle:
    """One decode step at a time over caller-owned bf16 KV caches.

    ``weights`` maps the tensor names of the weight layout (row-major
    [out, in], stacked over layers) to uint16 bf16 arrays.  ``keep_f64`` keeps
    the widened float64 matrices between steps (faster, more memory).
    """

    def __init__(self, shape, weights: Dict[str, np.ndarray], keep_f64: bool = True):
        self.s = shape
        self.w = weights
        self.keep = keep_f64
        self._f64: Dict[Tuple[str, int, int], np.ndarray] = {}

    # widened weights, per layer (and per expert)
    def m(self, name: str, layer: int = -1, expert: int = -1) -> np.ndarray:
        key = (name, layer, expert)
        hit = self._f64.get(key)
        if hit is not None:
            return hit
        src = self.w[name]
        if layer >= 0:
            src = src[layer]
        if expert >= 0:
            src = src[expert]
        val = bf16_to_f64(src)
        if self.keep:
            self._f64[key] = val
        return val

    def step(self, tokens: np.ndarray, pos: int, k_cache: np.ndarray,
             v_cache: np.ndarray, trace: Optional[dict] = None, seqs=None):
        """Decode one token per sequence at position ``pos``.

        tokens: int [B]; k_cache/v_cache: uint16 [L, B, G, max_seq, Dh], updated
        in place at ``pos``.  Returns (logits float64 [B, V], next int64 [B]).
        ``trace`` (optional dict) receives per-layer intermediates of sequence 0.
        ``seqs`` (optional) limits the work to those sequences (they do not
        interact); the other rows of the results are NaN / -1 and their cache
        rows are left as they were.
        """
        s = self.s
        if not 0 <= pos < s.max_seq:
            raise ValueError("pos outside the KV cache")
        B = s.batch
        logits = np.full((B, s.vocab), np.nan, dtype=np.float64)
        nxt = np.full(B, -1, dtype=np.int64)
        for b in (range(B) if seqs is None else seqs):
            x = bf16_to_f64(self.w["embed"][int(tokens[b])])
            for layer in range(s.n_layers):
                if s.parallel_block:
                    x = self._parallel_layer(x, layer, b, pos, k_cache, v_cache,
                                             trace if b == 0 else None)
                else:
                    x = self._dense_layer(x, layer, b, pos, k_cache, v_cache,
                                          trace if b == 0 else None)
            n = rms_norm(x, self.m("final_norm"), s.rms_eps)
            logits[b] = self.m("lm_head") @ n
            nxt[b] = greedy(logits[b])
            if trace is not None and b == 0:
                trace["final_norm"] = n
        return logits, nxt

    # attention sub-block shared by both layer kinds; returns Wo . o
    def _attention(self, n, layer, b, pos, k_cache, v_cache, tr):
        s = self.s
        H, G, dh = s.n_q_heads, s.n_kv_heads, s.head_dim
        q = (self.m("wq", layer) @ n).reshape(H, dh)
        k = (self.m("wk", layer) @ n).reshape(G, dh)
        v = (self.m("wv", layer) @ n).reshape(G, dh)
        if tr is not None:
            tr.setdefault("q_raw", []).append(q.copy())
            tr.setdefault("k_raw", []).append(k.copy())
            tr.setdefault("v_raw", []).append(v.copy())
        q = rope(q, pos, s.rope_theta)
        k = rope(k, pos, s.rope_theta)
        k_cache[layer, b, :, pos, :] = f64_to_bf16(k)
        v_cache[layer, b, :, pos, :] = f64_to_bf16(v)
        o = np.empty((H, dh))
        group = H // G
        for h in range(H):
            g = h // group
            keys = bf16_to_f64(k_cache[layer, b, g, :pos + 1, :])
            vals = bf16_to_f64(v_cache[layer, b, g, :pos + 1, :])
            o[h] = attend(q[h], keys, vals)
        if tr is not None:
            tr.setdefault("attn_out", []).append(o.reshape(-1).copy())
        return self.m("wo", layer) @ o.reshape(-1)

    def _dense_layer(self, x, layer, b, pos, k_cache, v_cache, tr):
        s = self.s
        n = rms_norm(x, self.m("attn_norm", layer), s.rms_eps)
        h = x + self._attention(n, layer, b, pos, k_cache, v_cache, tr)
        n2 = rms_norm(h, self.m("mlp_norm", layer), s.rms_eps)
        mid = silu(self.m("w_gate", layer) @ n2) * (self.m("w_up", layer) @ n2)
        out = h + self.m("w_down", layer) @ mid
        if tr is not None:
            tr.setdefault("x_in", []).append(x.copy())
            tr.setdefault("h", []).append(h.copy())
            tr.setdefault("mlp_mid", []).append(mid.copy())
            tr.setdefault("x_out", []).append(out.copy())
        return out

    def moe(self, n, layer, tr=None):
        """Top-k softmax-weighted sum of SwiGLU experts on one normed vector."""
        s = self.s
        r = self.m("router", layer) @ n
        ids = top_k_ids(r, s.top_k)
        wts = softmax(r[ids])
        acc = np.zeros_like(n)
        for e, wt in zip(ids, wts):
            mid = silu(self.m("e_gate", layer, int(e)) @ n) * (self.m("e_up", layer, int(e)) @ n)
            acc = acc + wt * (self.m("e_down", layer, int(e)) @ mid)
        if tr is not None:
            tr.setdefault("router_ids", []).append(ids)
            tr.setdefault("router_w", []).append(wts)
        return acc

    def _parallel_layer(self, x, layer, b, pos, k_cache, v_cache, tr):
        s = self.s
        n = rms_norm(x, self.m("attn_norm", layer), s.rms_eps)
        attn = self._attention(n, layer, b, pos, k_cache, v_cache, tr)
        out = x + attn + self.moe(n, layer, tr)
        if tr is not None:
            tr.setdefault("x_in", []).append(x.copy())
            tr.setdefault("x_out", []).append(out.copy())
        return out


def greedy_decode(shape, weights, k_cache, v_cache, tokens, pos0: int, steps: int,
                  oracle: Optional[DecoderOracle] = None):
    """Run ``steps`` greedy steps from ``pos0``; each step feeds its own argmax
    back as the next token.  Returns (list of logits, list of next tokens)."""
    orc = oracle or DecoderOracle(shape, weights)
    toks = np.asarray(tokens).copy()
    all_logits, all_next = [], []
    for i in range(steps):
        lg, nx = orc.step(toks, pos0 + i, k_cache, v_cache)
        all_logits.append(lg)
        all_next.append(nx.copy())
        toks = nx
    return all_logits, all_next
