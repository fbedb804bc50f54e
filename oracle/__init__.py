"""CPU oracle of the decode step (test infrastructure only; see decoder.py)."""
from .decoder import (DecoderOracle, attend, bf16_to_f64, f64_to_bf16, greedy,
                      greedy_decode, rms_norm, rope, silu, softmax, top_k_ids)

__all__ = ["DecoderOracle", "attend", "bf16_to_f64", "f64_to_bf16", "greedy",
           "greedy_decode", "rms_norm", "rope", "silu", "softmax", "top_k_ids"]
