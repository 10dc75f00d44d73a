"""CPU oracle (float64) for the DiT block: test infrastructure, never product code."""
from .h3dit_oracle import (LOG2E, apply_rope, attention, bf16_round, block_forward, gelu_tanh,
                           modulated_norm, modulation, rms_normalize, rope_frequencies,
                           scaled_query, split_modulation)

__all__ = ["LOG2E", "apply_rope", "attention", "bf16_round", "block_forward", "gelu_tanh",
           "modulated_norm", "modulation", "rms_normalize", "rope_frequencies",
           "scaled_query", "split_modulation"]
