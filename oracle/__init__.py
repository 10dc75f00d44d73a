"""CPU oracle (float64) for the DiT block: test infrastructure, never product code."""
from .h3dit_oracle import (LOG2E, apply_rope, attention, bf16_round, block_forward, dit_forward,
                           euler_sample, final_layer, gelu_tanh, modulated_norm, modulation,
                           patchify, rms_normalize, rope_frequencies, scaled_query,
                           split_modulation, unpatchify)

__all__ = ["LOG2E", "apply_rope", "attention", "bf16_round", "block_forward", "dit_forward",
           "euler_sample", "final_layer", "gelu_tanh", "modulated_norm", "modulation", "patchify",
           "rms_normalize", "rope_frequencies", "scaled_query", "split_modulation", "unpatchify"]
