"""Seeded synthetic inputs shared by the oracle, the tests and the bench.

This package generates inputs and nothing else. It holds none of the
verification arithmetic (no dequantisation, no matvec, no routing, no
recurrence), so the CPU oracle and the HIP path can both draw from it
without sharing any of the method's code.

Two generators are used:

* numpy ``default_rng`` seeded with ``[SEED, cfg, tensor, layer, step]`` for
  the small floating-point tensors (activations, router logits, GDN state and
  per-row q/k/v/g/beta);
* a counter-based generator (SplitMix64's output function applied to
  ``key + (ctr + 1) * gamma``; Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014) for the packed Q4 weight banks,
  which reach tens of GB.  Its values are pure integer functions of
  (key, counter), so ``synth/fill.hip`` fills the same banks on the device bit
  for bit, and the CPU side can regenerate any single expert or row on demand.
"""

from .counter import (GAMMA, SEED, derive_key, mix64, rand64, bf16_bits_from_f32,
                      q4_code_words, q4_affine_bf16, q4_rows)
from . import configs
from .inputs import (BankKeys, bank_keys, activations, dense_weight, moe_layer_inputs, gdn_layer_inputs,
                     gdn_state, accepted_prefix, integer_exact_weight, verify_block, gumbel_noise,
                     gdn_raw_inputs, q8_0_weight, q3_weight)

__all__ = [
    "GAMMA", "SEED", "derive_key", "mix64", "rand64", "bf16_bits_from_f32",
    "q4_code_words", "q4_affine_bf16", "q4_rows", "configs", "BankKeys", "bank_keys", "activations",
    "dense_weight", "moe_layer_inputs", "gdn_layer_inputs", "gdn_state", "verify_block", "gumbel_noise",
    "gdn_raw_inputs", "q8_0_weight", "q3_weight",
    "accepted_prefix", "integer_exact_weight",
]
