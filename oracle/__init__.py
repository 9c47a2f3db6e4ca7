"""CPU oracle for the exact k-row verification step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The library in
``speculative_decode_verification_amd`` never does, and this package imports
nothing from it: the two share no code (only the seeded input generators in
``synth`` serve both).

Everything is plain numpy in fp64.  The method (decode-once multi-row
products, in-kernel snapshots, rollback by selection) reaches its plain
definition exactly up to rounding order, so each function here is that plain
definition written out.  Sources, by page and section:

* mere.run transfer report ("Flash-Next optimization transfer to Ornith and
  Qwen 27B"): "Shared architecture and implemented paths" (affine Q4, group
  size 64, bf16 tensors; fused gate/up expert weights; accepted-prefix
  rollback), "Exact verification kernels and benchmark admission" (a width-k
  row equals the serial width-1 product exactly; gathered experts over the
  rows' top-8 of 256), "Checkpoint correctness" (every accepted-prefix GDN
  rollback; snapshot isolation).
* Red Lite dev45 ("speculative decoding with the Qwen3-Next MTP block"),
  "What it is": each row of a multi-row product is computed separately; row
  t of the DeltaNet runs from the state after row t-1 and that state is
  snapshotted; one router dispatch and the union of the rows' experts;
  rolling back means picking the snapshot of the accepted prefix.
* Red Lite dev45, "Acceptance": draft t stands when it equals the token
  sampled from row t-1's logits, which leaves the output distribution that of
  plain decoding for any sampler; dev45b: a draft that matches the
  end-of-answer token is refused.
* Flash-Next plan, "2.1 Gated DeltaNet" and "5.1 Gated DeltaNet": the
  preparation (a 4-tap filter along time per q, k and v channel over the
  current and the three earlier inputs, the earlier ones carried between
  calls; q and k scaled to unit L2 norm per head; g from A_log and dt_bias
  by softplus and exp, beta = sigmoid(b)) and the gated RMSNorm output.
* mere.run transfer report, "Shared architecture and implemented paths": the
  gathered expert kernel's Flash-Next Q3 specialization (affine, group 64,
  3-bit codes; the bit packing is our definition).
* Red Lite dev45, "What it is": the MTP block's experts are Q8_0 (GGUF
  blocks of 32 signed 8-bit codes and one half-precision scale), with the
  same value per code as the dense Q8_0 decode.
* Flash-Next plan (QWEN38FLASH.md): "2.1 Gated DeltaNet" (decay, kv_mem,
  delta, rank-1 update, readout on fp32 [Hv, Dv, Dk]), "2.3 MoE" (routed +
  shared experts, SwiGLU, gate+up concatenated), "3.1 Overlap" (per-head
  scalar decay and beta; each k head shared by Hv/Hk v heads).

Pins (tests/test_oracle_pins.py) tie each function to something other than
itself: exact rational brute force, integer-exact cases, closed forms,
invariants the pages state, and reductions to textbook routines.  Readings
the pages leave open (nibble order, router tie-break, union order, combine
order, GQA head grouping, shared-expert gate) are our definitions; where a
choice is not fixed by the pages it is marked "parity unpinned by the pages"
in the function's docstring.
"""

from .ref import (bf16_to_f64, unpack_q4, dequant, qmv, route, union_pairs, silu, swiglu,
                  combine, moe_verify, gdn_verify, rollback, sample_tokens, accept, verify_cycle,
                  softplus, gdn_prepare, gdn_gated_norm, CONV_TAPS, fp16_to_f64, dequant_q8_0,
                  qmv_q8_0, Q8_BLOCK, unpack_q3, dequant_q3, qmv_q3)

__all__ = ["bf16_to_f64", "unpack_q4", "dequant", "qmv", "route", "union_pairs", "silu",
           "swiglu", "combine", "moe_verify", "gdn_verify", "rollback", "sample_tokens", "accept",
           "verify_cycle", "softplus", "gdn_prepare", "gdn_gated_norm", "CONV_TAPS", "fp16_to_f64",
           "dequant_q8_0", "qmv_q8_0", "Q8_BLOCK", "unpack_q3", "dequant_q3", "qmv_q3"]
