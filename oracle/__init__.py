"""CPU oracle for the prefill-only decision path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  The product path (the HIP library and its
Python binding) never imports, calls or falls back to it, and this package
imports nothing from the product path: the two share no code.  Both consume
the same seeded input bytes from `s1_workloads`, which holds no arithmetic of
the method.

The oracle is the plain definition of what the path computes, written out in
numpy (float64 by default, float32 on request), slowly and without blocking
or fusion:

* hybrid decoder forward: pre-norm residual blocks; linear-attention or full
  causal-attention mixer, then a SwiGLU FFN (the 24-linear / 8-full 4B hybrid
  of RFC #114 "Native Rust/CUDA support for OmniJev-4B", section 1, and of the
  Cua-S1 4B 0.2 issue, first plan comment);
* the gated linear-attention recurrence S_t = g_t S_{t-1} + k_t v_t^T,
  o_t = S_t^T q_t (a stand-in for Gated DeltaNet, whose equations the pages do
  not print), with an fp32-or-wider state (RFC #114, section 5);
* causal softmax attention with GQA and rotate-half RoPE;
* LoRA merged into the storage dtype, W' = W + (alpha/r) B A (RFC #114,
  section 3: merge at load, qualified against the unmerged form);
* readout: softmax over the option-token logits of the tied embedding at the
  question's marker position (Cua-S1 issue, first plan comment), and the
  answer fields (sys1rust README, "Try it": answer types and the two
  confidence numbers);
* Gated DeltaNet (the gated delta rule with its short convolution and q/k
  L2 normalisation), token by token and in the chunked WY form (Yang et al.
  2024; Yang, Kautz, Hatamizadeh 2025), for shapes that ask for it;
* language-model features: token log-probabilities normalised over the full
  vocabulary, computed chunk by chunk, and a candidate score normalised across
  the candidates of a question (RFC #114, section 4, note under the semantics
  table);
* branches: a branch is the plain forward of prefix + suffix (RFC #114,
  section 4 "Branching" row and the "Plan: native OmniJev-4B v1.1" comment,
  which states a continuation equals the plain forward up to rounding).

Pins (tests marked "not gpu"): closed forms of the recurrence (g = 1, g = 0,
scalar case), brute-force attention loops, library attention, RoPE as complex
rotation, LoRA associativity, readout special cases printed on the sys1rust
page (even split -> confidence 0 and noul 0.5; one-hot -> confidence 1),
varlen = independent, continuation = plain forward.
"""
from .reference import (OracleModel, bf16_bits_to_float, round_to_bf16_bits,
                        rms_norm, rope_rotate_half, la_scan_recurrent,
                        la_scan_unrolled, la_scan_segmented, causal_attention, swiglu,
                        lora_merge, softmax, decision_fields, readout,
                        vocab_log_probs, candidate_log_probs, prefill_decide,
                        l2_normalize, silu, causal_conv_silu, gdn_recurrent, gdn_chunked, QTYPE_CHOICE, QTYPE_SCORE, QTYPE_NOUL)

__all__ = [
    "OracleModel", "bf16_bits_to_float", "round_to_bf16_bits", "rms_norm",
    "rope_rotate_half", "la_scan_recurrent", "la_scan_unrolled", "la_scan_segmented",
    "causal_attention", "swiglu", "lora_merge", "softmax", "decision_fields",
    "readout", "vocab_log_probs", "candidate_log_probs", "prefill_decide",
    "l2_normalize", "silu", "causal_conv_silu", "gdn_recurrent", "gdn_chunked", "QTYPE_CHOICE", "QTYPE_SCORE", "QTYPE_NOUL",
]
