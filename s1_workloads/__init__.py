"""Seeded synthetic inputs for the prefill-only decision path.

This package only *draws* inputs: model shapes, random weights (stored as raw
bf16 bit patterns or float32), token ids, sequence lengths and question
layouts.  It contains none of the method's arithmetic (no norms, no
projections, no attention, no scan, no readout) so that both the CPU oracle
and the HIP path can consume the same bytes without sharing any code that
computes.

Workloads (shapes fixed here; the pages describe a 4B hybrid with 24 linear
and 8 full-attention layers and a rank-32/alpha-64 LoRA merged into bf16
weights -- RFC #114 "Native Rust/CUDA support for OmniJev-4B", section 1,
and Cua-S1 4B 0.2 issue #10, first plan comment):

  tiny-fp32          2 layers (linear, full), d 256, fp32
  4b-single-512      4B-class bf16, one 512-token request, 3 questions
  4b-varlen-16       4B-class bf16, 16 packed requests of 256..2048 tokens
  4b-branch-4096x20  4B-class bf16, 4096-token prefix + 20 branches of 64
  27b-single-1024    27B-class bf16, one 1024-token request, 1 question
"""
from .configs import (ModelShape, SHAPES, WORKLOADS, Workload, shape_of,
                      workload)
from .batch import Batch, make_batch, QTYPE_CHOICE, QTYPE_SCORE, QTYPE_NOUL
from .weights import (WeightSet, make_weights, tensor_specs, f32_to_bf16_bits)

__all__ = [
    "ModelShape", "SHAPES", "WORKLOADS", "Workload", "shape_of", "workload",
    "Batch", "make_batch", "QTYPE_CHOICE", "QTYPE_SCORE", "QTYPE_NOUL",
    "WeightSet", "make_weights", "tensor_specs", "f32_to_bf16_bits",
]
