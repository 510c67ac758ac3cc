"""Seeded random-init weights, stored as raw bf16 bit patterns or float32.

Every projection, the tied embedding and both LoRA factors are drawn i.i.d.
from N(0, init_std^2).  Norm gains are ones: gains drawn from N(0, 0.02^2)
would shrink every normalised activation by ~50x.  LoRA B is drawn non-zero
on purpose so that the merged weights differ from the base weights.

Generation is split into fixed blocks, each seeded from
(shape_id, tensor index, block index), so the bytes do not depend on the
number of threads used to produce them.
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, List, Tuple

import numpy as np

from .configs import ModelShape

BLOCK = 1 << 22  # elements per independently seeded block


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns as uint16.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


@dataclass
class TensorSpec:
    name: str
    shape: Tuple[int, ...]
    kind: str            # "normal" or "ones"
    std: float = 0.0     # normal: 0 means the shape's init_std


def _mixer_shapes(s: ModelShape, full: bool) -> List[Tuple[str, Tuple[int, int]]]:
    d = s.d_model
    if full:
        hq, hkv, hd = s.fa_q_heads, s.fa_kv_heads, s.fa_head_dim
        return [("q", (hq * hd, d)), ("k", (hkv * hd, d)), ("v", (hkv * hd, d)),
                ("o", (d, hq * hd))]
    h, dk, dv = s.la_heads, s.la_dk, s.la_dv
    out = [("q", (h * dk, d)), ("k", (h * dk, d)), ("v", (h * dv, d)),
           ("g", (h, d)), ("o", (d, h * dv))]
    if s.la_kind == "gdn":
        out.append(("b", (h, d)))          # write strength beta = sigmoid(u . w_b)
    return out


def tensor_specs(s: ModelShape) -> List[TensorSpec]:
    """All tensors in their fixed generation order."""
    r = s.lora_rank
    specs = [TensorSpec("embed", (s.vocab, s.d_model), "normal")]
    for l in range(s.n_layers):
        p = f"layers.{l}"
        specs.append(TensorSpec(f"{p}.attn_norm", (s.d_model,), "ones"))
        mix = "fa" if s.is_full(l) else "la"
        for t, shp in _mixer_shapes(s, s.is_full(l)):
            specs.append(TensorSpec(f"{p}.{mix}.{t}", shp, "normal"))
        if mix == "la" and s.la_kind == "gdn":
            # depthwise causal convolution taps over the q | k | v channels
            specs.append(TensorSpec(f"{p}.la.conv", (s.la_heads * (2 * s.la_dk + s.la_dv), 4), "normal",
                                    s.conv_std))
        for t, shp in _mixer_shapes(s, s.is_full(l)):
            if t in s.lora_targets:
                specs.append(TensorSpec(f"{p}.{mix}.{t}.lora_A", (r, shp[1]), "normal"))
                specs.append(TensorSpec(f"{p}.{mix}.{t}.lora_B", (shp[0], r), "normal"))
        specs.append(TensorSpec(f"{p}.ffn_norm", (s.d_model,), "ones"))
        fshapes = [("gate", (s.ffn, s.d_model)), ("up", (s.ffn, s.d_model)),
                   ("down", (s.d_model, s.ffn))]
        for t, shp in fshapes:
            specs.append(TensorSpec(f"{p}.ffn.{t}", shp, "normal"))
        for t, shp in fshapes:
            if t in s.lora_targets:
                specs.append(TensorSpec(f"{p}.ffn.{t}.lora_A", (r, shp[1]), "normal"))
                specs.append(TensorSpec(f"{p}.ffn.{t}.lora_B", (shp[0], r), "normal"))
    specs.append(TensorSpec("final_norm", (s.d_model,), "ones"))
    return specs


@dataclass
class WeightSet:
    shape: ModelShape
    tensors: Dict[str, np.ndarray]   # uint16 bf16 bits (dtype bf16) or float32
    specs: List[TensorSpec]

    @property
    def storage(self) -> str:
        return self.shape.dtype

    def nbytes(self) -> int:
        return sum(a.nbytes for a in self.tensors.values())


def _fill_block(shape: ModelShape, tensor_index: int, block: int, out: np.ndarray, std: float = 0.0):
    rng = np.random.default_rng([shape.shape_id, 0, tensor_index, block])
    tmp = rng.standard_normal(out.size, dtype=np.float32)
    tmp *= np.float32(std or shape.init_std)
    if out.dtype == np.uint16:
        out[:] = f32_to_bf16_bits(tmp)
    else:
        out[:] = tmp


def make_weights(shape: ModelShape, threads: int = 0) -> WeightSet:
    """Draw every tensor of `shape`.  bf16 shapes return uint16 bit patterns."""
    specs = tensor_specs(shape)
    dt = np.uint16 if shape.dtype == "bf16" else np.float32
    one = np.uint16(0x3F80) if shape.dtype == "bf16" else np.float32(1.0)
    tensors: Dict[str, np.ndarray] = {}
    jobs = []
    for i, sp in enumerate(specs):
        a = np.empty(sp.shape, dtype=dt)
        tensors[sp.name] = a
        if sp.kind == "ones":
            a.fill(one)
            continue
        flat = a.reshape(-1)
        for b in range(0, flat.size, BLOCK):
            jobs.append((i, b // BLOCK, flat[b:b + BLOCK], sp.std))
    if threads <= 0:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads == 1 or len(jobs) < 4:
        for i, b, view, std in jobs:
            _fill_block(shape, i, b, view, std)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda j: _fill_block(shape, *j), jobs))
    return WeightSet(shape=shape, tensors=tensors, specs=specs)
