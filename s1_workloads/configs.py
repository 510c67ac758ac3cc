"""Model shapes and named workloads (plain data, no arithmetic)."""
from dataclasses import dataclass, field
from typing import Tuple

# LoRA target names.  "gate" is the FFN gate projection, not the decay gate of
# the linear-attention mixer (which is never adapted).
LORA_MIXER = ("q", "k", "v", "o")
LORA_ALL = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    full_every: int          # layer l is full attention iff l % full_every == full_every - 1
    d_model: int
    ffn: int
    vocab: int
    la_heads: int
    la_dk: int
    la_dv: int
    fa_q_heads: int
    fa_kv_heads: int
    fa_head_dim: int
    lora_rank: int
    lora_alpha: float
    lora_targets: Tuple[str, ...]
    dtype: str               # "f32" or "bf16": storage and GEMM operand type
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    init_std: float = 0.02
    shape_id: int = 0        # seed component
    la_kind: str = "gla"     # "gla": the stated gated linear-attention stand-in;
                             # "gdn": Gated DeltaNet (short conv, L2-normalised q/k, delta rule)
    conv_std: float = 0.5    # GDN short-convolution taps (width 4)

    def is_full(self, layer: int) -> bool:
        return layer % self.full_every == self.full_every - 1

    @property
    def n_full(self) -> int:
        return sum(self.is_full(l) for l in range(self.n_layers))

    @property
    def n_linear(self) -> int:
        return self.n_layers - self.n_full

    def linear_params(self) -> int:
        """Parameters of every projection (no embedding, no norms)."""
        d, f = self.d_model, self.ffn
        la = d * self.la_heads * (2 * self.la_dk + self.la_dv) + d * self.la_heads \
            + self.la_heads * self.la_dv * d + (d * self.la_heads if self.la_kind == "gdn" else 0)
        fa = d * self.fa_head_dim * (self.fa_q_heads + 2 * self.fa_kv_heads) \
            + self.fa_q_heads * self.fa_head_dim * d
        ffn = 3 * d * f
        return self.n_linear * la + self.n_full * fa + self.n_layers * ffn


TINY = ModelShape(
    name="tiny-fp32", n_layers=2, full_every=2, d_model=256, ffn=688, vocab=4096,
    la_heads=4, la_dk=64, la_dv=64, fa_q_heads=4, fa_kv_heads=4, fa_head_dim=64,
    lora_rank=8, lora_alpha=16.0, lora_targets=LORA_MIXER, dtype="f32", shape_id=1)

H4B = ModelShape(
    name="4b", n_layers=32, full_every=4, d_model=2560, ffn=9728, vocab=151936,
    la_heads=16, la_dk=128, la_dv=128, fa_q_heads=16, fa_kv_heads=4, fa_head_dim=128,
    lora_rank=32, lora_alpha=64.0, lora_targets=LORA_ALL, dtype="bf16", shape_id=2)

H27B = ModelShape(
    name="27b", n_layers=64, full_every=4, d_model=5120, ffn=17408, vocab=151936,
    la_heads=40, la_dk=128, la_dv=128, fa_q_heads=40, fa_kv_heads=8, fa_head_dim=128,
    lora_rank=32, lora_alpha=64.0, lora_targets=LORA_ALL, dtype="bf16", shape_id=5)

H4B_GDN = ModelShape(
    name="4b-gdn", n_layers=32, full_every=4, d_model=2560, ffn=9728, vocab=151936,
    la_heads=16, la_dk=128, la_dv=128, fa_q_heads=16, fa_kv_heads=4, fa_head_dim=128,
    lora_rank=32, lora_alpha=64.0, lora_targets=LORA_ALL, dtype="bf16", shape_id=6, la_kind="gdn")

SHAPES = {s.name: s for s in (TINY, H4B, H27B, H4B_GDN)}


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    workload_id: int         # seed component for tokens / layout
    description: str = ""


WORKLOADS = {w.name: w for w in (
    Workload("tiny-fp32", TINY, 1,
             "tiny fp32 hybrid, 1 x 128 tokens, choice(3)+score(4)+noul"),
    Workload("4b-single-512", H4B, 2,
             "4B-class bf16, 1 x 512 tokens, choice(3)+score(4)+noul"),
    Workload("4b-varlen-16", H4B, 3,
             "4B-class bf16, 16 packed requests, lengths U[256,2048], 1-6 questions each"),
    Workload("4b-branch-4096x20", H4B, 4,
             "4B-class bf16, 4096-token prefix + 20 branches x 64 tokens"),
    Workload("27b-single-1024", H27B, 5,
             "27B-class bf16, 1 x 1024 tokens, one choice over 10 options"),
    Workload("4b-gdn-single-512", H4B_GDN, 6,
             "4B-class bf16 with Gated DeltaNet layers, 1 x 512 tokens, choice(3)+score(4)+noul"),
)}


def shape_of(name: str) -> ModelShape:
    return WORKLOADS[name].shape if name in WORKLOADS else SHAPES[name]


def workload(name: str) -> Workload:
    return WORKLOADS[name]
