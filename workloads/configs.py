"""The five synthetic workloads of the QK-Norm + RoPE prologue.

Shapes follow the models the pages name: the Qwen2.5-0.5B fine-tuning run of
"Chronicals: A High-Performance Framework for LLM Fine-Tuning with 3.51x
Speedup over Unsloth" (abstract), grouped-query attention (HobbyLM and
JugnuLM abstracts), packed sequences from Best-Fit-Decreasing packing
(Chronicals abstract, contribution (4)) and partial rotation ("Fractional
Rotation, Full Potential? Investigating Performance and Convergence of Partial
RoPE", abstract).  Values the pages leave open (eps and value scale of the
packed and long-context cases, the outlier recipe) are fixed here.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int          # sequences (positions restart at 0 per sequence)
    seq: int            # tokens per sequence
    hq: int
    hkv: int
    head_dim: int
    rotary_dim: int
    dtype: str          # "bf16" or "f32": inputs, outputs, weights and weight grads
    eps: float
    theta: float
    backward: bool      # whether the workload includes the backward pass
    value_scale: float = 1.0          # Q/K ~ N(0, 1) * value_scale
    outlier_frac: float = 0.0         # fraction of [H*D] channels scaled by outlier_gain
    outlier_gain: float = 20.0
    packed: bool = False              # positions from a BFD-packed buffer of documents
    doc_len_min: int = 16
    doc_len_max: int = 4096
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def rows(self) -> int:
        return self.tokens * (self.hq + self.hkv)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def fwd_bytes(self) -> int:
        """Algorithmic bytes of one forward: read Q, K and positions, write the
        two outputs."""
        return self.tokens * (2 * (self.hq + self.hkv) * self.head_dim * self.elem_bytes + 4)

    def bwd_bytes(self) -> int:
        """Algorithmic bytes of one backward: read Q, K, their upstream
        gradients and positions, write dQ and dK."""
        return self.tokens * (3 * (self.hq + self.hkv) * self.head_dim * self.elem_bytes + 4)

    def with_tokens(self, batch: int, seq: int) -> "Workload":
        return replace(self, batch=batch, seq=seq)


TINY = Workload(
    name="tiny", seed=1, batch=1, seq=128, hq=4, hkv=2, head_dim=64, rotary_dim=64,
    dtype="f32", eps=1e-6, theta=1e4, backward=True,
    description="tiny fp32 fwd+bwd, 1x128 tokens, Hq=4 Hkv=2 D=64 full rotary")

QWEN05 = Workload(
    name="qwen05", seed=2, batch=8, seq=4096, hq=14, hkv=2, head_dim=64, rotary_dim=64,
    dtype="bf16", eps=1e-6, theta=1e6, backward=True, value_scale=2.0,
    description="Qwen2.5-0.5B-shaped bf16 fwd+bwd, 8x4096 tokens, Hq=14 Hkv=2 D=64")

PACKED = Workload(
    name="packed", seed=3, batch=1, seq=32768, hq=14, hkv=2, head_dim=64, rotary_dim=64,
    dtype="bf16", eps=1e-6, theta=1e6, backward=True, value_scale=2.0, packed=True,
    description="BFD-packed bf16 fwd+bwd, one 32768-token buffer, Hq=14 Hkv=2 D=64")

LLAMA7B = Workload(
    name="7b", seed=4, batch=4, seq=8192, hq=32, hkv=8, head_dim=128, rotary_dim=128,
    dtype="bf16", eps=1e-5, theta=5e5, backward=True, outlier_frac=0.01,
    description="7B-shaped bf16 fwd+bwd, 4x8192 tokens, Hq=32 Hkv=8 D=128, 1% outlier channels")

LONG = Workload(
    name="long", seed=5, batch=1, seq=131072, hq=64, hkv=8, head_dim=128, rotary_dim=32,
    dtype="bf16", eps=1e-6, theta=1e6, backward=False,
    description="long-context bf16 fwd-only, 131072 tokens, Hq=64 Hkv=8 D=128, rotary_dim=32")

ALL = {w.name: w for w in (TINY, QWEN05, PACKED, LLAMA7B, LONG)}


def get(name: str) -> Workload:
    return ALL[name]
