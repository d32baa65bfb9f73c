"""Model shapes for the batch-1 fp16 decode path and the byte arithmetic that
prices one decode token against the HBM roofline.

The pages (Kog's inference engine KIE, as described on the studioglobal.ai
explainer pages, section on the monokernel and Delayed Tensor Parallelism)
never define the transformer block; they name a ~2.3B-parameter coding model
(Laneformer 2B) decoded at batch 1 in FP16 ("Laneformer 2B: results" table).
The shapes below are the synthetic stand-ins this package measures on: a
Llama-style pre-norm decoder (RMSNorm, rotate-half RoPE, SwiGLU, untied
embedding and LM head) at five sizes, plus the lane-structured variant with the
residual update delayed by two layers (the pages' 8 lanes and delay 2).

Nothing in this module computes the method; it only carries sizes.
"""
from __future__ import annotations

from dataclasses import dataclass, field, asdict, replace
from typing import Dict


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    # lane structure: n_lanes parallel lanes whose summed partials reach the
    # residual stream lane_delay layers later (parallel block).  n_lanes == 1
    # and lane_delay == 0 with sequential=True is the ordinary pre-norm block.
    n_lanes: int = 1
    lane_delay: int = 0
    sequential: bool = True
    # workload
    prompt_len: int = 16
    decode_steps: int = 32
    seed_index: int = 0
    description: str = ""

    # ----- derived sizes -------------------------------------------------
    @property
    def group(self) -> int:
        """query heads per KV head"""
        return self.n_heads // self.n_kv_heads

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def max_ctx(self) -> int:
        return self.prompt_len + self.decode_steps

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)

    def as_dict(self) -> Dict:
        return asdict(self)

    # ----- parameter / byte counts ---------------------------------------
    def layer_weight_elems(self) -> int:
        d, F = self.d_model, self.ffn_dim
        qkv = (self.q_dim + 2 * self.kv_dim) * d
        o = d * self.q_dim
        mlp = 3 * F * d
        norms = 2 * d
        return qkv + o + mlp + norms

    def param_elems(self) -> int:
        """every parameter, embedding table included"""
        return (self.n_layers * self.layer_weight_elems()
                + 2 * self.vocab * self.d_model + self.d_model)

    def streamed_weight_bytes(self) -> int:
        """fp16 bytes one decode token must read: all layer matrices and
        gains, the final gain, the LM head and ONE embedding row (the table
        itself is gathered, not streamed)."""
        elems = (self.n_layers * self.layer_weight_elems()
                 + self.vocab * self.d_model + self.d_model + self.d_model)
        return 2 * elems

    def kv_bytes_per_pos(self) -> int:
        """fp16 K and V bytes of one position over all layers"""
        return self.n_layers * 2 * self.kv_dim * 2

    def token_bytes(self, n_ctx: int) -> int:
        """algorithmic HBM bytes of one decode token attending over n_ctx
        positions (the current one included): weights + KV read + KV write"""
        kvp = self.kv_bytes_per_pos()
        return self.streamed_weight_bytes() + kvp * n_ctx + kvp

    def run_bytes(self, pos0: int, n_steps: int) -> int:
        """algorithmic bytes of n_steps decode tokens starting at position
        pos0 (step k attends over pos0 + k + 1 positions)"""
        kvp = self.kv_bytes_per_pos()
        ctx_sum = n_steps * (pos0 + 1) + n_steps * (n_steps - 1) // 2
        return n_steps * (self.streamed_weight_bytes() + kvp) + kvp * ctx_sum

    def token_flops(self, n_ctx: int) -> int:
        w = self.streamed_weight_bytes() // 2 - self.d_model  # MACs over matrices
        attn = 2 * self.n_heads * self.head_dim * n_ctx
        return 2 * w + 2 * attn


_STD = dict(rms_eps=1e-5, n_lanes=1, lane_delay=0, sequential=True)

CFG0 = ModelConfig(
    name="cfg0", n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
    ffn_dim=1024, vocab=4096, rope_base=10000.0, prompt_len=16, decode_steps=32,
    seed_index=0, description="tiny decoder, 2L d256 4x64 MHA F1024 V4096", **_STD)

CFG1 = ModelConfig(
    name="cfg1", n_layers=24, d_model=1024, n_heads=16, n_kv_heads=16, head_dim=64,
    ffn_dim=4096, vocab=32000, rope_base=10000.0, prompt_len=1024, decode_steps=256,
    seed_index=1, description="~400M-shaped dense decoder, 24L d1024 16x64 F4096 V32000",
    **_STD)

CFG2 = ModelConfig(
    name="cfg2", n_layers=28, d_model=2560, n_heads=20, n_kv_heads=20, head_dim=128,
    ffn_dim=6912, vocab=32000, rope_base=10000.0, prompt_len=2048, decode_steps=512,
    seed_index=2,
    description="~2.4B-shaped dense decoder, 28L d2560 20x128 MHA F6912 V32000", **_STD)

CFG3 = ModelConfig(
    name="cfg3", n_layers=28, d_model=2560, n_heads=32, n_kv_heads=32, head_dim=80,
    ffn_dim=6912, vocab=32000, rope_base=10000.0, rms_eps=1e-5, n_lanes=8,
    lane_delay=2, sequential=False, prompt_len=2048, decode_steps=512, seed_index=3,
    description=("lane-structured 2.4B-shaped decoder, 28L d2560 32x80, 8 lanes "
                 "(4 heads, 864 FFN columns each), residual delay 2 layers"))

CFG4 = ModelConfig(
    name="cfg4", n_layers=32, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128,
    ffn_dim=14336, vocab=128256, rope_base=500000.0, prompt_len=32768,
    decode_steps=256, seed_index=4,
    description="~8B-shaped GQA decoder, 32L d4096 32q/8kv x128 F14336 V128256, 32K ctx",
    **_STD)

PRESETS: Dict[str, ModelConfig] = {c.name: c for c in (CFG0, CFG1, CFG2, CFG3, CFG4)}


def preset(name: str) -> ModelConfig:
    if name.isdigit():
        name = "cfg" + name
    return PRESETS[name]
