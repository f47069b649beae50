"""Model shapes and workload presets for the DM0-style dual-expert merged-attention path.

Shapes: page "DM0 paper definition vs. Dexbotic code" (dregs-remover.com news 27019),
section 1 (key architecture conclusion): both experts are 28-layer Qwen3 stacks, the VLM
expert has hidden size 2048 and the action expert 1024, both use 16 query heads, 8 KV heads
and head dim 128, the action dimension is 32 and the chunk is 50 actions.
Denoising defaults: page "DM0.5: High-Performance Embodied VLA and OpenDM Open Source
Introduction", section 5.3 (10 diffusion steps) and section 7.3 (chunk size 50).
The FFN widths (6144 / 3072), RMSNorm eps 1e-6 and RoPE base 1e6 are fixed by the workload
definitions, not by the pages.

This module holds shapes only: no arithmetic of the method.
"""
from dataclasses import dataclass, field, replace

F32 = "f32"
BF16 = "bf16"
FP8 = "fp8_e4m3"


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    vlm_hidden: int
    act_hidden: int
    vlm_ffn: int
    act_ffn: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    action_dim: int
    chunk: int
    rms_eps: float = 1e-6
    rope_base: float = 1e6
    time_base: float = 1e4
    dtype: str = BF16
    vlm_mlp_dtype: str = BF16
    time_mod: bool = False     # DM0.5-style time-modulated action expert (page 2, section 5.2)
    qk_norm: bool = False      # Qwen3 per-head QK-norm in both experts (page 1, section 1: Qwen3 stacks)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: the model shape plus batch, prefix lengths and step count."""
    config_id: int
    name: str
    shape: ModelShape
    batch: int
    prefix_len: int            # fixed prefix length (ragged workloads: the cap)
    ragged: tuple = None       # (lo, hi) inclusive range of per-sample prefix lengths
    steps: int = 10
    kind: str = "denoise"      # "layer" | "denoise" | "prefill_denoise"
    extra: dict = field(default_factory=dict)


TINY = ModelShape(n_layers=2, vlm_hidden=256, act_hidden=128, vlm_ffn=768, act_ffn=384,
                  n_q_heads=4, n_kv_heads=2, head_dim=32, action_dim=32, chunk=50, dtype=F32,
                  vlm_mlp_dtype=F32)

DM0_BASE = ModelShape(n_layers=28, vlm_hidden=2048, act_hidden=1024, vlm_ffn=6144, act_ffn=3072,
                      n_q_heads=16, n_kv_heads=8, head_dim=128, action_dim=32, chunk=50,
                      dtype=BF16, vlm_mlp_dtype=BF16)


def _round_up(x, m):
    return (x + m - 1) // m * m


WORKLOADS = {
    1: Workload(1, "tiny merged-attention model, fp32, B=1, prefix 64, 4 Euler steps",
                TINY, batch=1, prefix_len=64, steps=4, kind="prefill_denoise"),
    2: Workload(2, "one DM0-base merged layer, bf16, B=1, prefix 816 + 50 action tokens",
                replace(DM0_BASE, n_layers=1), batch=1, prefix_len=816, steps=0, kind="layer"),
    3: Workload(3, "DM0-base 28-layer suffix denoise, bf16, B=1, prefix KV 816, 10 steps",
                DM0_BASE, batch=1, prefix_len=816, steps=10, kind="denoise"),
    4: Workload(4, "DM0-base suffix denoise, bf16, B=32, ragged prefix 600-1100, 10 steps",
                DM0_BASE, batch=32, prefix_len=_round_up(1100, 16), ragged=(600, 1100), steps=10,
                kind="denoise"),
    5: Workload(5, "DM0-base prefill (28 VLM layers, 816 tokens) + suffix denoise, bf16, B=8",
                DM0_BASE, batch=8, prefix_len=816, steps=10, kind="prefill_denoise"),
    6: Workload(6, "tiny model with the time-modulated action expert, fp32, B=3 ragged prefix 1-64, "
                   "4 Euler steps", replace(TINY, time_mod=True), batch=3, prefix_len=64, ragged=(1, 64),
                steps=4, kind="denoise"),
    7: Workload(7, "DM0-base suffix denoise with the time-modulated action expert, bf16, B=4, prefix KV 816, "
                   "10 steps", replace(DM0_BASE, time_mod=True), batch=4, prefix_len=816, steps=10,
                kind="denoise"),
    8: Workload(8, "tiny model with per-head QK-norm in both experts, fp32, B=2 ragged prefix 1-64, 3 Euler steps",
                replace(TINY, qk_norm=True), batch=2, prefix_len=64, ragged=(1, 64), steps=3,
                kind="prefill_denoise"),
    9: Workload(9, "DM0-base suffix denoise with per-head QK-norm, bf16, B=2, prefix KV 816, 10 steps",
                replace(DM0_BASE, qk_norm=True), batch=2, prefix_len=816, steps=10, kind="denoise"),
}


def workload(config_id: int, **overrides) -> Workload:
    w = WORKLOADS[config_id]
    return replace(w, **overrides) if overrides else w
