"""The five synthetic workloads, shaped like the models and contexts the pages
name (Llama-3.1-8B at 32K, a 70B model at 128K, Qwen2.5-3B with ragged
lengths; Super KV Compression page, background and results table;
TurboQuant page, long-context evaluation; nd-kv-quant page, background).

Shapes only: no weights or datasets are involved.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    index: int              # 1..5; seeds are 1000 + index
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    n_ctx: int              # cached tokens per sequence (upper bound if ragged)
    group_size: int
    k_bits: int = 6
    v_bits: int = 4
    dtype: str = "bf16"     # dtype of Q/K/V inputs
    outliers: bool = False  # 4 K channels per KV head scaled by 12
    tiered: bool = False    # attention-aware tiers + sparse-V skip
    fp16_layers: int = 0    # sensitive layers (of layers_per_stack) held in fp16
    layers_per_stack: int = 32
    ragged: tuple | None = None   # (lo, hi) context lengths
    steps: int = 1          # decode steps (append 1 token + decode)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


TINY = Workload("tiny_b1_h1_d64_n256_fp32", 1, batch=1, num_q_heads=1, num_kv_heads=1,
                head_dim=64, n_ctx=256, group_size=32, dtype="f32")

LLAMA8B_32K = Workload("llama8b_b8_hq32_hkv8_d128_n32768_k6v4", 2, batch=8, num_q_heads=32,
                       num_kv_heads=8, head_dim=128, n_ctx=32768, group_size=64, outliers=True)

LLAMA8B_32K_TIERED = replace(LLAMA8B_32K, name="llama8b_tiered_b8_n32768_k6v6_to_h6m4", index=3,
                             v_bits=6, tiered=True)

LLAMA70B_128K = Workload("llama70b_b2_hq64_hkv8_d128_n131072_k6v4", 4, batch=2, num_q_heads=64,
                         num_kv_heads=8, head_dim=128, n_ctx=131072, group_size=64, outliers=True,
                         fp16_layers=2)

QWEN3B_RAGGED = Workload("qwen3b_b64_hq16_hkv2_d128_ragged1k_16k_paged", 5, batch=64, num_q_heads=16,
                         num_kv_heads=2, head_dim=128, n_ctx=16384, group_size=64,
                         ragged=(1024, 16384), steps=128)

ALL = [TINY, LLAMA8B_32K, LLAMA8B_32K_TIERED, LLAMA70B_128K, QWEN3B_RAGGED]
BY_INDEX = {w.index: w for w in ALL}
