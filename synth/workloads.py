"""The decode workloads: shapes, dtypes, batch/length recipes.

Shapes are those of the public model families the pages evaluate (Llama-3.1-8B,
Qwen3-30B-A3B, Llama-70B) with random weights; nothing here is a trained model
or a dataset item. ``-shaped`` means dimensions only: no vocabulary head, no
long-context RoPE scaling, no biases, no per-head q/k norm.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": storage of weights and KV cache
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int          # dense SwiGLU width (0 for MoE layers)
    n_experts: int = 0
    top_k: int = 0
    expert_ffn_dim: int = 0
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    w_std: float = 0.02
    batches: tuple = (1,)
    seq_lo: int = 0       # ragged lengths ~ U{seq_lo..seq_hi}; equal lo/hi = fixed length
    seq_hi: int = 0
    decode_steps: int = 1
    notes: str = ""
    tol: float = 1e-2     # relative L2 bound on the output, GPU vs oracle

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def layer_params(self) -> int:
        """Parameters of one layer that a decode step streams (all experts counted)."""
        H, d = self.hidden, self.head_dim
        p = self.qkv_rows * H + H * self.q_dim
        if self.n_experts:
            p += self.n_experts * H + self.n_experts * 3 * H * self.expert_ffn_dim
        else:
            p += 3 * H * self.ffn_dim
        return p


WORKLOADS = {
    # tiny single layer, fp32, batch 1, 128 cached positions
    "c1_tiny_f32": Workload(
        name="c1_tiny_f32", dtype="f32", n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
        ffn_dim=688, batches=(1,), seq_lo=128, seq_hi=128, tol=1e-5,
        notes="tiny single decoder layer, fp32"),
    # Llama-3.1-8B-shaped 32-layer stack, bf16, batch 1, 512 cached positions, 100 decode steps
    "c2_8b_b1": Workload(
        name="c2_8b_b1", dtype="bf16", n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        ffn_dim=14336, batches=(1,), seq_lo=512, seq_hi=512, decode_steps=100,
        notes="Llama-3.1-8B-shaped decode stack"),
    # same stack, batch sweep with ragged lengths U{512..8192}
    "c3_8b_sweep": Workload(
        name="c3_8b_sweep", dtype="bf16", n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        ffn_dim=14336, batches=(1, 4, 16, 64, 128), seq_lo=512, seq_hi=8192,
        notes="Llama-3.1-8B-shaped decode stack, ragged batch sweep"),
    # Qwen3-30B-A3B-shaped MoE layer: 128 experts, top-8, expert FFN 768, KV length 2048
    "c4_moe": Workload(
        name="c4_moe", dtype="bf16", n_layers=1, hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128,
        ffn_dim=0, n_experts=128, top_k=8, expert_ffn_dim=768, batches=(1, 4, 16, 64, 128),
        seq_lo=2048, seq_hi=2048, notes="Qwen3-30B-A3B-shaped MoE decode layer"),
    # one GPU's share of the Llama-70B shape under 8-way tensor parallelism: 8 query heads and 1 KV head
    # (the heads split 8 ways), FFN 28672 / 8; all 80 layers, batch 8, ragged U{8192..16384}
    "c5_tp8_share": Workload(
        name="c5_tp8_share", dtype="bf16", n_layers=80, hidden=8192, n_q_heads=8, n_kv_heads=1, head_dim=128,
        ffn_dim=3584, batches=(8,), seq_lo=8192, seq_hi=16384,
        notes="per-GPU share of the 70B-shaped stack under 8-way tensor parallelism (no all-reduce)"),
    # one GPU's share of the MoE layer under 8-way expert parallelism: the 16 local experts of 128; each
    # token brings one routed row (top-1 over the local experts), so T tokens give T rows at T / 16 per
    # expert, the density that an 8-way dispatch of T tokens' top-8 choices delivers to one GPU
    "c4_ep8_share": Workload(
        name="c4_ep8_share", dtype="bf16", n_layers=1, hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128,
        ffn_dim=0, n_experts=16, top_k=1, expert_ffn_dim=768, batches=(1, 16, 128), seq_lo=2048, seq_hi=2048,
        notes="per-GPU share of the MoE layer under 8-way expert parallelism (no all-to-all)"),
    # Llama-70B-shaped 80-layer stack, bf16, batch 8, ragged U{8192..16384}
    "c5_70b": Workload(
        name="c5_70b", dtype="bf16", n_layers=80, hidden=8192, n_q_heads=64, n_kv_heads=8, head_dim=128,
        ffn_dim=28672, batches=(8,), seq_lo=8192, seq_hi=16384,
        notes="Llama-70B-shaped decode stack at full HBM footprint"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
