"""Seeded synthetic inputs for the decode-step workloads.

This module only *produces inputs*: projection weights, norm gains, KV caches,
hidden states and ragged request lengths, all from fixed seeds. It holds none of
the decode step's arithmetic, and it is the only code that the oracle and the
GPU path share. Values are drawn with torch's counter-based Philox generator on
whatever device the tensor lives on, so a test that needs the same inputs on the
CPU copies them from the device instead of regenerating them.

Distributions (the workloads state them; see ``workloads.py``):
  * projection weights   N(0, 0.02)   (0.02 is the standard deviation)
  * RMSNorm gains        1.0          (or N(1, 0.1) when ``random_gains``)
  * KV cache entries     N(0, 1)
  * input hidden states  N(0, 1)
  * ragged lengths       integers uniform on a closed range
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

from .workloads import Workload, WORKLOADS, get as get_workload  # noqa: F401


def seed_for(*key) -> int:
    """A stable 63-bit seed for a tuple key such as ("c2", "w_qkv", 7)."""
    h = hashlib.sha256(repr(tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def normal(shape, std: float, key, device="cpu", dtype=torch.float32, mean: float = 0.0) -> torch.Tensor:
    """N(mean, std) of ``shape`` drawn from the seed of ``key``, cast to ``dtype``
    (round-to-nearest-even for bfloat16)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_for(*key))
    t = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t if dtype == torch.float32 else t.to(dtype)


def fill_normal_(out: torch.Tensor, std: float, key, slab_elems: int = 1 << 28) -> torch.Tensor:
    """Fill a (possibly huge) tensor in place with N(0, std), slab by slab along
    dim 0, so the float32 staging buffer never exceeds ``slab_elems`` elements.
    Slab i uses the key ``key + ("slab", i)``."""
    flat0 = out.shape[0]
    inner = out[0].numel() if out.dim() > 1 else 1
    rows = max(1, slab_elems // max(inner, 1))
    i = 0
    for r0 in range(0, flat0, rows):
        r1 = min(flat0, r0 + rows)
        out[r0:r1].copy_(normal(out[r0:r1].shape, std, tuple(key) + ("slab", i), out.device, out.dtype))
        i += 1
    return out


def ragged_lengths(n: int, lo: int, hi: int, key) -> np.ndarray:
    """``n`` integers uniform on the closed range [lo, hi]."""
    rng = np.random.default_rng(seed_for(*key))
    return rng.integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.int32)


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_layer_weights(w: Workload, layer: int, device="cpu", random_gains: bool = False, tag: str = "") -> dict:
    """One decoder layer's tensors in the library's layout (row-major [out][in]).

    Dense layer: attn_norm[H], w_qkv[(Hq+2Hkv)d][H] (q rows, then k, then v),
    w_o[H][Hq d], ffn_norm[H], w_gate[F][H], w_up[F][H], w_down[H][F].
    MoE layer: the attention tensors plus w_router[E][H], w_exp_gate[E][Fe][H],
    w_exp_up[E][Fe][H], w_exp_down[E][H][Fe]. Norm gains are float32.
    """
    dt = torch_dtype(w.dtype)
    H, d = w.hidden, w.head_dim
    qkv_rows = (w.n_q_heads + 2 * w.n_kv_heads) * d
    k = (w.name + tag, layer)
    out = {}
    if random_gains:
        out["attn_norm"] = normal((H,), 0.1, k + ("attn_norm",), device, torch.float32, mean=1.0)
        out["ffn_norm"] = normal((H,), 0.1, k + ("ffn_norm",), device, torch.float32, mean=1.0)
    else:
        out["attn_norm"] = torch.ones(H, dtype=torch.float32, device=device)
        out["ffn_norm"] = torch.ones(H, dtype=torch.float32, device=device)
    out["w_qkv"] = normal((qkv_rows, H), w.w_std, k + ("w_qkv",), device, dt)
    out["w_o"] = normal((H, w.n_q_heads * d), w.w_std, k + ("w_o",), device, dt)
    if w.n_experts:
        E, Fe = w.n_experts, w.expert_ffn_dim
        out["w_router"] = normal((E, H), w.w_std, k + ("w_router",), device, dt)
        for name, shape in (("w_exp_gate", (E, Fe, H)), ("w_exp_up", (E, Fe, H)), ("w_exp_down", (E, H, Fe))):
            t = torch.empty(shape, dtype=dt, device=device)
            out[name] = fill_normal_(t, w.w_std, k + (name,))
    else:
        F = w.ffn_dim
        out["w_gate"] = normal((F, H), w.w_std, k + ("w_gate",), device, dt)
        out["w_up"] = normal((F, H), w.w_std, k + ("w_up",), device, dt)
        out["w_down"] = normal((H, F), w.w_std, k + ("w_down",), device, dt)
    return out


def make_kv_cache(w: Workload, max_batch: int, max_seq: int, device="cpu", n_layers=None, tag: str = "") -> torch.Tensor:
    """KV cache [L][2][max_batch][Hkv][max_seq][d] filled with N(0, 1).

    Every slot is filled, including slots past a request's length; the decode
    step only reads the first ``seq_lens[b] + 1`` positions. Cached keys are
    taken as already rotated (they stand for earlier decode steps' output).
    """
    L = w.n_layers if n_layers is None else n_layers
    kv = torch.empty((L, 2, max_batch, w.n_kv_heads, max_seq, w.head_dim), dtype=torch_dtype(w.dtype), device=device)
    for layer in range(L):
        fill_normal_(kv[layer], 1.0, (w.name + tag, "kv", layer))
    return kv


def make_hidden(w: Workload, batch: int, step: int = 0, device="cpu", tag: str = "") -> torch.Tensor:
    """Input hidden states [batch][H] float32, N(0, 1); a fresh draw per step."""
    return normal((batch, w.hidden), 1.0, (w.name + tag, "hidden", batch, step), device, torch.float32)
