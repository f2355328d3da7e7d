"""Shared builders for the GPU parity tests, smoke() and bench.py's parity check.

Inputs come from the seeded generator (``synth``); the oracle receives host
copies of exactly the tensors the GPU receives, taken before the GPU step runs.
Nothing here computes any part of the decode step.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import synth


def to_np(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor: float32 stays float32, bfloat16 becomes its uint16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@dataclass
class Case:
    w: object            # synth Workload
    n_layers: int
    layers: list         # per-layer dicts of device tensors
    kv: torch.Tensor     # device KV cache
    hidden: torch.Tensor
    seq_lens: torch.Tensor
    max_batch: int
    max_seq: int


def build_case(w, batch: int, lens, n_layers: int | None = None, max_seq: int | None = None, max_batch=None,
               device="cuda", tag: str = "", random_gains: bool = False) -> Case:
    L = w.n_layers if n_layers is None else n_layers
    lens = np.asarray(lens, np.int32)
    assert lens.shape == (batch,)
    ms = int(max_seq if max_seq is not None else lens.max() + 1)
    mb = int(max_batch if max_batch is not None else batch)
    layers = [synth.make_layer_weights(w, l, device=device, random_gains=random_gains, tag=tag) for l in range(L)]
    kv = synth.make_kv_cache(w, mb, ms, device=device, n_layers=L, tag=tag)
    hidden = synth.make_hidden(w, batch, 0, device=device, tag=tag)
    sl = torch.tensor(lens, dtype=torch.int32, device=device)
    return Case(w, L, layers, kv, hidden, sl, mb, ms)


def oracle_inputs(case: Case, requests=None):
    """Host copies for the oracle (call before the GPU step). ``requests``
    selects a subset of batch rows (each request is independent)."""
    rq = list(range(case.hidden.shape[0])) if requests is None else list(requests)
    kv = case.kv[:, :, rq] if requests is not None else case.kv
    return {
        "layers": [{k: to_np(v) for k, v in L.items()} for L in case.layers],
        "kv": np.ascontiguousarray(to_np(kv)),
        "hidden": to_np(case.hidden)[rq].astype(np.float64),
        "seq_lens": to_np(case.seq_lens)[rq],
        "requests": rq,
    }


def run_oracle_dense(orc, case: Case, inp) -> tuple[np.ndarray, np.ndarray]:
    desc = orc.make_desc(case.w, len(inp["requests"]), case.max_seq, n_layers=case.n_layers)
    kv = inp["kv"]
    out = orc.decode_stack(desc, inp["layers"], kv, inp["seq_lens"], inp["hidden"])
    return out, kv


def make_model(case: Case, watchdog_ms: int = 0, weight_layout: str = "rows"):
    from persistent_megakernel_04_amd import DecodeModel
    return DecodeModel.from_workload(case.w, case.layers, case.max_batch, case.max_seq, n_layers=case.n_layers,
                                     watchdog_ms=watchdog_ms, weight_layout=weight_layout)
