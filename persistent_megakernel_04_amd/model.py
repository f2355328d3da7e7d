"""A handle on the decode library, holding torch tensors for device memory.

PyTorch provides device memory and streams only; every operation of the decode
step runs inside libpmk.so's kernels. The methods below pass data pointers and
the current HIP stream through the C ABI with the same names as the C entry
points.
"""
from __future__ import annotations

import ctypes

import torch

from . import _abi


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# weight matrices of a layer (the RMSNorm gains stay as they are)
MATRIX_FIELDS = ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "w_router", "w_exp_gate", "w_exp_up", "w_exp_down")


def pack_weights(t: torch.Tensor) -> torch.Tensor:
    """pmk_pack_weights: a new tensor holding the bfloat16 weight tensor t
    ([..., rows, cols], the leading dimensions stacked) in the tile layout."""
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError("pack_weights takes a contiguous bfloat16 device tensor")
    cols = t.shape[-1]
    out = torch.empty_like(t)
    _abi.check(_abi.load().pmk_pack_weights(_ptr(t), _ptr(out), t.numel() // cols, cols, _stream()),
               "pmk_pack_weights")
    return out


def pack_layers(layers: list) -> list:
    """Each layer dict with its weight matrices replaced by tile-layout copies."""
    return [{k: (pack_weights(v) if k in MATRIX_FIELDS and v is not None else v) for k, v in L.items()}
            for L in layers]


class DecodeModel:
    """Wraps decode_layer_init / decode_step / moe_layer_step / decode_layer_destroy.

    ``layers`` is a list of dicts of device tensors in the library layout
    (see include/pmk.h); the tensors must stay alive while the model is used
    (this object keeps references)."""

    def __init__(self, *, dtype: str, n_layers: int, hidden: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 ffn_dim: int = 0, n_experts: int = 0, top_k: int = 0, expert_ffn_dim: int = 0,
                 max_batch: int, max_seq: int, rms_eps: float = 1e-5, rope_theta: float = 10000.0,
                 layers: list, watchdog_ms: int = 0, weight_layout: str = "rows"):
        self.lib = _abi.load()
        d = _abi.ModelDesc()
        d.abi_version = _abi.PMK_ABI_VERSION
        d.dtype = _abi.PMK_BF16 if dtype == "bf16" else _abi.PMK_F32
        d.n_layers, d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim = n_layers, hidden, n_q_heads, n_kv_heads, head_dim
        d.ffn_dim, d.n_experts, d.top_k, d.expert_ffn_dim = ffn_dim, n_experts, top_k, expert_ffn_dim
        d.max_batch, d.max_seq, d.rms_eps, d.rope_theta, d.watchdog_ms = max_batch, max_seq, rms_eps, rope_theta, watchdog_ms
        if weight_layout not in ("rows", "tiles"):
            raise ValueError(f"weight_layout must be 'rows' or 'tiles', not {weight_layout!r}")
        d.weight_layout = _abi.PMK_TILES if weight_layout == "tiles" else _abi.PMK_ROWS
        self.desc = d
        self._layers = layers
        arr = (_abi.LayerWeights * n_layers)()
        for i, L in enumerate(layers):
            for f in _abi.LAYER_FIELDS:
                t = L.get(f)
                setattr(arr[i], f, None if t is None else t.data_ptr())
        self._arr = arr
        w = _abi.Weights(n_layers, arr)
        h = ctypes.c_void_p()
        _abi.check(self.lib.decode_layer_init(ctypes.byref(d), ctypes.byref(w), ctypes.byref(h)), "decode_layer_init")
        self.handle = h

    @classmethod
    def from_workload(cls, w, layers, max_batch, max_seq, n_layers=None, watchdog_ms=0, weight_layout="rows",
                      pack=True):
        """weight_layout "tiles": with pack, `layers` are row-major and are
        packed into tile-layout copies held by the model (twice the weight
        memory while the caller keeps its tensors); without, they already are
        in the tile layout (pack_layers)."""
        if weight_layout == "tiles" and pack:
            layers = pack_layers(layers)
        return cls(dtype=w.dtype, n_layers=w.n_layers if n_layers is None else n_layers, hidden=w.hidden,
                   n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn_dim=w.ffn_dim,
                   n_experts=w.n_experts, top_k=w.top_k, expert_ffn_dim=w.expert_ffn_dim, max_batch=max_batch,
                   max_seq=max_seq, rms_eps=w.rms_eps, rope_theta=w.rope_theta, layers=layers,
                   watchdog_ms=watchdog_ms, weight_layout=weight_layout)

    # -- entry points -------------------------------------------------------
    def decode_step(self, hidden: torch.Tensor, kv_cache: torch.Tensor, seq_lens: torch.Tensor) -> int:
        """Raw status of decode_step (0 = launched)."""
        return self.lib.decode_step(self.handle, _ptr(hidden), _ptr(kv_cache), _ptr(seq_lens),
                                    int(hidden.shape[0]), _stream())

    def moe_layer_step(self, hidden, kv_cache, seq_lens, routing: dict | None = None) -> int:
        r = None
        if routing is not None:
            r = _abi.Routing(*[None if routing.get(f) is None else routing[f].data_ptr() for f in _abi.ROUTING_FIELDS])
        return self.lib.moe_layer_step(self.handle, _ptr(hidden), _ptr(kv_cache), _ptr(seq_lens),
                                       int(hidden.shape[0]), None if r is None else ctypes.byref(r), _stream())

    def decode_step_static(self, hidden: torch.Tensor, kv_cache: torch.Tensor, seq_lens: torch.Tensor,
                           status: torch.Tensor | None = None) -> int:
        """Raw status of decode_step_static with this model's descriptor and
        weights: the same step without the handle's workspace (the library's
        static scratch instead; nothing is allocated). `status`: an optional
        one-element int32 device tensor for the step's device error code."""
        w = _abi.Weights(self.desc.n_layers, self._arr)
        return self.lib.decode_step_static(ctypes.byref(self.desc), ctypes.byref(w), _ptr(hidden), _ptr(kv_cache),
                                           _ptr(seq_lens), int(hidden.shape[0]), _ptr(status), _stream())

    def step(self, hidden, kv_cache, seq_lens, routing=None):
        """Checked call: decode_step (dense) or moe_layer_step (MoE)."""
        if self.desc.n_experts:
            _abi.check(self.moe_layer_step(hidden, kv_cache, seq_lens, routing), "moe_layer_step")
        else:
            _abi.check(self.decode_step(hidden, kv_cache, seq_lens), "decode_step")

    def device_error(self) -> int:
        return self.lib.pmk_get_device_error(self.handle)

    def info(self) -> dict:
        i = _abi.Info()
        _abi.check(self.lib.pmk_query(self.handle, ctypes.byref(i)), "pmk_query")
        return {f: getattr(i, f) for f, _ in _abi.Info._fields_ if f != "reserved"}

    def timing_enable(self, on: bool = True):
        _abi.check(self.lib.pmk_timing_enable(self.handle, 1 if on else 0), "pmk_timing_enable")

    def timing_read(self):
        ms, n = ctypes.c_double(), ctypes.c_int32()
        _abi.check(self.lib.pmk_timing_read(self.handle, ctypes.byref(ms), ctypes.byref(n)), "pmk_timing_read")
        return ms.value, n.value

    def trace_attach(self, buf, entries_per_wg: int = 0):
        """Attach a device uint32/int32 tensor of grid * entries_per_wg * 8 elements as the task trace
        (None detaches)."""
        _abi.check(self.lib.pmk_trace_attach(self.handle, _ptr(buf), int(entries_per_wg)), "pmk_trace_attach")
        self._trace = buf

    def set_schedule(self, mode):
        """'fused' (one persistent launch per step, stages chained by events), 'layer' (one launch per layer),
        'stage' (one launch per stage of each layer) or 'barrier' (one launch, a grid-wide barrier after every
        stage): the same task code in every mode."""
        m = _abi.SCHEDULES[mode] if isinstance(mode, str) else int(mode)
        _abi.check(self.lib.pmk_set_schedule(self.handle, m), "pmk_set_schedule")

    def set_event_granularity(self, mode):
        """'group' (the default: per KV group), 'tile' (per KV group and, beyond 16 rows, batch block) or 'stage' (one event
        per stage): how finely the dense chain's consumers wait on their producers."""
        m = _abi.EVENT_MODES[mode] if isinstance(mode, str) else int(mode)
        _abi.check(self.lib.pmk_set_event_granularity(self.handle, m), "pmk_set_event_granularity")

    def set_moe_scheduler(self, mode):
        """'static' (each workgroup a fixed share of the grouped expert tasks), 'dynamic' (tasks popped from
        a per-layer queue, down tasks queued as their experts' gate/up tasks finish) or 'xcd' (the same tasks
        popped from a counter per XCD, with stealing)."""
        m = _abi.MOE_SCHEDULERS[mode] if isinstance(mode, str) else int(mode)
        _abi.check(self.lib.pmk_set_moe_scheduler(self.handle, m), "pmk_set_moe_scheduler")

    def set_watchdog_us(self, us: int):
        """Event-wait limit of later steps in microseconds; 0 restores the limit set at init."""
        _abi.check(self.lib.pmk_set_watchdog_us(self.handle, int(us)), "pmk_set_watchdog_us")

    def close(self):
        if getattr(self, "handle", None):
            self.lib.decode_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
