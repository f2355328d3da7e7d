"""ctypes mirror of include/pmk.h and loader of the in-tree libpmk.so.

Argument marshalling only: every step of the decode path runs in the HIP
library. If libpmk.so is missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpmk.so")

PMK_ABI_VERSION = 1
(PMK_OK, PMK_ERR_ARG, PMK_ERR_OOM, PMK_ERR_DEVICE, PMK_ERR_TIMEOUT, PMK_ERR_SEQ, PMK_ERR_UNSUPPORTED,
 PMK_ERR_SCRATCH) = range(8)
PMK_F32, PMK_BF16 = 0, 1
PMK_ROWS, PMK_TILES = 0, 1

# pmk_set_schedule modes (include/pmk.h)
SCHED_FUSED, SCHED_PER_LAYER, SCHED_PER_STAGE, SCHED_BARRIER, SCHED_PER_OP = 0, 1, 2, 3, 4
SCHEDULES = {"fused": SCHED_FUSED, "layer": SCHED_PER_LAYER, "stage": SCHED_PER_STAGE, "barrier": SCHED_BARRIER,
             "op": SCHED_PER_OP}
# pmk_set_event_granularity modes
EVENTS_TILE, EVENTS_GROUP, EVENTS_STAGE = 0, 1, 2
EVENT_MODES = {"tile": EVENTS_TILE, "group": EVENTS_GROUP, "stage": EVENTS_STAGE}
# pmk_set_moe_scheduler modes
MOE_STATIC, MOE_DYNAMIC, MOE_DYNAMIC_XCD = 0, 1, 2
MOE_SCHEDULERS = {"static": MOE_STATIC, "dynamic": MOE_DYNAMIC, "xcd": MOE_DYNAMIC_XCD}

EXPORTS = ("decode_layer_init", "decode_step", "moe_layer_step", "decode_layer_destroy", "pmk_strerror",
           "pmk_get_device_error", "pmk_query", "pmk_timing_enable", "pmk_timing_read", "pmk_trace_attach",
           "pmk_set_schedule", "pmk_set_moe_scheduler", "pmk_set_watchdog_us", "pmk_pack_weights",
           "pmk_stream_probe", "pmk_set_event_granularity", "decode_step_static",
           "pmk_event_litmus")

i32, f32, vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class ModelDesc(ctypes.Structure):
    _fields_ = [("abi_version", i32), ("dtype", i32), ("n_layers", i32), ("hidden", i32), ("n_q_heads", i32),
                ("n_kv_heads", i32), ("head_dim", i32), ("ffn_dim", i32), ("n_experts", i32), ("top_k", i32),
                ("expert_ffn_dim", i32), ("max_batch", i32), ("max_seq", i32), ("rms_eps", f32),
                ("rope_theta", f32), ("watchdog_ms", i32), ("weight_layout", i32), ("reserved", i32 * 5)]


LAYER_FIELDS = ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate", "w_up", "w_down", "w_router",
                "w_exp_gate", "w_exp_up", "w_exp_down")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, vp) for n in LAYER_FIELDS]


class Weights(ctypes.Structure):
    _fields_ = [("n_layers", i32), ("layers", ctypes.POINTER(LayerWeights))]


ROUTING_FIELDS = ("topk_idx", "topk_w", "router_logits", "exp_indptr", "tile_indptr", "sorted_tok", "sorted_slot")


class Routing(ctypes.Structure):
    _fields_ = [(n, vp) for n in ROUTING_FIELDS]


class Info(ctypes.Structure):
    _fields_ = [("grid", i32), ("block", i32), ("lds_bytes", i32), ("moe_bm", i32), ("attn_chunk", i32),
                ("max_queue", i32), ("workspace_bytes", ctypes.c_int64), ("arch", i32), ("reserved", i32 * 7)]


_lib = None


def load():
    """Load libpmk.so from the package directory (built by build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m persistent_megakernel_04_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.decode_layer_init.argtypes = [P(ModelDesc), P(Weights), P(vp)]
    L.decode_layer_init.restype = i32
    L.decode_step.argtypes = [vp, vp, vp, vp, i32, vp]
    L.decode_step.restype = i32
    L.moe_layer_step.argtypes = [vp, vp, vp, vp, i32, P(Routing), vp]
    L.moe_layer_step.restype = i32
    L.decode_layer_destroy.argtypes = [vp]
    L.decode_layer_destroy.restype = i32
    L.pmk_strerror.argtypes = [i32]
    L.pmk_strerror.restype = ctypes.c_char_p
    L.pmk_get_device_error.argtypes = [vp]
    L.pmk_get_device_error.restype = i32
    L.pmk_query.argtypes = [vp, P(Info)]
    L.pmk_query.restype = i32
    L.pmk_timing_enable.argtypes = [vp, i32]
    L.pmk_timing_enable.restype = i32
    L.pmk_timing_read.argtypes = [vp, P(ctypes.c_double), P(i32)]
    L.pmk_timing_read.restype = i32
    L.pmk_trace_attach.argtypes = [vp, vp, i32]
    L.pmk_trace_attach.restype = i32
    L.pmk_set_schedule.argtypes = [vp, i32]
    L.pmk_set_schedule.restype = i32
    L.pmk_set_moe_scheduler.argtypes = [vp, i32]
    L.pmk_set_moe_scheduler.restype = i32
    L.pmk_set_watchdog_us.argtypes = [vp, i32]
    L.pmk_set_watchdog_us.restype = i32
    L.pmk_pack_weights.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, vp]
    L.pmk_pack_weights.restype = i32
    L.pmk_stream_probe.argtypes = [vp, ctypes.c_int64, i32, i32, vp, vp, P(ctypes.c_double)]
    L.pmk_stream_probe.restype = i32
    L.pmk_set_event_granularity.argtypes = [vp, i32]
    L.pmk_set_event_granularity.restype = i32
    L.decode_step_static.argtypes = [P(ModelDesc), P(Weights), vp, vp, vp, i32, vp, vp]
    L.decode_step_static.restype = i32
    L.pmk_event_litmus.argtypes = [vp, ctypes.c_int64, i32, vp, vp]
    L.pmk_event_litmus.restype = i32
    _lib = L
    return L


class PmkError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        msg = load().pmk_strerror(code).decode() if _lib is not None else str(code)
        super().__init__(f"{what}: {msg} (code {code})")


def check(code: int, what: str):
    if code != PMK_OK:
        raise PmkError(code, what)
