"""CPU oracle for the decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never does, and this
package imports nothing from it: the two share no code. Inputs come from the
seeded generator (``synth``) and are handed over as numpy arrays.

The arithmetic lives in ``pmk_oracle.c`` (plain C, double precision, OpenMP over
output rows and heads); this file only marshals arrays. bfloat16 tensors are
passed as their raw uint16 bit patterns.

Pinning: every function is pinned by ``tests/test_oracle_pins.py`` to closed
forms, invariants, library routines or brute force on tiny inputs (listed per
function there). The end-to-end layer has no worked example on the pages; it is
pinned through special cases that reduce to the separately pinned functions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pmk_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn_dim", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("expert_ffn_dim", ctypes.c_int32), ("max_batch", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double)]


_LAYER_FIELDS = ["attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate", "w_up", "w_down",
                 "w_router", "w_exp_gate", "w_exp_up", "w_exp_down"]


class Layer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _LAYER_FIELDS]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.orc_round_bf16.restype = D
        L.orc_round_bf16.argtypes = [D]
        L.orc_rmsnorm.argtypes = [P, P, I, D, P]
        L.orc_matvec.argtypes = [P, I, I, I, P, P]
        L.orc_rope.argtypes = [P, I, ctypes.c_long, D]
        L.orc_silu.restype = D
        L.orc_silu.argtypes = [D]
        L.orc_attention.argtypes = [P, P, P, I, I, I, I, I, I, P]
        L.orc_topk.argtypes = [P, I, I, P, P]
        L.orc_group.argtypes = [P, I, I, I, I, P, P, P, P]
        L.orc_decode_layer.argtypes = [P, P, P, P, I, P]
        L.orc_decode_layer_given_append.argtypes = [P, P, P, P, I, P]
        L.orc_decode_stack.argtypes = [P, P, P, P, I, P]
        L.orc_moe_layer.argtypes = [P, P, P, P, I, I, P, P, P, P, P, P, P, P]
        L.orc_moe_layer_routed.argtypes = [P, P, P, P, I, P, P, P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _storage(a):
    """Raw storage of a weight/cache array: float32, or uint16 bf16 bits."""
    if a.dtype == np.uint16:
        return np.ascontiguousarray(a), BF16
    return np.ascontiguousarray(a, dtype=np.float32), F32


# ------------------------------------------------------------------ ops ----

def round_bf16(v: float) -> float:
    return lib().orc_round_bf16(float(v))


def rmsnorm(x, g, eps):
    x = _c(x, np.float64)
    g = _c(g, np.float32)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_ptr(x), _ptr(g), x.size, float(eps), _ptr(out))
    return out


def matvec(W, x):
    W, dt = _storage(W)
    x = _c(x, np.float64)
    rows, cols = W.shape
    assert x.size == cols
    y = np.empty(rows, dtype=np.float64)
    lib().orc_matvec(_ptr(W), dt, rows, cols, _ptr(x), _ptr(y))
    return y


def rope(z, pos, theta):
    z = np.array(z, dtype=np.float64, copy=True)
    lib().orc_rope(_ptr(z), z.size, int(pos), float(theta))
    return z


def silu(z):
    return lib().orc_silu(float(z))


def attention(q, K, V, n):
    """q [Hq][d] doubles; K, V [Hkv][max_seq][d] (float32 or uint16 bf16 bits);
    attends over the first n positions. Returns o [Hq][d]."""
    q = _c(q, np.float64)
    K, dt = _storage(K)
    V, dt2 = _storage(V)
    assert dt == dt2
    Hq, d = q.shape
    Hkv, max_seq, d2 = K.shape
    assert d == d2 and 0 < n <= max_seq
    o = np.empty((Hq, d), dtype=np.float64)
    lib().orc_attention(_ptr(q), _ptr(K), _ptr(V), dt, Hq, Hkv, d, max_seq, int(n), _ptr(o))
    return o


def topk(z, k):
    z = _c(z, np.float32)
    idx = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    lib().orc_topk(_ptr(z), z.size, int(k), _ptr(idx), _ptr(w))
    return idx, w


def group(idx, n_experts, bm):
    """idx [T][k] int32 -> (exp_indptr, tile_indptr, sorted_tok, sorted_slot)."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    ep = np.empty(n_experts + 1, dtype=np.int32)
    tp = np.empty(n_experts + 1, dtype=np.int32)
    st = np.empty(T * k, dtype=np.int32)
    ss = np.empty(T * k, dtype=np.int32)
    lib().orc_group(_ptr(idx), T, k, int(n_experts), int(bm), _ptr(ep), _ptr(tp), _ptr(st), _ptr(ss))
    return ep, tp, st, ss


# --------------------------------------------------------------- layers ----

def make_desc(w, max_batch, max_seq, n_layers=None) -> Desc:
    """Descriptor from a ``synth.workloads.Workload``-like object."""
    return Desc(dtype=BF16 if w.dtype == "bf16" else F32,
                n_layers=w.n_layers if n_layers is None else n_layers, hidden=w.hidden,
                n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn_dim=w.ffn_dim,
                n_experts=w.n_experts, top_k=w.top_k, expert_ffn_dim=w.expert_ffn_dim,
                max_batch=max_batch, max_seq=max_seq, rms_eps=w.rms_eps, rope_theta=w.rope_theta)


def _layer_struct(layer: dict):
    """Build the ctypes layer struct; returns (struct, keepalive list)."""
    keep = []
    vals = {}
    for n in _LAYER_FIELDS:
        a = layer.get(n)
        if a is None:
            vals[n] = None
            continue
        if n in ("attn_norm", "ffn_norm"):
            a = _c(a, np.float32)
        else:
            a, _ = _storage(a)
        keep.append(a)
        vals[n] = a.ctypes.data
    return Layer(**vals), keep


def decode_layer(desc: Desc, layer: dict, kv_layer, seq_lens, hidden, given_append: bool = False):
    """One dense layer. kv_layer [2][max_batch][Hkv][max_seq][d] is updated in
    place (K/V appended); returns the new hidden [batch][H] (float64). With
    given_append, each request's new K/V entry is read from slot seq_len as it
    stands in kv_layer (another implementation's append) instead of written."""
    s, keep = _layer_struct(layer)
    h = np.array(hidden, dtype=np.float64, copy=True)
    sl = _c(seq_lens, np.int32)
    assert kv_layer.flags["C_CONTIGUOUS"]
    fn = lib().orc_decode_layer_given_append if given_append else lib().orc_decode_layer
    rc = fn(ctypes.byref(desc), ctypes.byref(s), _ptr(kv_layer), _ptr(sl), h.shape[0], _ptr(h))
    if rc:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return h


def decode_stack(desc: Desc, layers: list, kv, seq_lens, hidden, given_append: bool = False):
    """The full stack; kv [L][2][max_batch][Hkv][max_seq][d] updated in place
    (with given_append: read, see decode_layer)."""
    h = np.array(hidden, dtype=np.float64, copy=True)
    for l, layer in enumerate(layers):
        h = decode_layer(desc, layer, kv[l], seq_lens, h, given_append)
    return h


def moe_layer(desc: Desc, layer: dict, kv_layer, seq_lens, hidden, bm):
    """One MoE layer over T tokens. Returns (hidden', routing dict)."""
    s, keep = _layer_struct(layer)
    h = np.array(hidden, dtype=np.float64, copy=True)
    T = h.shape[0]
    E, k = desc.n_experts, desc.top_k
    sl = _c(seq_lens, np.int32)
    r = {"router_logits": np.empty((T, E), np.float32), "topk_idx": np.empty((T, k), np.int32),
         "topk_w": np.empty((T, k), np.float64), "exp_indptr": np.empty(E + 1, np.int32),
         "tile_indptr": np.empty(E + 1, np.int32), "sorted_tok": np.empty(T * k, np.int32),
         "sorted_slot": np.empty(T * k, np.int32)}
    rc = lib().orc_moe_layer(ctypes.byref(desc), ctypes.byref(s), _ptr(kv_layer), _ptr(sl), T, int(bm), _ptr(h),
                             _ptr(r["router_logits"]), _ptr(r["topk_idx"]), _ptr(r["topk_w"]),
                             _ptr(r["exp_indptr"]), _ptr(r["tile_indptr"]), _ptr(r["sorted_tok"]),
                             _ptr(r["sorted_slot"]))
    if rc:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return h, r


def moe_layer_routed(desc: Desc, layer: dict, kv_layer, seq_lens, hidden, topk_idx):
    """One MoE layer with each token's experts given (``topk_idx`` [T][k]):
    gates are the softmax over the layer's own float32 logits at those experts.
    Returns (hidden', gates [T][k])."""
    s, keep = _layer_struct(layer)
    h = np.array(hidden, dtype=np.float64, copy=True)
    T = h.shape[0]
    idx = _c(topk_idx, np.int32)
    assert idx.shape == (T, desc.top_k)
    sl = _c(seq_lens, np.int32)
    w = np.empty((T, desc.top_k), np.float64)
    rc = lib().orc_moe_layer_routed(ctypes.byref(desc), ctypes.byref(s), _ptr(kv_layer), _ptr(sl), T, _ptr(idx),
                                    _ptr(h), _ptr(w))
    if rc:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return h, w
