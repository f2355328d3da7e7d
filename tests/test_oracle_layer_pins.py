"""Pins for the oracle's whole-layer functions (dense decode layer, stack, MoE
layer). The pages print no worked example, so the layer is pinned through
hand-built weights whose output has a closed form, and the MoE layer through
special cases that reduce it to the dense layer and to the pinned top-k.
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest
import scipy.special as sps


def tiny(**kw):
    base = dict(dtype="f32", n_layers=1, hidden=8, n_q_heads=2, n_kv_heads=1, head_dim=4, ffn_dim=8,
                n_experts=0, top_k=0, expert_ffn_dim=0, rms_eps=1e-5, rope_theta=10000.0)
    base.update(kw)
    return SimpleNamespace(**base)


def rnd_layer(rng, w, moe=False):
    H, d = w.hidden, w.head_dim
    L = {"attn_norm": (1 + 0.1 * rng.standard_normal(H)).astype(np.float32),
         "ffn_norm": (1 + 0.1 * rng.standard_normal(H)).astype(np.float32),
         "w_qkv": (0.3 * rng.standard_normal(((w.n_q_heads + 2 * w.n_kv_heads) * d, H))).astype(np.float32),
         "w_o": (0.3 * rng.standard_normal((H, w.n_q_heads * d))).astype(np.float32)}
    if moe:
        E, Fe = w.n_experts, w.expert_ffn_dim
        L["w_router"] = (0.5 * rng.standard_normal((E, H))).astype(np.float32)
        L["w_exp_gate"] = (0.3 * rng.standard_normal((E, Fe, H))).astype(np.float32)
        L["w_exp_up"] = (0.3 * rng.standard_normal((E, Fe, H))).astype(np.float32)
        L["w_exp_down"] = (0.3 * rng.standard_normal((E, H, Fe))).astype(np.float32)
    else:
        F = w.ffn_dim
        L["w_gate"] = (0.3 * rng.standard_normal((F, H))).astype(np.float32)
        L["w_up"] = (0.3 * rng.standard_normal((F, H))).astype(np.float32)
        L["w_down"] = (0.3 * rng.standard_normal((H, F))).astype(np.float32)
    return L


def rnd_kv(rng, w, B, S):
    return rng.standard_normal((2, B, w.n_kv_heads, S, w.head_dim)).astype(np.float32)


def rms(x, g, eps):
    return x / math.sqrt(np.mean(x * x) + eps) * g.astype(np.float64)


def test_zero_output_projections_give_identity_layer(orc):
    rng = np.random.default_rng(20)
    w = tiny()
    L = rnd_layer(rng, w)
    L["w_o"][:] = 0
    L["w_down"][:] = 0
    kv = rnd_kv(rng, w, 2, 6)
    x = rng.standard_normal((2, 8))
    out = orc.decode_layer(orc.make_desc(w, 2, 6), L, kv, [3, 0], x)
    np.testing.assert_array_equal(out, x)


def test_wiring_closed_form_empty_cache(orc):
    """seq_len 0: the new token attends only to itself, so o_h = v for both
    heads (one KV head). v picks u[0:4] and is stored in the cache dtype
    (float32) before attention reads it; W_o = I; W_gate = c I, W_up = I,
    W_down = I. Then h1 = x + [v, v] with v = f32(u[0:4]), u = RMSNorm(x; g1),
    and x' = h1 + silu(c u2) * u2 with u2 = RMSNorm(h1; g2)."""
    rng = np.random.default_rng(21)
    w = tiny()
    c = 1.75
    g1 = (1 + 0.2 * rng.standard_normal(8)).astype(np.float32)
    g2 = (1 + 0.2 * rng.standard_normal(8)).astype(np.float32)
    Wqkv = (0.3 * rng.standard_normal((16, 8))).astype(np.float32)
    Wqkv[12:16] = 0
    Wqkv[12:16, 0:4] = np.eye(4)
    L = {"attn_norm": g1, "ffn_norm": g2, "w_qkv": Wqkv, "w_o": np.eye(8, dtype=np.float32),
         "w_gate": (c * np.eye(8)).astype(np.float32), "w_up": np.eye(8, dtype=np.float32),
         "w_down": np.eye(8, dtype=np.float32)}
    kv = np.zeros((2, 1, 1, 4, 4), np.float32)
    x = rng.standard_normal((1, 8))
    out = orc.decode_layer(orc.make_desc(w, 1, 4), L, kv, [0], x)
    u = rms(x[0], g1, 1e-5)
    v = u[:4].astype(np.float32).astype(np.float64)
    h1 = x[0] + np.concatenate([v, v])
    u2 = rms(h1, g2, 1e-5)
    expect = h1 + (c * u2) * sps.expit(c * u2) * u2
    np.testing.assert_allclose(out[0], expect, rtol=1e-12)
    # the appended entries: k at position 0 is unrotated, v = u[0:4]
    np.testing.assert_allclose(kv[0, 0, 0, 0], (Wqkv[8:12].astype(np.float64) @ u).astype(np.float32), rtol=1e-6)
    np.testing.assert_allclose(kv[1, 0, 0, 0], u[:4].astype(np.float32), rtol=1e-6)


def test_appended_key_rotated_at_seq_len(orc):
    """d = 2: the key written at slot S is k turned by the angle S."""
    rng = np.random.default_rng(22)
    w = tiny(hidden=4, n_q_heads=2, n_kv_heads=1, head_dim=2, ffn_dim=4)
    L = rnd_layer(rng, w)
    S = 5
    kv = rnd_kv(rng, w, 1, 8)
    x = rng.standard_normal((1, 4))
    orc.decode_layer(orc.make_desc(w, 1, 8), L, kv, [S], x)
    u = rms(x[0], L["attn_norm"], 1e-5)
    k = L["w_qkv"][4:6].astype(np.float64) @ u
    rot = np.array([k[0] * math.cos(S) - k[1] * math.sin(S), k[1] * math.cos(S) + k[0] * math.sin(S)])
    np.testing.assert_allclose(kv[0, 0, 0, S], rot.astype(np.float32), rtol=1e-6)


def test_query_rotated_at_seq_len(orc):
    """The query is rotated at position S: with d = 2, cached keys R(S)k (and
    one R(0)k) and W_o selecting o, the layer's attention output equals the
    closed form softmax(<R(S)q, key_j> / sqrt(2)) . V, so a query rotated at any
    other position (or not at all) fails."""
    rng = np.random.default_rng(23)
    w = tiny(hidden=4, n_q_heads=1, n_kv_heads=1, head_dim=2, ffn_dim=4)
    L = rnd_layer(rng, w)
    L["w_o"] = np.eye(4, 2, dtype=np.float32)        # h1 = x + [o, 0, 0]
    L["w_down"][:] = 0
    S = 3
    x = rng.standard_normal((1, 4))
    u = rms(x[0], L["attn_norm"], 1e-5)
    q, k = L["w_qkv"][0:2].astype(np.float64) @ u, L["w_qkv"][2:4].astype(np.float64) @ u

    def R(a, z):
        return np.array([z[0] * math.cos(a) - z[1] * math.sin(a), z[1] * math.cos(a) + z[0] * math.sin(a)])

    kv = np.zeros((2, 1, 1, 8, 2), np.float32)
    kv[0, 0, 0, :S] = R(S, k)
    kv[1, 0, 0, :S] = rng.standard_normal((S, 2))
    kv[0, 0, 0, 0] = R(0, k)
    out = orc.decode_layer(orc.make_desc(w, 1, 8), L, kv, [S], x)
    keys = kv[0, 0, 0, :S + 1].astype(np.float64)
    s = keys @ R(S, q) / math.sqrt(2)
    p = sps.softmax(s)
    o = p @ kv[1, 0, 0, :S + 1].astype(np.float64)
    np.testing.assert_allclose(out[0, :2] - x[0, :2], o, rtol=1e-5)
    assert s[0] != pytest.approx(s[1])


def test_appended_value_not_rotated_at_seq_len(orc):
    """d = 2, S = 5: RoPE turns q and k only. The value written at slot S is
    the plain projection W_v u, and attention reads that entry: with W_q = 0
    every score is 0, so o is the mean of the S + 1 values, and W_o selecting
    o gives h1 = x + [o, 0, 0]. A value rotated by the angle S (in the cache or
    only inside attention) fails both checks."""
    rng = np.random.default_rng(27)
    w = tiny(hidden=4, n_q_heads=1, n_kv_heads=1, head_dim=2, ffn_dim=4)
    L = rnd_layer(rng, w)
    L["w_qkv"][0:2] = 0                              # q = 0: uniform attention weights
    L["w_o"] = np.eye(4, 2, dtype=np.float32)        # h1 = x + [o, 0, 0]
    L["w_down"][:] = 0
    S = 5
    kv = rnd_kv(rng, w, 1, 8)
    cached_v = kv[1, 0, 0, :S].astype(np.float64).copy()
    x = rng.standard_normal((1, 4))
    out = orc.decode_layer(orc.make_desc(w, 1, 8), L, kv, [S], x)
    u = rms(x[0], L["attn_norm"], 1e-5)
    v = L["w_qkv"][4:6].astype(np.float64) @ u
    v_rot = np.array([v[0] * math.cos(S) - v[1] * math.sin(S), v[1] * math.cos(S) + v[0] * math.sin(S)])
    assert np.abs(v_rot - v).max() > 1e-2            # the mistake would be visible
    np.testing.assert_allclose(kv[1, 0, 0, S], v.astype(np.float32), rtol=1e-6)
    expect = (cached_v.sum(axis=0) + v.astype(np.float32).astype(np.float64)) / (S + 1)
    np.testing.assert_allclose(out[0, :2] - x[0, :2], expect, rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(out[0, 2:], x[0, 2:])


def _bf16_bits(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_val(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("S", [0, 3])
def test_attention_reads_appended_entry_rounded_to_cache_dtype(orc, S):
    """bfloat16 cache: the new K/V entry is stored rounded to bfloat16, and
    attention reads the stored (rounded) entry, not the unrounded projection.
    W_q = 0 makes every score 0, so o = mean of the S + 1 stored values; with
    S = 0 it is the rounded new value alone. W_o selects o and W_down = 0, so
    x' - x = [o, 0, 0]. The expected o is built from the entry rounded by hand
    (round_bf16, pinned separately); attending over the unrounded v misses it
    by far more than the tolerance."""
    rng = np.random.default_rng(28 + S)
    w = tiny(dtype="bf16", hidden=4, n_q_heads=1, n_kv_heads=1, head_dim=2, ffn_dim=4)
    L = rnd_layer(rng, w)
    L["w_qkv"][0:2] = 0
    L["w_o"] = np.eye(4, 2, dtype=np.float32)
    L["w_down"][:] = 0
    Lb = {n: (a if n.endswith("norm") else _bf16_bits(a)) for n, a in L.items()}
    kvb = _bf16_bits(rnd_kv(rng, w, 1, 8))
    cached_v = _bf16_val(kvb[1, 0, 0, :S]).copy()
    x = rng.standard_normal((1, 4))
    out = orc.decode_layer(orc.make_desc(w, 1, 8), Lb, kvb, [S], x)
    u = rms(x[0], L["attn_norm"], 1e-5)
    v = _bf16_val(Lb["w_qkv"][4:6]) @ u
    v_rnd = np.array([orc.round_bf16(t) for t in v])
    assert np.abs(v_rnd - v).max() > 1e-5            # rounding moves v by far more than the tolerance below
    np.testing.assert_array_equal(_bf16_val(kvb[1, 0, 0, S]), v_rnd)
    expect = (cached_v.sum(axis=0) + v_rnd) / (S + 1)
    np.testing.assert_allclose(out[0, :2] - x[0, :2], expect, rtol=1e-12, atol=1e-14)


def test_batch_requests_are_independent(orc):
    rng = np.random.default_rng(24)
    w = tiny()
    L = rnd_layer(rng, w)
    kv = rnd_kv(rng, w, 3, 10)
    x = rng.standard_normal((3, 8))
    sl = [4, 9, 0]
    kv_all = kv.copy()
    out = orc.decode_layer(orc.make_desc(w, 3, 10), L, kv_all, sl, x)
    for b in range(3):
        kvb = np.ascontiguousarray(kv[:, b:b + 1])
        ob = orc.decode_layer(orc.make_desc(w, 1, 10), L, kvb, [sl[b]], x[b:b + 1])
        np.testing.assert_array_equal(ob[0], out[b])
        np.testing.assert_array_equal(kvb[:, 0], kv_all[:, b])


def test_stack_is_composition_of_layers(orc):
    rng = np.random.default_rng(25)
    w = tiny(n_layers=3)
    layers = [rnd_layer(rng, w) for _ in range(3)]
    kv = rng.standard_normal((3, 2, 2, 1, 7, 4)).astype(np.float32)
    x = rng.standard_normal((2, 8))
    sl = [2, 5]
    d = orc.make_desc(w, 2, 7)
    kv2 = kv.copy()
    out = orc.decode_stack(d, layers, kv, sl, x)
    h = x
    for l in range(3):
        h = orc.decode_layer(d, layers[l], kv2[l], sl, h)
    np.testing.assert_array_equal(out, h)


def test_rejects_bad_seq_len(orc):
    rng = np.random.default_rng(26)
    w = tiny()
    L = rnd_layer(rng, w)
    kv = rnd_kv(rng, w, 1, 4)
    with pytest.raises(ValueError):
        orc.decode_layer(orc.make_desc(w, 1, 4), L, kv, [4], np.zeros((1, 8)))


# ---------------------------------------------------------------------- MoE --

def moe_cfg(E, k, Fe=6):
    return tiny(n_experts=E, top_k=k, expert_ffn_dim=Fe, ffn_dim=0)


def dense_from_expert(L, e):
    D = {n: L[n] for n in ("attn_norm", "ffn_norm", "w_qkv", "w_o")}
    D["w_gate"], D["w_up"], D["w_down"] = L["w_exp_gate"][e], L["w_exp_up"][e], L["w_exp_down"][e]
    return D


def test_moe_single_expert_equals_dense(orc):
    rng = np.random.default_rng(30)
    w = moe_cfg(1, 1)
    L = rnd_layer(rng, w, moe=True)
    kv = rnd_kv(rng, w, 2, 6)
    x = rng.standard_normal((2, 8))
    kv2 = kv.copy()
    out, r = orc.moe_layer(orc.make_desc(w, 2, 6), L, kv, [2, 4], x, bm=4)
    dw = tiny(ffn_dim=6)
    ref = orc.decode_layer(orc.make_desc(dw, 2, 6), dense_from_expert(L, 0), kv2, [2, 4], x)
    np.testing.assert_allclose(out, ref, rtol=1e-14)
    np.testing.assert_array_equal(kv, kv2)
    np.testing.assert_array_equal(r["topk_idx"], [[0], [0]])
    np.testing.assert_array_equal(r["topk_w"], [[1.0], [1.0]])


@pytest.mark.parametrize("E,k", [(8, 2), (6, 6), (16, 3)])
def test_moe_equals_gate_weighted_dense_layers(orc, E, k):
    """Brute force: run every expert as a dense layer on every token and mix the
    outputs with the sparse gate vector; since the gates sum to 1 the residual
    passes through unchanged. With k = E the gates are the full softmax."""
    rng = np.random.default_rng(31 + E + k)
    w = moe_cfg(E, k)
    L = rnd_layer(rng, w, moe=True)
    T = 5
    kv = rnd_kv(rng, w, T, 9)
    x = rng.standard_normal((T, 8))
    sl = [0, 3, 8, 1, 5]
    out, r = orc.moe_layer(orc.make_desc(w, T, 9), L, kv.copy(), sl, x, bm=2)
    dw = tiny(ffn_dim=6)
    dense = [orc.decode_layer(orc.make_desc(dw, T, 9), dense_from_expert(L, e), kv.copy(), sl, x) for e in range(E)]
    for t in range(T):
        z = r["router_logits"][t].astype(np.float64)
        gates = np.zeros(E)
        gates[r["topk_idx"][t]] = r["topk_w"][t]
        if k == E:
            np.testing.assert_allclose(gates, sps.softmax(z), rtol=1e-12)
        ref = sum(gates[e] * dense[e][t] for e in range(E))
        np.testing.assert_allclose(out[t], ref, rtol=1e-11, atol=1e-12)
        order = np.lexsort((np.arange(E), -z))
        np.testing.assert_array_equal(r["topk_idx"][t], order[:k])


def test_moe_router_logits_are_rounded_projection(orc):
    rng = np.random.default_rng(32)
    w = moe_cfg(8, 2)
    L = rnd_layer(rng, w, moe=True)
    kv = rnd_kv(rng, w, 1, 4)
    x = rng.standard_normal((1, 8))
    kv2 = kv.copy()
    _, r = orc.moe_layer(orc.make_desc(w, 1, 4), L, kv, [1], x, bm=1)
    # h1 from the dense path with a zero FFN
    D = dense_from_expert(L, 0)
    D["w_down"] = np.zeros_like(D["w_down"])
    h1 = orc.decode_layer(orc.make_desc(tiny(ffn_dim=6), 1, 4), D, kv2, [1], x)[0]
    u2 = rms(h1, L["ffn_norm"], 1e-5)
    np.testing.assert_array_equal(r["router_logits"][0], (L["w_router"].astype(np.float64) @ u2).astype(np.float32))


def test_moe_forced_tie_routes_to_lowest_experts(orc):
    rng = np.random.default_rng(33)
    w = moe_cfg(16, 4)
    L = rnd_layer(rng, w, moe=True)
    L["w_router"][:] = 0
    T = 3
    kv = rnd_kv(rng, w, T, 4)
    _, r = orc.moe_layer(orc.make_desc(w, T, 4), L, kv, [0, 1, 2], rng.standard_normal((T, 8)), bm=2)
    np.testing.assert_array_equal(r["topk_idx"], np.tile(np.arange(4), (T, 1)))
    np.testing.assert_allclose(r["topk_w"], 0.25)
    np.testing.assert_array_equal(r["exp_indptr"], [0, 3, 6, 9, 12] + [12] * 12)
    np.testing.assert_array_equal(r["tile_indptr"], [0, 2, 4, 6, 8] + [8] * 12)
    np.testing.assert_array_equal(r["sorted_tok"], [0, 1, 2] * 4)
    np.testing.assert_array_equal(r["sorted_slot"], np.repeat(np.arange(4), 3))


def test_bf16_storage_consistent_with_f32_storage(orc):
    """Same bf16-representable weights and cache stored as bfloat16 and as
    float32: the layers differ only through the rounding of the appended K/V
    entry, so they agree closely but not exactly."""
    import torch
    rng = np.random.default_rng(34)
    w32 = tiny(hidden=16, n_q_heads=4, n_kv_heads=2, head_dim=4, ffn_dim=24)
    L = rnd_layer(rng, w32)

    def tobf(a):
        return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    def fromb(b):
        return (b.astype(np.uint32) << 16).view(np.float32)

    Lb = {n: (a if n.endswith("norm") else tobf(a)) for n, a in L.items()}
    Lf = {n: (a if n.endswith("norm") else fromb(Lb[n])) for n, a in L.items()}
    kv = rnd_kv(rng, w32, 2, 12)
    kvb = tobf(kv)
    kvf = fromb(kvb).copy()
    x = rng.standard_normal((2, 16))
    wb = tiny(dtype="bf16", hidden=16, n_q_heads=4, n_kv_heads=2, head_dim=4, ffn_dim=24)
    ob = orc.decode_layer(orc.make_desc(wb, 2, 12), Lb, kvb, [5, 11], x)
    of = orc.decode_layer(orc.make_desc(w32, 2, 12), Lf, kvf, [5, 11], x)
    assert np.linalg.norm(ob - of) / np.linalg.norm(of) < 1e-2
    assert not np.array_equal(ob, of)
    # the appended entries are the float32 ones rounded to bfloat16
    for b, s in ((0, 5), (1, 11)):
        np.testing.assert_array_equal(kvb[:, b, :, s], tobf(kvf[:, b, :, s]))


def test_moe_routed_with_own_topk_equals_moe_layer(orc):
    """The layer with each token's experts given: handed the layer's own
    top-k, it reproduces the routed layer exactly (outputs and gates)."""
    rng = np.random.default_rng(35)
    w = moe_cfg(8, 3)
    L = rnd_layer(rng, w, moe=True)
    T = 4
    kv = rnd_kv(rng, w, T, 7)
    x = rng.standard_normal((T, 8))
    sl = [0, 2, 6, 3]
    out, r = orc.moe_layer(orc.make_desc(w, T, 7), L, kv.copy(), sl, x, bm=2)
    out2, g2 = orc.moe_layer_routed(orc.make_desc(w, T, 7), L, kv.copy(), sl, x, r["topk_idx"])
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(g2, r["topk_w"])


def test_moe_routed_other_selection_is_gate_weighted_mixture(orc):
    """Any given selection: the output is h1 plus the dense SwiGLU of each
    given expert weighted by the softmax of the layer's logits over the
    selection (brute force through the dense layer); a selection in another
    order gives the same gates, permuted, and the same output up to the
    order of the sum."""
    rng = np.random.default_rng(36)
    E, k = 8, 3
    w = moe_cfg(E, k)
    L = rnd_layer(rng, w, moe=True)
    T = 3
    kv = rnd_kv(rng, w, T, 6)
    x = rng.standard_normal((T, 8))
    sl = [1, 4, 0]
    _, r = orc.moe_layer(orc.make_desc(w, T, 6), L, kv.copy(), sl, x, bm=1)
    sel = np.array([[7, 0, 3], [2, 5, 1], [6, 4, 0]], np.int32)
    out, g = orc.moe_layer_routed(orc.make_desc(w, T, 6), L, kv.copy(), sl, x, sel)
    dw = tiny(ffn_dim=6)
    dense = [orc.decode_layer(orc.make_desc(dw, T, 6), dense_from_expert(L, e), kv.copy(), sl, x) for e in range(E)]
    for t in range(T):
        zs = r["router_logits"][t, sel[t]].astype(np.float64)
        np.testing.assert_allclose(g[t], sps.softmax(zs), rtol=1e-13)
        ref = sum(g[t, j] * dense[sel[t, j]][t] for j in range(k))
        np.testing.assert_allclose(out[t], ref, rtol=1e-11, atol=1e-12)
    out_p, g_p = orc.moe_layer_routed(orc.make_desc(w, T, 6), L, kv.copy(), sl, x, sel[:, ::-1].copy())
    np.testing.assert_allclose(g_p, g[:, ::-1], rtol=1e-13)
    np.testing.assert_allclose(out_p, out, rtol=1e-12, atol=1e-13)


def test_given_append_with_own_entries_equals_layer(orc):
    """The layer that reads the new K/V entry from the cache as given: handed
    a cache whose slot seq_len already holds the layer's own appended entries,
    it reproduces the layer exactly (bf16 cache) and leaves the cache alone."""
    rng = np.random.default_rng(37)
    w = tiny(dtype="bf16", hidden=16, n_q_heads=4, n_kv_heads=2, head_dim=4, ffn_dim=24)
    L = {n: (a if n.endswith("norm") else _bf16_bits(a)) for n, a in rnd_layer(rng, w).items()}
    kv = _bf16_bits(rnd_kv(rng, w, 3, 9))
    x = rng.standard_normal((3, 16))
    sl = [0, 4, 8]
    kv_own = kv.copy()
    out = orc.decode_layer(orc.make_desc(w, 3, 9), L, kv_own, sl, x)
    kv_given = kv_own.copy()
    out2 = orc.decode_layer(orc.make_desc(w, 3, 9), L, kv_given, sl, x, given_append=True)
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(kv_given, kv_own)


def test_given_append_reads_the_slot_as_stored(orc):
    """d = 2, W_q = 0 (uniform attention), W_o selecting o, W_down = 0: with
    an arbitrary entry planted at slot S the output is x + [mean of the S + 1
    stored values, 0, 0], the planted value included; the layer that appends
    overwrites the plant with its own entry instead."""
    rng = np.random.default_rng(38)
    w = tiny(hidden=4, n_q_heads=1, n_kv_heads=1, head_dim=2, ffn_dim=4)
    L = rnd_layer(rng, w)
    L["w_qkv"][0:2] = 0
    L["w_o"] = np.eye(4, 2, dtype=np.float32)
    L["w_down"][:] = 0
    S = 4
    kv = rnd_kv(rng, w, 1, 8)
    kv[1, 0, 0, S] = [7.5, -3.25]
    x = rng.standard_normal((1, 4))
    expect = kv[1, 0, 0, :S + 1].astype(np.float64).mean(axis=0)
    out = orc.decode_layer(orc.make_desc(w, 1, 8), L, kv.copy(), [S], x, given_append=True)
    np.testing.assert_allclose(out[0, :2] - x[0, :2], expect, rtol=1e-12)
    own = orc.decode_layer(orc.make_desc(w, 1, 8), L, kv.copy(), [S], x)
    assert np.abs(own[0, :2] - out[0, :2]).max() > 0.1
