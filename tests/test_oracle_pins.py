"""Pins for the CPU oracle: each oracle function checked against something
other than itself -- closed forms, invariants, library routines (numpy, scipy,
torch's bfloat16 conversion) and brute force on tiny inputs. The cases are
chosen so that a plausible mistake (a dropped term, a wrong sign or index, a
transposed operand, a wrong pairing or scale) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch


def bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------ bf16 rounding --

def test_round_bf16_ties_to_even(orc):
    assert orc.round_bf16(1.0) == 1.0
    assert orc.round_bf16(1 + 2 ** -8) == 1.0                      # halfway, even neighbour is 1.0
    assert orc.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6          # halfway, even neighbour is up
    assert orc.round_bf16(-(1 + 2 ** -8)) == -1.0
    assert orc.round_bf16(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7    # just above halfway rounds up
    assert orc.round_bf16(0.0) == 0.0


def test_round_bf16_matches_torch_on_float32_values(orc):
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.standard_normal(2000), rng.standard_normal(200) * 1e-38,
                           rng.standard_normal(200) * 1e30]).astype(np.float32)
    ref = bf16_to_f64(bf16_bits(vals))
    got = np.array([orc.round_bf16(float(v)) for v in vals])
    np.testing.assert_array_equal(got, ref)


# ------------------------------------------------------------------ RMSNorm --

def test_rmsnorm_constant_vector_closed_form(orc):
    g = np.array([0.5, -2.0, 1.0, 3.0], np.float32)
    for c in (3.0, -0.01, 1e-3):
        out = orc.rmsnorm(np.full(4, c), g, 1e-5)
        np.testing.assert_allclose(out, g.astype(np.float64) * c / math.sqrt(c * c + 1e-5), rtol=1e-14)


def test_rmsnorm_eps_inside_root_and_mean_not_sum(orc):
    x = np.array([1e-3, -1e-3, 1e-3, -1e-3, 1e-3, -1e-3])          # mean square 1e-6
    out = orc.rmsnorm(x, np.ones(6, np.float32), 1e-6)
    np.testing.assert_allclose(out, x / math.sqrt(2e-6), rtol=1e-14)


def test_rmsnorm_unit_rms_before_gain(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(257) * 3.0
    g = (rng.standard_normal(257) + 2).astype(np.float32)
    out = orc.rmsnorm(x, g, 1e-5)
    m = np.mean(x * x)
    np.testing.assert_allclose(np.sqrt(np.mean((out / g.astype(np.float64)) ** 2)), math.sqrt(m / (m + 1e-5)), rtol=1e-13)
    assert np.all(orc.rmsnorm(np.zeros(5), np.ones(5, np.float32), 1e-5) == 0)


# ----------------------------------------------------------------- matvec --

def test_matvec_matches_numpy_f32_and_bf16_rectangular(orc):
    rng = np.random.default_rng(3)
    W = rng.standard_normal((7, 13)).astype(np.float32)
    x = rng.standard_normal(13)
    np.testing.assert_allclose(orc.matvec(W, x), W.astype(np.float64) @ x, rtol=1e-13, atol=1e-13)
    Wb = bf16_bits(W)
    np.testing.assert_allclose(orc.matvec(Wb, x), bf16_to_f64(Wb).reshape(7, 13) @ x, rtol=1e-13, atol=1e-13)


def test_matvec_basis_vectors_pick_columns(orc):
    W = np.arange(12, dtype=np.float32).reshape(3, 4)
    for i in range(4):
        e = np.zeros(4)
        e[i] = 1.0
        np.testing.assert_array_equal(orc.matvec(W, e), W[:, i])


# -------------------------------------------------------------------- RoPE --

def test_rope_single_pair_closed_form(orc):
    for p in (0, 1, 7, 1000):
        np.testing.assert_allclose(orc.rope([1.0, 0.0], p, 10000.0), [math.cos(p), math.sin(p)], atol=1e-12)
        np.testing.assert_allclose(orc.rope([0.0, 1.0], p, 10000.0), [-math.sin(p), math.cos(p)], atol=1e-12)


def test_rope_rotate_half_pairing_and_frequencies(orc):
    p, theta = 3, 100.0
    # d=4: pairs (0,2) at angle p, (1,3) at angle p * theta^(-2/4) = p/10
    out = orc.rope([1.0, 0.0, 0.0, 0.0], p, theta)
    np.testing.assert_allclose(out, [math.cos(p), 0, math.sin(p), 0], atol=1e-12)
    out = orc.rope([0.0, 1.0, 0.0, 0.0], p, theta)
    np.testing.assert_allclose(out, [0, math.cos(p / 10), 0, math.sin(p / 10)], atol=1e-12)


def test_rope_invariants(orc):
    rng = np.random.default_rng(4)
    d, theta = 16, 10000.0
    z = rng.standard_normal(d)
    np.testing.assert_allclose(orc.rope(z, 0, theta), z, atol=0)
    r = orc.rope(z, 37, theta)
    h = d // 2
    np.testing.assert_allclose(r[:h] ** 2 + r[h:] ** 2, z[:h] ** 2 + z[h:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(orc.rope(orc.rope(z, 11, theta), 26, theta), r, atol=1e-12)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    m, n = 50, 13
    np.testing.assert_allclose(orc.rope(q, m, theta) @ orc.rope(k, n, theta), orc.rope(q, m - n, theta) @ k, rtol=1e-10)


# ------------------------------------------------------------------- SiLU --

def test_silu(orc):
    assert orc.silu(0.0) == 0.0
    for z in (-5.0, -0.3, 0.7, 4.0):
        assert orc.silu(z) == pytest.approx(z * sps.expit(z), rel=1e-14)
        assert orc.silu(z) - orc.silu(-z) == pytest.approx(z, rel=1e-13)


# -------------------------------------------------------------- attention --

def _kv(rng, Hkv, S, d, n):
    K = np.zeros((Hkv, S, d), np.float32)
    V = np.zeros((Hkv, S, d), np.float32)
    K[:, :n] = rng.standard_normal((Hkv, n, d))
    V[:, :n] = rng.standard_normal((Hkv, n, d))
    return K, V


def test_attention_single_entry_returns_v(orc):
    rng = np.random.default_rng(5)
    K, V = _kv(rng, 2, 8, 4, 1)
    q = rng.standard_normal((4, 4))
    o = orc.attention(q, K, V, 1)
    np.testing.assert_allclose(o, V[[0, 0, 1, 1], 0], atol=1e-15)   # heads 0,1 -> kv 0; heads 2,3 -> kv 1


def test_attention_two_keys_closed_form_scale(orc):
    d, a = 16, 2.5
    K = np.zeros((1, 4, d), np.float32)
    V = np.zeros((1, 4, d), np.float32)
    K[0, 0, 0] = 1.0
    V[0, 0, :] = 3.0
    V[0, 1, :] = -1.0
    q = np.zeros((1, d))
    q[0, 0] = a
    p0 = sps.expit(a / math.sqrt(d))
    np.testing.assert_allclose(orc.attention(q, K, V, 2)[0], np.full(d, 3 * p0 - (1 - p0)), rtol=1e-13)


def test_attention_equal_keys_mean_and_permutation(orc):
    rng = np.random.default_rng(6)
    Hkv, S, d, n = 1, 12, 8, 9
    K, V = _kv(rng, Hkv, S, d, n)
    q = rng.standard_normal((3, d))
    Keq = K.copy()
    Keq[:, :n] = K[:, :1]
    np.testing.assert_allclose(orc.attention(q, Keq, V, n), np.repeat(V[:, :n].astype(np.float64).mean(1), 3, 0), rtol=1e-12)
    perm = rng.permutation(n)
    K2, V2 = K.copy(), V.copy()
    K2[:, :n] = K[:, perm]
    V2[:, :n] = V[:, perm]
    np.testing.assert_allclose(orc.attention(q, K2, V2, n), orc.attention(q, K, V, n), rtol=1e-12)


def test_attention_gqa_equals_mha_with_duplicated_kv(orc):
    rng = np.random.default_rng(7)
    Hq, Hkv, S, d, n = 8, 2, 10, 8, 7
    K, V = _kv(rng, Hkv, S, d, n)
    q = rng.standard_normal((Hq, d))
    Kd = np.repeat(K, Hq // Hkv, axis=0)
    Vd = np.repeat(V, Hq // Hkv, axis=0)
    np.testing.assert_allclose(orc.attention(q, K, V, n), orc.attention(q, Kd, Vd, n), rtol=1e-13)


def test_attention_softmax_library_reference(orc):
    rng = np.random.default_rng(8)
    Hq, Hkv, S, d, n = 4, 2, 9, 8, 9
    K, V = _kv(rng, Hkv, S, d, n)
    q = rng.standard_normal((Hq, d)) * 3
    o = orc.attention(q, K, V, n)
    for h in range(Hq):
        g = h // 2
        p = sps.softmax(K[g, :n].astype(np.float64) @ q[h] / math.sqrt(d))
        np.testing.assert_allclose(p.sum(), 1.0)
        np.testing.assert_allclose(o[h], p @ V[g, :n], rtol=1e-12)


def test_attention_bf16_cache(orc):
    rng = np.random.default_rng(9)
    K, V = _kv(rng, 1, 6, 8, 5)
    q = rng.standard_normal((2, 8))
    Kb, Vb = bf16_bits(K), bf16_bits(V)
    ref = orc.attention(q, bf16_to_f64(Kb).reshape(K.shape).astype(np.float32),
                        bf16_to_f64(Vb).reshape(V.shape).astype(np.float32), 5)
    np.testing.assert_allclose(orc.attention(q, Kb, Vb, 5), ref, rtol=1e-14)


# ------------------------------------------------------------------- TopK --

def test_topk_matches_stable_full_sort(orc):
    rng = np.random.default_rng(10)
    for _ in range(50):
        E, k = 32, 6
        z = np.round(rng.standard_normal(E) * 2, 1).astype(np.float32)   # rounding creates ties
        idx, w = orc.topk(z, k)
        order = np.lexsort((np.arange(E), -z.astype(np.float64)))
        np.testing.assert_array_equal(idx, order[:k])
        np.testing.assert_allclose(w, sps.softmax(z[idx].astype(np.float64)), rtol=1e-13)
        full = sps.softmax(z.astype(np.float64))
        np.testing.assert_allclose(w, full[idx] / full[idx].sum(), rtol=1e-12)
        assert w.sum() == pytest.approx(1.0, abs=1e-15)


def test_topk_ties_go_to_lower_index(orc):
    idx, w = orc.topk(np.zeros(128, np.float32), 8)
    np.testing.assert_array_equal(idx, np.arange(8))
    np.testing.assert_allclose(w, np.full(8, 1 / 8))
    idx, _ = orc.topk(np.array([1, 3, 3, 2, 3], np.float32), 2)
    np.testing.assert_array_equal(idx, [1, 2])


# --------------------------------------------------------------- grouping --

@pytest.mark.parametrize("T,k,E,bm", [(1, 8, 128, 16), (5, 2, 8, 2), (64, 8, 128, 16), (3, 3, 3, 1)])
def test_group_against_library_sort(orc, T, k, E, bm):
    rng = np.random.default_rng(T * 100 + k)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ep, tp, st, ss = orc.group(idx, E, bm)
    counts = np.bincount(idx.ravel(), minlength=E)
    np.testing.assert_array_equal(ep, np.concatenate([[0], np.cumsum(counts)]))
    assert ep[-1] == T * k and np.all(np.diff(ep) >= 0)
    np.testing.assert_array_equal(tp, np.concatenate([[0], np.cumsum(-(-counts // bm))]))
    tok = np.repeat(np.arange(T), k)
    slot = np.tile(np.arange(k), T)
    order = np.lexsort((tok, idx.ravel()))          # by expert, then token
    np.testing.assert_array_equal(st, tok[order])
    np.testing.assert_array_equal(ss, slot[order])
    pairs = set(zip(st.tolist(), ss.tolist()))
    assert len(pairs) == T * k
