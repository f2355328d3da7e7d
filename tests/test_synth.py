"""The seeded input generator: deterministic, key-separated, right moments."""
import numpy as np
import torch

import synth


def test_same_key_same_values_and_keys_differ():
    a = synth.normal((64, 32), 0.02, ("t", "w", 0))
    b = synth.normal((64, 32), 0.02, ("t", "w", 0))
    c = synth.normal((64, 32), 0.02, ("t", "w", 1))
    assert torch.equal(a, b)
    assert not torch.equal(a, c)


def test_moments_and_bf16_is_rne_of_f32():
    x = synth.normal((512, 512), 0.02, ("t", "m"))
    assert abs(float(x.mean())) < 1e-3
    assert abs(float(x.std()) - 0.02) < 5e-4
    xb = synth.normal((512, 512), 0.02, ("t", "m"), dtype=torch.bfloat16)
    assert torch.equal(xb, x.to(torch.bfloat16))


def test_fill_normal_slabs_deterministic():
    t1 = torch.empty(10, 7, 3)
    t2 = torch.empty(10, 7, 3)
    synth.fill_normal_(t1, 1.0, ("t", "kv"), slab_elems=50)
    synth.fill_normal_(t2, 1.0, ("t", "kv"), slab_elems=50)
    assert torch.equal(t1, t2)
    assert float(t1.std()) > 0.5


def test_ragged_lengths_closed_range():
    r = synth.ragged_lengths(10000, 512, 8192, ("t", "len"))
    assert r.min() >= 512 and r.max() <= 8192
    assert r.min() < 600 and r.max() > 8100
    assert np.array_equal(r, synth.ragged_lengths(10000, 512, 8192, ("t", "len")))


def test_workload_param_counts():
    w = synth.get_workload("c2_8b_b1")
    assert w.layer_params() == 218_103_808
    w5 = synth.get_workload("c5_70b")
    assert w5.layer_params() == 855_638_016
