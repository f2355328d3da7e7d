"""GPU parity of decode_step against the CPU oracle (through the C ABI).

Each case prints its name, shape and seed tag before touching the GPU, so a
failure can be traced from whatever output survives.
"""
import numpy as np
import pytest
import torch

import synth
from _cases import build_case, make_model, oracle_inputs, rel_l2, run_oracle_dense, to_np

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[case] {msg}", flush=True)


def check_dense(orc, case, tol, requests=None, kv_tol=None, sched=None):
    inp = oracle_inputs(case, requests)
    model = make_model(case)
    if sched is not None:
        model.set_schedule(sched)
    announce(f"decode_step {case.w.name} L={case.n_layers} B={case.hidden.shape[0]} "
             f"lens={to_np(case.seq_lens).tolist()[:8]} schedule={sched or 'fused'}")
    model.step(case.hidden, case.kv, case.seq_lens)
    torch.cuda.synchronize()
    assert model.device_error() == 0
    ref, kv_ref = run_oracle_dense(orc, case, inp)
    got = to_np(case.hidden).astype(np.float64)[inp["requests"]]
    err = rel_l2(got, ref)
    print(f"  rel_l2(hidden) = {err:.3e} (tol {tol})", flush=True)
    assert err <= tol
    # the appended K/V entries of every layer, compared in float
    kv_gpu = case.kv[:, :, inp["requests"]] if requests is not None else case.kv
    sl = inp["seq_lens"]
    for i, s in enumerate(sl):
        a = kv_gpu[:, :, i, :, int(s)].float().cpu().numpy()
        ref_bits = kv_ref[:, :, i, :, int(s)]
        b = (ref_bits.astype(np.uint32) << 16).view(np.float32) if ref_bits.dtype == np.uint16 else ref_bits
        e = rel_l2(a, b)
        assert e <= (kv_tol if kv_tol is not None else tol), f"appended K/V of request {i}: {e}"
    model.close()
    return err


def test_c1_tiny_f32(orc):
    w = synth.get_workload("c1_tiny_f32")
    case = build_case(w, 1, [128], tag="t1")
    check_dense(orc, case, w.tol)


def test_c1_shapes_ragged_batch_multichunk(orc):
    """Tiny fp32 layer, batch 3 with ragged lengths spanning several 128-entry
    attention chunks and the empty-cache case."""
    w = synth.get_workload("c1_tiny_f32")
    case = build_case(w, 3, [0, 127, 300], max_seq=512, tag="t2")
    check_dense(orc, case, w.tol)


def test_c1_shapes_two_layers_random_gains(orc):
    w = synth.get_workload("c1_tiny_f32")
    case = build_case(w, 2, [5, 257], n_layers=2, max_seq=300, tag="t3", random_gains=True)
    check_dense(orc, case, w.tol)


def test_8b_shape_two_layers_b1(orc):
    w = synth.get_workload("c2_8b_b1")
    case = build_case(w, 1, [512], n_layers=2, max_seq=640, tag="t4")
    check_dense(orc, case, w.tol)


def test_8b_shape_ragged_b4(orc):
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(4, 512, 8192, ("c3_8b_sweep", "lens", 4))
    case = build_case(w, 4, lens, n_layers=2, max_seq=8193, tag="t5")
    check_dense(orc, case, w.tol)


def test_shape_changes_reuse_handle(orc):
    """One handle, three calls with different batch sizes and lengths: the
    queues and event counts are rebuilt on the device each call."""
    w = synth.get_workload("c1_tiny_f32")
    base = build_case(w, 4, [10, 20, 30, 40], max_seq=400, max_batch=4, tag="t6")
    model = make_model(base)
    for B, lens in ((1, [130]), (4, [3, 260, 99, 384]), (2, [0, 1])):
        hidden = synth.make_hidden(w, B, B, device="cuda", tag="t6")
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        case = base.__class__(w, 1, base.layers, base.kv, hidden, sl, 4, 400)
        inp = oracle_inputs(case, list(range(B)))
        # oracle on the first B request slots of the cache
        inp["kv"] = np.ascontiguousarray(to_np(base.kv[:, :, :B]))
        announce(f"reuse handle B={B} lens={lens}")
        model.step(hidden, base.kv, sl)
        torch.cuda.synchronize()
        assert model.device_error() == 0
        ref, _ = run_oracle_dense(orc, case, inp)
        assert rel_l2(to_np(hidden), ref) <= w.tol
    model.close()


def test_bad_length_is_reported_and_step_skipped():
    w = synth.get_workload("c1_tiny_f32")
    case = build_case(w, 2, [3, 4], max_seq=64, tag="t7")
    model = make_model(case)
    before = case.hidden.clone()
    bad = torch.tensor([3, 64], dtype=torch.int32, device="cuda")
    announce("bad seq_len")
    assert model.decode_step(case.hidden, case.kv, bad) == 0     # launched; the device rejects it
    torch.cuda.synchronize()
    assert model.device_error() == 5                                # PMK_ERR_SEQ
    assert torch.equal(case.hidden, before)
    assert model.device_error() == 0                                # cleared by the read
    assert model.decode_step(case.hidden, case.kv, case.seq_lens[:0]) == 1   # batch 0: PMK_ERR_ARG
    model.close()


def test_watchdog_abandons_step_then_handle_recovers(orc):
    """A 1 us event-wait limit, forced from the host, makes the step's first
    long wait expire: the step is abandoned with PMK_ERR_TIMEOUT and every
    workgroup leaves it (the kernel returns). With the limit restored and the
    inputs put back, the same handle runs a step that matches the oracle."""
    from persistent_megakernel_04_amd import _abi
    w = synth.get_workload("c2_8b_b1")
    case = build_case(w, 1, [512], n_layers=2, max_seq=600, tag="t21")
    hidden0, kv0 = case.hidden.clone(), case.kv.clone()
    model = make_model(case)
    model.set_watchdog_us(1)
    announce("decode_step with a 1 us watchdog")
    model.step(case.hidden, case.kv, case.seq_lens)
    torch.cuda.synchronize()
    assert model.device_error() == _abi.PMK_ERR_TIMEOUT
    assert model.device_error() == 0   # reading the error word cleared it
    model.set_watchdog_us(0)
    case.hidden.copy_(hidden0)
    case.kv.copy_(kv0)
    inp = oracle_inputs(case)
    announce("decode_step after recovery")
    model.step(case.hidden, case.kv, case.seq_lens)
    torch.cuda.synchronize()
    assert model.device_error() == 0
    ref, _ = run_oracle_dense(orc, case, inp)
    err = rel_l2(to_np(case.hidden).astype(np.float64), ref)
    print(f"  rel_l2(hidden) after recovery = {err:.3e}", flush=True)
    assert err <= w.tol
    model.close()


def test_consecutive_steps_chain(orc):
    """Three decode steps in a row on one handle: each step's output and K/V
    append feed the next (lengths advance by one), against the oracle chained
    the same way."""
    w = synth.get_workload("c2_8b_b1")
    case = build_case(w, 2, [40, 200], n_layers=2, max_seq=260, tag="t8")
    inp = oracle_inputs(case)
    model = make_model(case)
    desc = orc.make_desc(w, 2, 260, n_layers=2)
    kv_ref, h_ref = inp["kv"], inp["hidden"]
    lens = np.array([40, 200], np.int32)
    for step in range(3):
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        announce(f"chained step {step} lens={lens.tolist()}")
        model.step(case.hidden, case.kv, sl)
        torch.cuda.synchronize()
        assert model.device_error() == 0
        h_ref = orc.decode_stack(desc, inp["layers"], kv_ref, lens, h_ref)
        err = rel_l2(to_np(case.hidden), h_ref)
        print(f"  step {step}: rel_l2 = {err:.3e}", flush=True)
        assert err <= w.tol
        lens = lens + 1
    model.close()


def test_8b_full_stack_b1_bench_config(orc):
    """The benchmark's workload: the full 32-layer 8B-shaped stack, batch 1,
    512 cached positions, one step, every output element against the oracle."""
    w = synth.get_workload("c2_8b_b1")
    case = build_case(w, 1, [512], max_seq=613, tag="")
    check_dense(orc, case, w.tol)


def test_8b_full_stack_b16_ragged_sampled(orc):
    """Batch 16 with ragged lengths in [512, 8192] over the full 32-layer stack;
    the oracle recomputes two sampled requests (requests are independent)."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(16, 512, 8192, ("c3_8b_sweep", "lens", 16))
    case = build_case(w, 16, lens, max_seq=int(lens.max()) + 2, tag="t9")
    check_dense(orc, case, w.tol, requests=[int(np.argmax(lens)), int(np.argmin(lens))])


def test_70b_shape_four_layers_b8_sampled(orc):
    """Llama-70B-shaped layers (H 8192, 64/8 heads, FFN 28672), batch 8 with
    lengths in [8192, 16384]; four layers, two sampled requests."""
    w = synth.get_workload("c5_70b")
    lens = synth.ragged_lengths(8, 8192, 16384, ("c5_70b", "lens", 8))
    case = build_case(w, 8, lens, n_layers=4, max_seq=int(lens.max()) + 2, tag="t10")
    check_dense(orc, case, w.tol, requests=[0, 5])


def test_70b_shape_b12_split_records_beyond_lds(orc):
    """A 70B-shaped layer at batch 12: gate/up runs in 4 K slices whose partial
    records (896 rows x 12 per tile) are too large to pull into LDS, so the last
    slice task of each tile adds them through register loads instead. One
    layer, lengths in [256, 1024], every request against the oracle."""
    w = synth.get_workload("c5_70b")
    lens = synth.ragged_lengths(12, 256, 1024, ("c5_70b", "lens", 12))
    case = build_case(w, 12, lens, n_layers=1, max_seq=int(lens.max()) + 2, tag="t16")
    check_dense(orc, case, w.tol)


@pytest.mark.parametrize("B", [64, 128])
def test_8b_shape_large_batch_sampled(orc, B):
    """The batch sweep's two largest points: passes of 16 rows over every
    projection, attention in equal shares of the laid-out positions; two
    layers, lengths in [512, 8192], three sampled requests."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(B, 512, 8192, ("c3_8b_sweep", "lens", B))
    case = build_case(w, B, lens, n_layers=2, max_seq=int(lens.max()) + 2, tag=f"t14_{B}")
    check_dense(orc, case, w.tol, requests=[int(np.argmax(lens)), int(np.argmin(lens)), B - 1])


def test_8b_shape_b1_256_position_chunks(orc):
    """Batch 1 with 1500 cached positions: 6 attention chunks of 256 positions
    (the longest chunk the O-projection merge takes), each on a workgroup of
    its own."""
    w = synth.get_workload("c2_8b_b1")
    case = build_case(w, 1, [1500], n_layers=2, max_seq=1600, tag="t20")
    check_dense(orc, case, w.tol)


def test_8b_shape_last_cache_slot_and_empty(orc):
    """The append goes to the cache's last slot (length max_seq - 1) for one
    request, next to an empty cache and a one-entry cache; every request
    against the oracle."""
    w = synth.get_workload("c3_8b_sweep")
    case = build_case(w, 3, [699, 0, 1], n_layers=1, max_seq=700, tag="t18")
    check_dense(orc, case, w.tol)


def test_8b_shape_largest_batch_short_caches(orc):
    """The largest batch a handle takes (1024 requests: 64 blocks of 16 rows per
    projection), lengths in [0, 24] in a 25-slot cache, so several requests
    start empty and several append into the last slot; one layer, four
    sampled requests."""
    w = synth.get_workload("c3_8b_sweep")
    B = 1024
    lens = synth.ragged_lengths(B, 0, 24, ("c3_8b_sweep", "lens_max_batch", B))
    case = build_case(w, B, lens, n_layers=1, max_seq=25, tag="t19")
    full = int(np.flatnonzero(lens == 24)[0])
    check_dense(orc, case, w.tol, requests=[int(np.argmin(lens)), full, B // 2, B - 1])


@pytest.mark.parametrize("B", [256, 512])
def test_8b_shape_batch_beyond_128_sampled(orc, B):
    """Decode batches beyond the sweep's largest point (16 to 32 blocks of 16
    rows per projection, thousands of attention pieces per layer), with short
    contexts in [16, 512] so that the cache stays small; two layers, three
    sampled requests."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(B, 16, 512, ("c3_8b_sweep", "lens_short", B))
    case = build_case(w, B, lens, n_layers=2, max_seq=int(lens.max()) + 2, tag=f"t17_{B}")
    check_dense(orc, case, w.tol, requests=[int(np.argmax(lens)), int(np.argmin(lens)), B - 1])


@pytest.mark.parametrize("B", [8, 12, 16])
def test_8b_shape_split_k_every_request(orc, B):
    """Batches whose staged inputs outgrow the LDS: the projections run as K
    slices whose partial sums the last slice task of each row tile adds (down
    in 4 to 7 slices, the 4096-deep projections in 2 at batch 12 and 16).
    Two layers, every request and every output element against the oracle."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(B, 512, 2048, ("c3_8b_sweep", "split_k", B))
    case = build_case(w, B, lens, n_layers=2, max_seq=int(lens.max()) + 2, tag=f"t11_{B}")
    check_dense(orc, case, w.tol)


F32_MID = synth.Workload(name="f32_mid", dtype="f32", n_layers=2, hidden=1024, n_q_heads=8, n_kv_heads=2,
                         head_dim=64, ffn_dim=4096, tol=1e-5)


def test_f32_split_k_batch16(orc):
    """float32 weights at batch 16: the 4096-deep down projection's inputs
    (256 KiB staged) take two K slices; the result stays at float32 accuracy."""
    lens = synth.ragged_lengths(16, 1, 300, ("f32_mid", "lens"))
    case = build_case(F32_MID, 16, lens, max_seq=302, tag="t12")
    check_dense(orc, case, F32_MID.tol)


@pytest.mark.parametrize("sched", ["layer", "stage", "barrier"])
@pytest.mark.parametrize("B", [1, 4])
def test_unfused_schedules_match_oracle(orc, sched, B):
    """The ablation schedules (one launch of the persistent kernel per layer or
    per stage of each layer, or one launch with a grid-wide barrier after every
    stage) run the same tasks: the same results, at batch 1 (attention on
    workgroups of its own, partials merged by the O-projection) and batch 4
    (streamed attention, down projection split over K)."""
    w = synth.get_workload("c3_8b_sweep")
    lens = [512] if B == 1 else synth.ragged_lengths(B, 512, 2048, ("c3_8b_sweep", "sched", B))
    case = build_case(w, B, lens, n_layers=2, max_seq=int(max(lens)) + 2, tag=f"t13_{sched}_{B}")
    check_dense(orc, case, w.tol, sched=sched)


def test_schedule_setters_reject_unknown_modes(orc):
    """pmk_set_schedule / pmk_set_moe_scheduler on a live handle: unknown
    modes are rejected and leave the handle working (fused step still matches)."""
    from persistent_megakernel_04_amd import _abi
    w = synth.get_workload("c1_tiny_f32")
    case = build_case(w, 1, [40], max_seq=64, tag="t15")
    model = make_model(case)
    assert model.lib.pmk_set_schedule(model.handle, 9) == _abi.PMK_ERR_ARG
    assert model.lib.pmk_set_schedule(model.handle, -1) == _abi.PMK_ERR_ARG
    assert model.lib.pmk_set_moe_scheduler(model.handle, 2) == _abi.PMK_ERR_ARG
    model.close()
    check_dense(orc, case, w.tol)
