"""GPU parity of decode_step against the CPU oracle (through the C ABI).

Each case prints its name, shape and seed tag before touching the GPU, so a
failure can be traced from whatever output survives. Outputs are compared per
element (check_rows): the relative L2 bound the workloads state over the whole
output and over every row, and every element within a tight multiple of its
row's RMS. Up to 16 requests, every request is recomputed by the oracle; above
that, one request in every 16-row block (the unit the kernels split a batch
into) plus the longest and the shortest.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from _cases import (BF16_ULP_REL, ELEM_TOL_OWN, block_requests, build_case, check_rows, make_model, oracle_inputs,
                    run_oracle_dense, to_np)

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[case] {msg}", flush=True)


def progress(msg):
    """A progress line that bypasses pytest's capture (long cases)."""
    print(f"[progress] {msg}", file=sys.__stderr__, flush=True)


def kv_as_float(a):
    a = np.asarray(a)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if a.dtype == np.uint16 else a


def check_appended(w, kv_gpu, kv_ref, lens, what="appended K/V"):
    """The K/V entries each request appended at its slot seq_len, in every
    layer: rows (request, layer, K or V) of Hkv d values. kv_gpu / kv_ref are
    [L][2][B][Hkv][max_seq][d] host arrays over the compared requests."""
    got, ref = [], []
    for i, s in enumerate(lens):
        got.append(kv_as_float(kv_gpu[:, :, i, :, int(s)]).reshape(-1, kv_gpu.shape[3] * kv_gpu.shape[5]))
        ref.append(kv_as_float(kv_ref[:, :, i, :, int(s)]).reshape(-1, kv_ref.shape[3] * kv_ref.shape[5]))
    ulp = BF16_ULP_REL if w.dtype == "bf16" else 0.0
    # against the oracle's own chain: in a deep stack the entries of later
    # layers also carry the drift of earlier layers' rounding decisions
    check_rows(np.concatenate(got), np.concatenate(ref), w, what, ulp_rel=ulp, elem_tol=ELEM_TOL_OWN[w.dtype])


def check_against_oracle(orc, case, inp, got, kv_gpu, what="hidden"):
    """`got` (the GPU's outputs over inp's requests) against the oracle with
    its own appended K/V entries (rel-L2 per row and overall within the
    workload's bound, elements within ELEM_TOL_OWN), the GPU's appended
    entries against the oracle's (one bfloat16 ulp at most per element), and
    `got` against the oracle fed the GPU's appended entries (elements within
    ELEM_TOL). kv_gpu: host copy of the GPU's cache after the step over the
    same requests."""
    w = case.w
    ref, kv_ref = run_oracle_dense(orc, case, inp)
    err = check_rows(got, ref, w, what + " vs oracle", elem_tol=ELEM_TOL_OWN[w.dtype])
    check_appended(w, kv_gpu, kv_ref, inp["seq_lens"])
    ref_g, _ = run_oracle_dense(orc, case, inp, kv_given=kv_gpu)
    check_rows(got, ref_g, w, what + " vs oracle on the GPU's appended entries")
    return err


def check_dense(orc, case, requests="auto", sched=None):
    """One step on a fresh handle, against the oracle on `requests` (default:
    all up to 16 requests, else one per 16-row block)."""
    B = case.hidden.shape[0]
    lens = to_np(case.seq_lens)
    if isinstance(requests, str):
        requests = None if B <= 16 else block_requests(lens)
    inp = oracle_inputs(case, requests)
    model = make_model(case)
    if sched is not None:
        model.set_schedule(sched)
    announce(f"decode_step {case.w.name} L={case.n_layers} B={B} lens={lens.tolist()[:8]} "
             f"schedule={sched or 'fused'} oracle requests={len(inp['requests'])}")
    model.step(case.hidden, case.kv, case.seq_lens)
    torch.cuda.synchronize()
    assert model.device_error() == 0
    model.close()
    got = to_np(case.hidden).astype(np.float64)[inp["requests"]]
    kv_gpu = to_np(case.kv[:, :, inp["requests"]] if requests is not None else case.kv)
    return check_against_oracle(orc, case, inp, got, kv_gpu)


def test_c1_tiny_f32(orc):
    w = synth.get_workload("c1_tiny_f32")
    case = build_case(w, 1, [128], tag="t1")
    check_dense(orc, case)


def test_c1_shapes_ragged_batch_multichunk(orc):
    """Tiny fp32 layer, batch 3 with ragged lengths spanning several 128-entry
    attention chunks and the empty-cache case."""
    w = synth.get_workload("c1_tiny_f32")
    case = build_case(w, 3, [0, 127, 300], max_seq=512, tag="t2")
    check_dense(orc, case)


def test_c1_shapes_two_layers_random_gains(orc):
    w = synth.get_workload("c1_tiny_f32")
    case = build_case(w, 2, [5, 257], n_layers=2, max_seq=300, tag="t3", random_gains=True)
    check_dense(orc, case)


@pytest.mark.parametrize("events", ["group", "stage"])
def test_more_than_64_kv_heads(orc, events):
    """72 KV heads (fp32, one query head each): an O-projection tile reads the
    attention of all 72 groups, so its wait spans 72 flat counters (per stage:
    attention waits on the QKV counters of all 72 groups too), more than the 64
    lanes of the waiting wave read at once."""
    import dataclasses
    w = dataclasses.replace(synth.get_workload("c1_tiny_f32"), name="c1_wide_kv", n_q_heads=72, n_kv_heads=72)
    case = build_case(w, 2, [40, 130], max_seq=160, tag="t21")
    inp = oracle_inputs(case)
    model = make_model(case)
    model.set_event_granularity(events)
    announce(f"decode_step {w.name} Hkv=72 B=2 events={events}")
    model.step(case.hidden, case.kv, case.seq_lens)
    torch.cuda.synchronize()
    assert model.device_error() == 0
    model.close()
    check_against_oracle(orc, case, inp, to_np(case.hidden).astype(np.float64), to_np(case.kv))


def test_8b_shape_two_layers_b1(orc):
    w = synth.get_workload("c2_8b_b1")
    case = build_case(w, 1, [512], n_layers=2, max_seq=640, tag="t4")
    check_dense(orc, case)


def test_8b_shape_ragged_b4(orc):
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(4, 512, 8192, ("c3_8b_sweep", "lens", 4))
    case = build_case(w, 4, lens, n_layers=2, max_seq=8193, tag="t5")
    check_dense(orc, case)


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
        check_rows(to_np(hidden), ref, w)
    model.close()


def test_bad_length_is_reported_and_step_skipped():
    """A length at max_seq: the prologue rejects the step (nothing is written),
    and the error reaches the host mirror, so the next call returns it without
    launching, until pmk_get_device_error has read and cleared it."""
    from persistent_megakernel_04_amd import _abi
    w = synth.get_workload("c1_tiny_f32")
    case = build_case(w, 2, [3, 4], max_seq=64, tag="t7")
    model = make_model(case)
    before = case.hidden.clone()
    bad = torch.tensor([3, 64], dtype=torch.int32, device="cuda")
    announce("bad seq_len")
    assert model.decode_step(case.hidden, case.kv, bad) == 0     # launched; the device rejects it
    torch.cuda.synchronize()
    assert torch.equal(case.hidden, before)
    # the step has finished: the next call sees the pending error and launches nothing
    assert model.decode_step(case.hidden, case.kv, case.seq_lens) == _abi.PMK_ERR_SEQ
    torch.cuda.synchronize()
    assert torch.equal(case.hidden, before)
    assert model.device_error() == _abi.PMK_ERR_SEQ
    assert model.device_error() == 0                                # cleared by the read
    assert model.decode_step(case.hidden, case.kv, case.seq_lens[:0]) == _abi.PMK_ERR_ARG   # batch 0
    # cleared: the handle runs again
    assert model.decode_step(case.hidden, case.kv, case.seq_lens) == 0
    torch.cuda.synchronize()
    assert model.device_error() == 0
    assert not torch.equal(case.hidden, before)
    model.close()


def test_watchdog_abandons_step_then_handle_recovers(orc):
    """A 1 us event-wait limit, forced from the host, makes the step's first
    long wait expire: the step is abandoned with PMK_ERR_TIMEOUT and every
    workgroup leaves it (the kernel returns); the next call returns the error
    from the host mirror. With the limit restored, the error read and the
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
    assert model.decode_step(case.hidden, case.kv, case.seq_lens) == _abi.PMK_ERR_TIMEOUT
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
    check_against_oracle(orc, case, inp, to_np(case.hidden), to_np(case.kv), "hidden after recovery")
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
    outs = []
    for step in range(3):
        sl = torch.tensor(lens + step, dtype=torch.int32, device="cuda")
        announce(f"chained step {step} lens={(lens + step).tolist()}")
        model.step(case.hidden, case.kv, sl)
        torch.cuda.synchronize()
        assert model.device_error() == 0
        outs.append(to_np(case.hidden).astype(np.float64))
    model.close()
    kv_gpu = to_np(case.kv)
    h_given = inp["hidden"]
    for step in range(3):
        # the oracle chained on its own appends, and on the GPU's (the cache
        # after the last step holds every step's entry; step i reads slots up
        # to lens + i only)
        h_ref = orc.decode_stack(desc, inp["layers"], kv_ref, lens + step, h_ref)
        check_rows(outs[step], h_ref, w, f"hidden at step {step} vs oracle", elem_tol=ELEM_TOL_OWN[w.dtype])
        h_given = orc.decode_stack(desc, inp["layers"], kv_gpu.copy(), lens + step, h_given, given_append=True)
        check_rows(outs[step], h_given, w, f"hidden at step {step} vs oracle on the GPU's appended entries")
    for b, s0 in enumerate(lens):   # rows (layer, K/V, Hkv, slot) of d values
        check_rows(kv_as_float(kv_gpu[:, :, b, :, s0:s0 + 3]).reshape(-1, w.head_dim),
                   kv_as_float(kv_ref[:, :, b, :, s0:s0 + 3]).reshape(-1, w.head_dim), w,
                   f"appended K/V of request {b}", ulp_rel=BF16_ULP_REL, elem_tol=ELEM_TOL_OWN[w.dtype])


def test_8b_full_stack_b1_bench_config(orc):
    """The benchmark's workload: the full 32-layer 8B-shaped stack, batch 1,
    512 cached positions, one step, every output element against the oracle."""
    w = synth.get_workload("c2_8b_b1")
    case = build_case(w, 1, [512], max_seq=613, tag="")
    check_dense(orc, case)


def test_c2_8b_full_stack_100_step_chain(orc):
    """The 8B-shaped workload as configured: the 32-layer stack at batch 1 with
    512 cached positions, then 100 decode steps on one handle, a fresh N(0, 1)
    input row per step and the cache growing 512 -> 611. Every step's output
    against the oracle chained the same way, then every appended K/V entry
    (100 positions x 32 layers)."""
    w = synth.get_workload("c2_8b_b1")
    n_steps, S0 = 100, 512
    case = build_case(w, 1, [S0], max_seq=S0 + n_steps + 1, tag="")
    inp = oracle_inputs(case)
    model = make_model(case)
    hid = [synth.make_hidden(w, 1, i, device="cuda", tag="chain") for i in range(n_steps)]
    ins = [h.cpu().numpy().astype(np.float64) for h in hid]
    lens = torch.arange(S0, S0 + n_steps, dtype=torch.int32, device="cuda").reshape(n_steps, 1)
    announce(f"decode_step {w.name} L=32 B=1 chain of {n_steps} steps from {S0} cached positions")
    for i in range(n_steps):
        model.step(hid[i], case.kv, lens[i])
    torch.cuda.synchronize()
    assert model.device_error() == 0
    model.close()
    outs = [to_np(h).astype(np.float64) for h in hid]
    desc = orc.make_desc(w, 1, case.max_seq)
    kv_ref = inp["kv"]
    kv_gpu = to_np(case.kv)
    worst = 0.0
    for i in range(n_steps):
        sl = np.array([S0 + i], np.int32)
        ref = orc.decode_stack(desc, inp["layers"], kv_ref, sl, ins[i])
        worst = max(worst, check_rows(outs[i], ref, w, f"hidden at step {i} vs oracle", elem_tol=ELEM_TOL_OWN[w.dtype]))
        # the GPU's cache after the last step holds every step's entry; step i reads slots up to S0 + i only
        ref_g = orc.decode_stack(desc, inp["layers"], kv_gpu.copy(), sl, ins[i], given_append=True)
        check_rows(outs[i], ref_g, w, f"hidden at step {i} vs oracle on the GPU's appended entries")
        if i % 10 == 9:
            progress(f"c2 chain: oracle at step {i + 1}/{n_steps}, worst rel_l2 so far {worst:.3e}")
    got = kv_as_float(kv_gpu[:, :, 0, :, S0:S0 + n_steps]).transpose(0, 1, 3, 2, 4).reshape(-1, w.n_kv_heads * 128)
    ref = kv_as_float(kv_ref[:, :, 0, :, S0:S0 + n_steps]).transpose(0, 1, 3, 2, 4).reshape(-1, w.n_kv_heads * 128)
    check_rows(got, ref, w, "appended K/V of all 100 steps", ulp_rel=BF16_ULP_REL, elem_tol=ELEM_TOL_OWN[w.dtype])


def test_8b_full_stack_b16_ragged_every_request(orc):
    """Batch 16 with ragged lengths in [512, 8192] over the full 32-layer
    stack; the oracle recomputes every request."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(16, 512, 8192, ("c3_8b_sweep", "lens", 16))
    case = build_case(w, 16, lens, max_seq=int(lens.max()) + 2, tag="t9")
    check_dense(orc, case)


def test_70b_shape_four_layers_b8(orc):
    """Llama-70B-shaped layers (H 8192, 64/8 heads, FFN 28672), batch 8 with
    lengths in [8192, 16384]; four layers, every request."""
    w = synth.get_workload("c5_70b")
    lens = synth.ragged_lengths(8, 8192, 16384, ("c5_70b", "lens", 8))
    case = build_case(w, 8, lens, n_layers=4, max_seq=int(lens.max()) + 2, tag="t10")
    check_dense(orc, case)


def stream_oracle_stack(orc, w, case, lens, hidden_in, n_layers, label):
    """The oracle over a stack too large to copy at once: layer by layer, each
    layer's weights and cache block copied to the host after the GPU step.
    Slots 0..S-1 of the cache are untouched by the step; slot S holds the GPU's
    appended entry. Each layer runs twice: reading the GPU's entry (the chain
    on the GPU's appended entries), then appending its own over it (the
    oracle's own chain). Returns (hidden, hidden on the GPU's entries, GPU
    appended entries [L][B][2][Hkv][d], oracle appended entries)."""
    desc = orc.make_desc(w, len(lens), case.max_seq, n_layers=1)
    h = h_g = hidden_in
    app_gpu, app_ref = [], []
    idx = np.arange(len(lens))
    for l in range(n_layers):
        layer = {k: to_np(v) for k, v in case.layers[l].items()}
        kv_l = np.ascontiguousarray(to_np(case.kv[l]))
        app_gpu.append(kv_l[:, idx, :, lens].copy())
        h_g = orc.decode_layer(desc, layer, kv_l, lens, h_g, given_append=True)
        h = orc.decode_layer(desc, layer, kv_l, lens, h)
        app_ref.append(kv_l[:, idx, :, lens].copy())
        del layer, kv_l
        if l % 10 == 9:
            progress(f"{label}: oracle at layer {l + 1}/{n_layers}")
    return h, h_g, np.stack(app_gpu), np.stack(app_ref)


def check_streamed(orc, w, B, lo, hi, key, tag):
    """A whole stack at its configured depth and batch, every request."""
    lens = synth.ragged_lengths(B, lo, hi, key)
    max_seq = int(lens.max()) + 2
    announce(f"decode_step {w.name} L={w.n_layers} B={B} lens={lens.tolist()} (weights generated on the device)")
    case = build_case(w, B, lens, max_seq=max_seq, tag=tag)
    progress(f"{w.name}: {w.n_layers} layers generated")
    hidden0 = to_np(case.hidden).astype(np.float64)
    model = make_model(case)
    model.step(case.hidden, case.kv, case.seq_lens)
    torch.cuda.synchronize()
    assert model.device_error() == 0
    model.close()
    got = to_np(case.hidden).astype(np.float64)
    ref, ref_g, app_gpu, app_ref = stream_oracle_stack(orc, w, case, lens, hidden0, w.n_layers, w.name)
    check_rows(got, ref, w, "hidden vs oracle", elem_tol=ELEM_TOL_OWN[w.dtype])
    check_rows(got, ref_g, w, "hidden vs oracle on the GPU's appended entries")
    d = w.head_dim
    # rows (layer, request, K/V) of Hkv d values; app arrays are [L][B][2][Hkv][d]
    check_rows(kv_as_float(app_gpu).reshape(-1, w.n_kv_heads * d), kv_as_float(app_ref).reshape(-1, w.n_kv_heads * d),
               w, "appended K/V", ulp_rel=BF16_ULP_REL, elem_tol=ELEM_TOL_OWN[w.dtype])


def test_c5_70b_full_80_layers_b8(orc):
    """The 70B-shaped workload as configured: 80 layers (137 GB of bfloat16
    weights on the device), batch 8 with lengths uniform on [8192, 16384], one
    step; every request against the oracle streamed layer by layer."""
    check_streamed(orc, synth.get_workload("c5_70b"), 8, 8192, 16384, ("c5_70b", "lens", 8), "")


def test_tp8_share_of_70b_full_80_layers_b8(orc):
    """One GPU's share of the 70B shape under 8-way tensor parallelism (8 query
    heads and 1 KV head, FFN 3584 = 28672 / 8, all 80 layers) at its real
    shape, batch 8 with lengths in [8192, 16384], every request. The share's
    all-reduces are not part of a one-GPU step."""
    check_streamed(orc, synth.get_workload("c5_tp8_share"), 8, 8192, 16384, ("c5_tp8_share", "lens", 8), "")


def test_70b_shape_b12_split_records_beyond_lds(orc):
    """A 70B-shaped layer at batch 12: gate/up runs in 4 K slices whose partial
    records (896 rows x 12 per tile) are too large to pull into LDS, so the last
    slice task of each tile adds them through register loads instead. One
    layer, lengths in [256, 1024], every request against the oracle."""
    w = synth.get_workload("c5_70b")
    lens = synth.ragged_lengths(12, 256, 1024, ("c5_70b", "lens", 12))
    case = build_case(w, 12, lens, n_layers=1, max_seq=int(lens.max()) + 2, tag="t16")
    check_dense(orc, case)


@pytest.mark.parametrize("B", [64, 128])
def test_8b_shape_large_batch_every_block(orc, B):
    """The batch sweep's two largest points: 16-row blocks over every
    projection, attention in equal shares of the laid-out positions; two
    layers, lengths in [512, 8192], one request of every 16-row block."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(B, 512, 8192, ("c3_8b_sweep", "lens", B))
    case = build_case(w, B, lens, n_layers=2, max_seq=int(lens.max()) + 2, tag=f"t14_{B}")
    check_dense(orc, case)


def test_8b_shape_b1_256_position_chunks(orc):
    """Batch 1 with 1500 cached positions: 6 attention chunks of 256 positions
    (the longest chunk the O-projection merge takes), each on a workgroup of
    its own."""
    w = synth.get_workload("c2_8b_b1")
    case = build_case(w, 1, [1500], n_layers=2, max_seq=1600, tag="t20")
    check_dense(orc, case)


def test_8b_shape_last_cache_slot_and_empty(orc):
    """The append goes to the cache's last slot (length max_seq - 1) for one
    request, next to an empty cache and a one-entry cache; every request
    against the oracle."""
    w = synth.get_workload("c3_8b_sweep")
    case = build_case(w, 3, [699, 0, 1], n_layers=1, max_seq=700, tag="t18")
    check_dense(orc, case)


def test_8b_shape_largest_batch_short_caches(orc):
    """The largest batch a handle takes (1024 requests: 64 blocks of 16 rows per
    projection), lengths in [0, 24] in a 25-slot cache, so several requests
    start empty and several append into the last slot; one layer, one request
    of every block plus an empty and a full cache."""
    w = synth.get_workload("c3_8b_sweep")
    B = 1024
    lens = synth.ragged_lengths(B, 0, 24, ("c3_8b_sweep", "lens_max_batch", B))
    case = build_case(w, B, lens, n_layers=1, max_seq=25, tag="t19")
    full = int(np.flatnonzero(lens == 24)[0])
    check_dense(orc, case, requests=sorted(set(block_requests(lens)) | {full}))


@pytest.mark.parametrize("B", [17, 33])
def test_8b_shape_odd_block_counts(orc, B):
    """Batches just past one and two 16-row blocks (the last block holding a
    single request): the blocked split sizes its row tiles for the block count
    (two and three blocks); one layer, every request compared."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(B, 16, 700, ("c3_8b_sweep", "lens_odd_blocks", B))
    case = build_case(w, B, lens, n_layers=1, max_seq=int(lens.max()) + 2, tag=f"t22_{B}")
    check_dense(orc, case, requests=list(range(B)))


@pytest.mark.parametrize("B", [256, 512])
def test_8b_shape_batch_beyond_128_every_block(orc, B):
    """Decode batches beyond the sweep's largest point (16 to 32 blocks of 16
    rows per projection, thousands of attention pieces per layer), with short
    contexts in [16, 512] so that the cache stays small; two layers, one
    request of every 16-row block."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(B, 16, 512, ("c3_8b_sweep", "lens_short", B))
    case = build_case(w, B, lens, n_layers=2, max_seq=int(lens.max()) + 2, tag=f"t17_{B}")
    check_dense(orc, case)


@pytest.mark.parametrize("B", [8, 12, 16])
def test_8b_shape_split_k_every_request(orc, B):
    """Batches whose staged inputs outgrow the LDS: the projections run as K
    slices whose partial sums the last slice task of each row tile adds (down
    in 4 to 7 slices, the 4096-deep projections in 2 at batch 12 and 16).
    Two layers, every request and every output element against the oracle."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(B, 512, 2048, ("c3_8b_sweep", "split_k", B))
    case = build_case(w, B, lens, n_layers=2, max_seq=int(lens.max()) + 2, tag=f"t11_{B}")
    check_dense(orc, case)


F32_MID = synth.Workload(name="f32_mid", dtype="f32", n_layers=2, hidden=1024, n_q_heads=8, n_kv_heads=2,
                         head_dim=64, ffn_dim=4096, tol=1e-5)


def test_f32_split_k_batch16(orc):
    """float32 weights at batch 16: the 4096-deep down projection's inputs
    (256 KiB staged) take two K slices; the result stays at float32 accuracy."""
    lens = synth.ragged_lengths(16, 1, 300, ("f32_mid", "lens"))
    case = build_case(F32_MID, 16, lens, max_seq=302, tag="t12")
    check_dense(orc, case)


F32_SMALL_QKV = synth.Workload(name="f32_small_qkv", dtype="f32", n_layers=1, hidden=4096, n_q_heads=4,
                               n_kv_heads=2, head_dim=64, ffn_dim=256, tol=1e-5)


def test_f32_small_qkv_batch16_split_records(orc):
    """float32, H 4096 with only 256 QKV rotation units, batch 16 with short
    caches: the QKV and O stages split over K on a grid share that changes
    with the attention tasks' own workgroups, the case whose split-K records
    outgrew an allocation sized for two grid shares only."""
    lens = synth.ragged_lengths(16, 1, 60, ("f32_small_qkv", "lens"))
    case = build_case(F32_SMALL_QKV, 16, lens, max_seq=64, tag="t22")
    check_dense(orc, case)


@pytest.mark.parametrize("sched", ["layer", "stage", "barrier", "op"])
@pytest.mark.parametrize("B", [1, 4])
def test_unfused_schedules_match_oracle(orc, sched, B):
    """The ablation schedules (one launch of the persistent kernel per layer,
    per stage of each layer or per operator, or one launch with a grid-wide
    barrier after every stage) run the same tasks: the same results, at batch
    1 (attention on workgroups of its own, partials merged by the
    O-projection; per-op: chunk partials merged by an op of their own) and
    batch 4 (streamed attention, down projection split over K)."""
    w = synth.get_workload("c3_8b_sweep")
    lens = [512] if B == 1 else synth.ragged_lengths(B, 512, 2048, ("c3_8b_sweep", "sched", B))
    case = build_case(w, B, lens, n_layers=2, max_seq=int(max(lens)) + 2, tag=f"t13_{sched}_{B}")
    check_dense(orc, case, sched=sched)


def test_schedule_setters_reject_unknown_modes(orc):
    """pmk_set_schedule / pmk_set_moe_scheduler on a live handle: unknown
    modes are rejected and leave the handle working (fused step still matches)."""
    from persistent_megakernel_04_amd import _abi
    w = synth.get_workload("c1_tiny_f32")
    case = build_case(w, 1, [40], max_seq=64, tag="t15")
    model = make_model(case)
    assert model.lib.pmk_set_schedule(model.handle, 9) == _abi.PMK_ERR_ARG
    assert model.lib.pmk_set_schedule(model.handle, -1) == _abi.PMK_ERR_ARG
    assert model.lib.pmk_set_moe_scheduler(model.handle, 3) == _abi.PMK_ERR_ARG
    model.close()
    check_dense(orc, case)


@pytest.mark.parametrize("B,L,lo,hi", [(1, 2, 512, 512), (16, 2, 512, 4096), (40, 1, 256, 2048)])
def test_event_granularities_give_identical_bits(orc, B, L, lo, hi):
    """The dense chain's events per tile (per KV group, and per 16-row block
    beyond 16 requests), per KV group only, or one per stage change only who
    waits on what, not the arithmetic: the same hidden states and K/V entries,
    bit for bit, and per tile against the oracle."""
    w = synth.get_workload("c3_8b_sweep")
    lens = [lo] * B if lo == hi else synth.ragged_lengths(B, lo, hi, ("c3_8b_sweep", "events", B))
    case = build_case(w, B, lens, n_layers=L, max_seq=int(max(lens)) + 2, tag=f"t23_{B}")
    inp = oracle_inputs(case, None if B <= 16 else block_requests(lens))
    outs = {}
    for mode in ("stage", "group", "tile"):
        hidden, kv = case.hidden.clone(), case.kv.clone()
        model = make_model(case)
        model.set_event_granularity(mode)
        announce(f"decode_step {w.name} L={L} B={B} events={mode}")
        model.step(hidden, kv, case.seq_lens)
        torch.cuda.synchronize()
        assert model.device_error() == 0
        model.close()
        outs[mode] = (hidden, kv)
    for mode in ("group", "tile"):
        assert torch.equal(outs[mode][0].view(torch.int32), outs["stage"][0].view(torch.int32)), mode
        assert torch.equal(outs[mode][1].view(torch.int16), outs["stage"][1].view(torch.int16)), mode
    hidden, kv = outs["tile"]
    rq = inp["requests"]
    kv_gpu = to_np(kv[:, :, rq] if B > 16 else kv)
    check_against_oracle(orc, case, inp, to_np(hidden).astype(np.float64)[rq], kv_gpu)
