"""The tile weight layout: pmk_pack_weights and handles with weight_layout
"tiles", through the C ABI.

The layout changes only where each 16-byte weight piece is read from: every
MFMA receives the same operands in the same order as with row-major weights,
so a step on packed weights must reproduce the row-major step bit for bit,
and both match the oracle. Each case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import synth
from _cases import block_requests, build_case, make_model, oracle_inputs, to_np

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[case] {msg}", flush=True)


def tile_layout_reference(m: np.ndarray) -> np.ndarray:
    """The layout written out from its definition: element (r, c) at
    ((r // 16) * (cols // 32) + c // 32) * 512 + (r % 16) * 32 + c % 32."""
    rows, cols = m.shape
    out = np.empty(rows * cols, m.dtype)
    for r in range(rows):
        for c in range(cols):
            out[((r // 16) * (cols // 32) + c // 32) * 512 + (r % 16) * 32 + c % 32] = m[r, c]
    return out


@pytest.mark.parametrize("rows,cols", [(16, 32), (48, 96), (64, 4096)])
def test_pack_layout_matches_definition(rows, cols):
    from persistent_megakernel_04_amd.model import pack_weights
    gen = torch.Generator().manual_seed(rows * 131 + cols)
    m = torch.randint(-32768, 32767, (rows, cols), generator=gen, dtype=torch.int16)
    announce(f"pmk_pack_weights {rows}x{cols}")
    got = pack_weights(m.view(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.view(torch.int16).cpu().numpy().ravel(), tile_layout_reference(m.numpy()))


def test_pack_large_stacked_matrix_sampled():
    """A stack of expert matrices [E][rows][cols] packs as one matrix of
    E rows rows; 8192 sampled pieces of a 128 x 768 x 2048 stack."""
    from persistent_megakernel_04_amd.model import pack_weights
    E, rows, cols = 128, 768, 2048
    gen = torch.Generator(device="cuda").manual_seed(11)
    announce(f"pmk_pack_weights stack {E}x{rows}x{cols}")
    src = torch.randint(-32768, 32767, (E, rows, cols), generator=gen, dtype=torch.int16, device="cuda")
    got = pack_weights(src.view(torch.bfloat16)).view(torch.int16)
    torch.cuda.synchronize()
    src_np, got_np = to_np(src).reshape(E * rows, cols), to_np(got).reshape(-1, 8)   # 16-byte pieces
    rng = np.random.default_rng(12)
    n = 8192
    r, s, g = rng.integers(0, E * rows, n), rng.integers(0, cols // 32, n), rng.integers(0, 4, n)
    c = 32 * s + 8 * g
    at = ((r // 16) * (cols // 32) + c // 32) * 512 + (r % 16) * 32 + c % 32   # element index of (r, c)
    want = src_np[r[:, None], c[:, None] + np.arange(8)]
    np.testing.assert_array_equal(got_np[at // 8], want)


def run_dense(case, layout, sched=None):
    hidden, kv = case.hidden.clone(), case.kv.clone()
    model = make_model(case, weight_layout=layout)
    if sched is not None:
        model.set_schedule(sched)
    model.step(hidden, kv, case.seq_lens)
    torch.cuda.synchronize()
    assert model.device_error() == 0
    model.close()
    return hidden, kv


def check_tiles_dense(orc, case, requests="auto", sched=None, oracle=True):
    B = case.hidden.shape[0]
    if isinstance(requests, str):
        requests = None if B <= 16 else block_requests(to_np(case.seq_lens))
    announce(f"tiles vs rows {case.w.name} L={case.n_layers} B={B} lens={to_np(case.seq_lens).tolist()[:8]} "
             f"schedule={sched or 'fused'}")
    h_rows, kv_rows = run_dense(case, "rows", sched)
    h_tiles, kv_tiles = run_dense(case, "tiles", sched)
    assert torch.equal(h_rows.view(torch.int32), h_tiles.view(torch.int32)), "hidden differs between layouts"
    assert torch.equal(kv_rows.view(torch.int16), kv_tiles.view(torch.int16)), "KV cache differs between layouts"
    if oracle:
        from test_gpu_dense import check_against_oracle
        inp = oracle_inputs(case, requests)
        print("  bit-identical between layouts", flush=True)
        kv_gpu = to_np(kv_tiles[:, :, inp["requests"]] if requests is not None else kv_tiles)
        check_against_oracle(orc, case, inp, to_np(h_tiles).astype(np.float64)[inp["requests"]], kv_gpu)


def test_tiles_8b_full_stack_b1_bench_config(orc):
    """The benchmark's workload with packed weights: 32 layers, batch 1."""
    w = synth.get_workload("c2_8b_b1")
    case = build_case(w, 1, [512], max_seq=613, tag="")
    check_tiles_dense(orc, case)


@pytest.mark.parametrize("B", [4, 16])
def test_tiles_8b_two_layers_ragged(orc, B):
    """Batch 4 (one pass) and batch 16 (split-K slices with partial records);
    every request against the oracle."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(B, 512, 8192, ("c3_8b_sweep", "lens", B))
    case = build_case(w, B, lens, n_layers=2, max_seq=int(lens.max()) + 2, tag=f"tl{B}")
    check_tiles_dense(orc, case)


def test_tiles_8b_batch_64_blocks(orc):
    """Batch 64: the batch in 16-row blocks, each block a task of its own."""
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(64, 512, 2048, ("c3_8b_sweep", "lens", 64, "tiles"))
    case = build_case(w, 64, lens, n_layers=1, max_seq=int(lens.max()) + 2, tag="tl64")
    check_tiles_dense(orc, case)


def test_tiles_70b_shape_two_layers_b8(orc):
    """70B-shaped layers: FFN depth 28672 in several K slices."""
    w = synth.get_workload("c5_70b")
    lens = synth.ragged_lengths(8, 8192, 16384, ("c5_70b", "lens", 8))
    case = build_case(w, 8, lens, n_layers=2, max_seq=int(lens.max()) + 2, tag="tl70")
    check_tiles_dense(orc, case)


@pytest.mark.parametrize("sched", ["layer", "barrier"])
def test_tiles_unfused_schedules(orc, sched):
    w = synth.get_workload("c3_8b_sweep")
    lens = synth.ragged_lengths(4, 512, 4096, ("c3_8b_sweep", "lens", 4, sched))
    case = build_case(w, 4, lens, n_layers=2, max_seq=int(lens.max()) + 2, tag=f"tls{sched}")
    check_tiles_dense(orc, case, sched=sched, oracle=False)


def run_moe_layout(case, layout, moe_sched=None):
    from persistent_megakernel_04_amd import DecodeModel
    from test_gpu_moe import routing_buffers
    w, T = case.w, case.hidden.shape[0]
    hidden, kv = case.hidden.clone(), case.kv.clone()
    model = DecodeModel.from_workload(w, case.layers, case.max_batch, case.max_seq, weight_layout=layout)
    assert model.info()["moe_bm"] == 16
    if moe_sched is not None:
        model.set_moe_scheduler(moe_sched)
    rb = routing_buffers(T, w.n_experts, w.top_k)
    assert model.moe_layer_step(hidden, kv, case.seq_lens, rb) == 0
    torch.cuda.synchronize()
    assert model.device_error() == 0
    model.close()
    return hidden, {k: to_np(v) for k, v in rb.items()}


@pytest.mark.parametrize("T,moe_sched", [(1, "static"), (16, "static"), (128, "dynamic")])
def test_tiles_moe_qwen3_shape(orc, T, moe_sched):
    """MoE layer (router, grouped expert gate/up and down) on packed weights:
    outputs and routing identical to the row-major handle, and against the
    oracle as the row-major layer is."""
    from test_gpu_moe import compare_moe
    w = synth.get_workload("c4_moe")
    case = build_case(w, T, [2048] * T, max_seq=2049, tag=f"tlm{T}")
    announce(f"moe tiles vs rows {w.name} T={T} scheduler={moe_sched}")
    inp = oracle_inputs(case)
    h_rows, r_rows = run_moe_layout(case, "rows", moe_sched)
    h_tiles, r_tiles = run_moe_layout(case, "tiles", moe_sched)
    assert torch.equal(h_rows.view(torch.int32), h_tiles.view(torch.int32)), "hidden differs between layouts"
    for k in r_rows:
        np.testing.assert_array_equal(r_rows[k], r_tiles[k], err_msg=k)
    desc = orc.make_desc(w, T, case.max_seq, n_layers=1)
    kv_ref = inp["kv"][0]
    ref, r_ref = orc.moe_layer(desc, inp["layers"][0], kv_ref, inp["seq_lens"], inp["hidden"], 16)
    r_ref["routed"] = lambda idx: orc.moe_layer_routed(desc, inp["layers"][0], kv_ref, inp["seq_lens"],
                                                       inp["hidden"], idx)[0]
    compare_moe(w, T, to_np(h_tiles).astype(np.float64), ref, r_tiles, r_ref, 16)
