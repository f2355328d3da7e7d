"""decode_step_static -- the decode step for callers that cannot allocate
(its workspace in the library's static device scratch) -- against decode_step
on a handle, through the C ABI: two calls in a row, the second with a smaller
batch and other lengths, each checked against the handle's outputs on the
same inputs within the parity bounds (every element within ELEM_TOL of its
row's RMS, appended K/V entries within one bfloat16 ulp), the first also
against the oracle; and a workspace beyond the scratch is refused before
anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from _cases import (BF16_ULP_REL, ELEM_TOL, ELEM_TOL_OWN, build_case, check_rows, make_model, oracle_inputs,
                    run_oracle_dense, to_np)

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[case] {msg}", flush=True)


def appended_rows(kv, lens):
    """Rows (request, layer, K or V) of the entries each request appended at its slot seq_len."""
    a = to_np(kv)
    rows = [a[:, :, i, :, int(s)].reshape(-1, a.shape[3] * a.shape[5]) for i, s in enumerate(lens)]
    r = np.concatenate(rows)
    return (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if r.dtype == np.uint16 else r


def test_static_step_matches_handle_step_twice(orc):
    w = synth.get_workload("c3_8b_sweep")
    B = 4
    lens = synth.ragged_lengths(B, 300, 2048, ("c3_8b_sweep", "static", B))
    case = build_case(w, B, lens, n_layers=2, max_seq=int(max(lens)) + 2, tag="t_static")
    model = make_model(case)
    for call, (nb, lens_c) in enumerate(((B, list(lens)), (2, [5, int(lens[0]) // 3]))):
        hidden0 = case.hidden[:nb].clone()
        sl = torch.tensor(lens_c, dtype=torch.int32, device="cuda")
        kv0 = case.kv.clone()
        inp = None
        if call == 0:
            inp = oracle_inputs(case, None)
        announce(f"decode_step (handle) 8B-shaped L=2 B={nb} lens={lens_c}")
        h_ref, kv_ref = hidden0.clone(), kv0.clone()
        assert model.decode_step(h_ref, kv_ref, sl) == 0
        torch.cuda.synchronize()
        assert model.device_error() == 0
        announce(f"decode_step_static 8B-shaped L=2 B={nb} lens={lens_c} (call {call + 1})")
        h_s, kv_s = hidden0.clone(), kv0.clone()
        status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        assert model.decode_step_static(h_s, kv_s, sl, status) == 0
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        check_rows(to_np(h_s).astype(np.float64), to_np(h_ref).astype(np.float64), w, "static vs handle hidden",
                   elem_tol=ELEM_TOL[w.dtype])
        check_rows(appended_rows(kv_s[:, :, :nb], lens_c), appended_rows(kv_ref[:, :, :nb], lens_c), w,
                   "static vs handle appended K/V", ulp_rel=BF16_ULP_REL, elem_tol=ELEM_TOL[w.dtype])
        # every other cache slot untouched by both
        for i, s in enumerate(lens_c):
            kv_s[:, :, i, :, s] = 0
            kv_ref[:, :, i, :, s] = 0
        assert torch.equal(kv_s, kv_ref)
        if inp is not None:   # the first call also against the oracle
            ref, _ = run_oracle_dense(orc, case, inp)
            check_rows(to_np(h_s).astype(np.float64), ref, w, "static vs oracle", elem_tol=ELEM_TOL_OWN[w.dtype])
    model.close()


def test_static_step_refuses_a_workspace_beyond_the_scratch():
    """32 layers at batch 64 and 8192 positions need more than the static
    scratch: PMK_ERR_SCRATCH, with nothing launched (the weight pointers are
    never read)."""
    from persistent_megakernel_04_amd import _abi
    lib = _abi.load()
    w = synth.get_workload("c2_8b_b1")
    d = _abi.ModelDesc()
    d.abi_version = _abi.PMK_ABI_VERSION
    d.dtype = _abi.PMK_BF16
    d.n_layers, d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim = 32, w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim
    d.ffn_dim, d.max_batch, d.max_seq, d.rms_eps, d.rope_theta = w.ffn_dim, 64, 8192, 1e-5, 10000.0
    d.weight_layout = _abi.PMK_ROWS
    dummy = torch.zeros(16, device="cuda")
    arr = (_abi.LayerWeights * 32)()
    for i in range(32):
        for f in _abi.LAYER_FIELDS[:7]:
            setattr(arr[i], f, dummy.data_ptr())
    wts = _abi.Weights(32, arr)
    p = ctypes.c_void_p(dummy.data_ptr())
    announce("decode_step_static with a workspace beyond the scratch (refused on the host)")
    rc = lib.decode_step_static(ctypes.byref(d), ctypes.byref(wts), p, p, p, 1, None, None)
    assert rc == _abi.PMK_ERR_SCRATCH, lib.pmk_strerror(rc)
    assert b"scratch" in lib.pmk_strerror(rc)
