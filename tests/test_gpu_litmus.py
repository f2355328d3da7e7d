"""Cross-XCD message passing with the persistent kernel's own synchronisation
primitives (pmk_event_litmus, through the C ABI): in every round one writer's
device-coherent stores, store drain and relaxed atomic notify must be visible
to eight readers -- one per XCD -- that spin on the counter and then read a
block written once through the caches (as activations are staged) and a block
rewritten every round device-coherently (as split-K records are read). The
run stops at the first stale value."""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_cross_xcd_notify_then_read_sees_no_stale_value():
    from persistent_megakernel_04_amd import _abi
    lib = _abi.load()
    rounds = 8192
    need = rounds * 4224 + 4352
    work = torch.empty(need, dtype=torch.uint8, device="cuda")
    res = torch.empty(8, dtype=torch.int32, device="cuda")
    print(f"[case] pmk_event_litmus rounds={rounds}", flush=True)
    rc = lib.pmk_event_litmus(ctypes.c_void_p(work.data_ptr()), need, rounds, ctypes.c_void_p(res.data_ptr()),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.pmk_strerror(rc)
    torch.cuda.synchronize()
    r = res.cpu().tolist()
    print(f"  first stale round {r[0]}, reader checks {r[6]}, stale values of the rewritten block read "
          f"through the caches (not used by the kernels): {r[7]}", flush=True)
    assert r[5] == 0, "a wait timed out"
    assert r[0] == -1, (f"round {r[0]}: element {r[1]} read {r[2]}, written {r[3]} "
                        f"({'rewritten block, coherent load' if r[4] else 'written-once block, cached load'})")
    assert r[6] == rounds * 8


def test_litmus_argument_checks():
    from persistent_megakernel_04_amd import _abi
    lib = _abi.load()
    assert lib.pmk_event_litmus(None, 0, 1, None, None) == _abi.PMK_ERR_ARG
    buf = torch.empty(1024, dtype=torch.uint8, device="cuda")
    res = torch.empty(8, dtype=torch.int32, device="cuda")
    # too small for 16 rounds: refused before anything is launched
    assert lib.pmk_event_litmus(ctypes.c_void_p(buf.data_ptr()), 1024, 16, ctypes.c_void_p(res.data_ptr()),
                                None) == _abi.PMK_ERR_ARG
