"""The C-ABI library loads on a machine without a GPU and exports every entry
point declared in include/pmk.h; the Python binding names the same set.
No compute call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pmk.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("decode_layer_init", "decode_step", "moe_layer_step", "decode_layer_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from persistent_megakernel_04_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("libpmk.so not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(_abi.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(_abi.EXPORTS) == declared_functions()


def test_strerror_and_null_handle_errors_need_no_gpu():
    from persistent_megakernel_04_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("libpmk.so not built")
    lib = _abi.load()
    assert lib.pmk_strerror(0) == b"ok"
    assert b"argument" in lib.pmk_strerror(_abi.PMK_ERR_ARG)
    # null handles are rejected before any HIP call
    assert lib.decode_step(None, None, None, None, 1, None) == _abi.PMK_ERR_ARG
    assert lib.moe_layer_step(None, None, None, None, 1, None, None) == _abi.PMK_ERR_ARG
    assert lib.pmk_get_device_error(None) == _abi.PMK_ERR_ARG
    assert lib.pmk_query(None, None) == _abi.PMK_ERR_ARG
    assert lib.decode_layer_destroy(None) == _abi.PMK_OK
    assert lib.pmk_trace_attach(None, None, 0) == _abi.PMK_ERR_ARG
    assert lib.pmk_set_schedule(None, _abi.SCHED_FUSED) == _abi.PMK_ERR_ARG
    assert lib.pmk_set_moe_scheduler(None, _abi.MOE_DYNAMIC) == _abi.PMK_ERR_ARG
    assert lib.pmk_set_watchdog_us(None, 1) == _abi.PMK_ERR_ARG
    assert lib.pmk_timing_enable(None, 1) == _abi.PMK_ERR_ARG
    out = ctypes.c_void_p()
    assert lib.decode_layer_init(None, None, ctypes.byref(out)) == _abi.PMK_ERR_ARG
