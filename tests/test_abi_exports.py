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
    # the no-allocation step checks its descriptor and pointers before any HIP call
    assert lib.decode_step_static(None, None, None, None, None, 1, None, None) == _abi.PMK_ERR_ARG
    assert b"scratch" in lib.pmk_strerror(_abi.PMK_ERR_SCRATCH)


def test_pack_weights_and_tile_layout_argument_checks_need_no_gpu():
    """pmk_pack_weights and the weight_layout field reject bad arguments before
    any HIP call."""
    from persistent_megakernel_04_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("libpmk.so not built")
    lib = _abi.load()
    a, b = 4096, 1 << 20   # host-side stand-ins: never dereferenced on these paths
    assert lib.pmk_pack_weights(None, b, 16, 32, None) == _abi.PMK_ERR_ARG
    assert lib.pmk_pack_weights(a, None, 16, 32, None) == _abi.PMK_ERR_ARG
    assert lib.pmk_pack_weights(a, b, 24, 32, None) == _abi.PMK_ERR_ARG    # rows not a multiple of 16
    assert lib.pmk_pack_weights(a, b, 16, 48, None) == _abi.PMK_ERR_ARG    # cols not a multiple of 32
    assert lib.pmk_pack_weights(a, b, 0, 32, None) == _abi.PMK_ERR_ARG
    assert lib.pmk_pack_weights(a + 8, b, 16, 32, None) == _abi.PMK_ERR_ARG   # unaligned
    assert lib.pmk_pack_weights(a, a + 512, 16, 32, None) == _abi.PMK_ERR_ARG  # overlapping

    def desc(**kw):
        d = _abi.ModelDesc(abi_version=_abi.PMK_ABI_VERSION, dtype=_abi.PMK_BF16, n_layers=1, hidden=4096,
                           n_q_heads=32, n_kv_heads=8, head_dim=128, ffn_dim=14336, max_batch=1, max_seq=16,
                           rms_eps=1e-5, rope_theta=1e4, weight_layout=_abi.PMK_TILES)
        for k, v in kw.items():
            setattr(d, k, v)
        return d
    out = ctypes.c_void_p()
    init = lambda d: lib.decode_layer_init(ctypes.byref(d), None, ctypes.byref(out))
    assert init(desc(weight_layout=2)) == _abi.PMK_ERR_ARG
    assert init(desc(dtype=_abi.PMK_F32, head_dim=64)) == _abi.PMK_ERR_UNSUPPORTED   # tiles are bfloat16 only
    assert init(desc(ffn_dim=14344)) == _abi.PMK_ERR_UNSUPPORTED                      # F not a multiple of 32
    assert init(desc(hidden=4104)) == _abi.PMK_ERR_UNSUPPORTED                        # H not a multiple of 32
    # a valid description still needs weights
    assert init(desc()) == _abi.PMK_ERR_ARG
