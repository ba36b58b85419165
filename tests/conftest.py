import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


# Host sanitizer runs (tests/test_host_sanitizers.py): a child pytest process
# gets the address/undefined-behaviour sanitized builds of the library's host
# code (metadata builder, layer plan, cache estimate) and of the oracle in
# these variables, and the tests then call those instead.
_HOST_LIB = os.environ.get("SWA_TEST_SANITIZED_HOST_LIB")
_ORACLE_LIB = os.environ.get("SWA_TEST_SANITIZED_ORACLE_LIB")
if _HOST_LIB:
    import ctypes

    import causal_sliding_window_swa_amd as _swa

    _L = ctypes.CDLL(_HOST_LIB)
    _P, _I = ctypes.c_void_p, ctypes.c_int
    _L.swa_blockmask_size.argtypes = [_I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t),
                                      ctypes.POINTER(ctypes.c_size_t)]
    _L.swa_blockmask_build.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P,
                                       _P, _P, _P, _P, _P, ctypes.POINTER(_swa.MaskStats)]
    _L.swa_layer_plan.argtypes = [_I, _I, _I, _I, _P, _P, _P]
    _L.swa_cache_bytes.argtypes = [_I, _I, _I, _I, ctypes.c_int64, _I, _P, _P]
    _L.swa_last_error.argtypes = []
    _L.swa_last_error.restype = ctypes.c_char_p
    for _n in ("swa_blockmask_size", "swa_blockmask_build", "swa_layer_plan", "swa_cache_bytes"):
        getattr(_L, _n).restype = ctypes.c_int
    _swa._lib = _L
if _ORACLE_LIB:
    import oracle as _oracle

    _oracle._default = _oracle.Oracle(_ORACLE_LIB)
