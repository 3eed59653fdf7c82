"""pytest plugin of the host sanitizer run (``-p tests.host_double.plugin``,
loaded by tests/test_host_sanitizers.py in a child process).

It rebinds the package's ctypes handle to the CPU build of the C ABI whose
kernel launchers only record (TP_HOST_DOUBLE_LIB), and the oracle to its
sanitizer build (ORACLE_SANITIZED_LIB); both were compiled with
-fsanitize=address,undefined.  At the end it prints how many launches broke
the launchers' stated argument invariants."""
import ctypes
import os

ACTIVE = False
recorder = None


def pytest_configure(config):
    global ACTIVE, recorder
    from megatron_tensor_transformer_colpar_amd import tp

    import oracle

    path = os.environ["TP_HOST_DOUBLE_LIB"]
    tp.raw = tp._bind(ctypes.CDLL(path))
    tp.LIB_PATH = path
    recorder = ctypes.CDLL(path)
    recorder.rec_count.restype = ctypes.c_int64
    recorder.rec_violations.restype = ctypes.c_int64
    recorder.rec_get.argtypes = [ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
    oracle._lib = oracle._bind(os.environ["ORACLE_SANITIZED_LIB"])
    ACTIVE = True


def log():
    """The recorded launches, each a tuple of its eight fields."""
    out = []
    buf = (ctypes.c_int64 * 8)()
    for k in range(recorder.rec_count()):
        assert recorder.rec_get(k, buf) == 0
        out.append(tuple(buf))
    return out


def pytest_sessionfinish(session, exitstatus):
    if recorder is not None:
        print("\nHOST DOUBLE VIOLATIONS: %d" % recorder.rec_violations(), flush=True)
