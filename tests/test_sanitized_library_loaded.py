"""Inside the sanitizer run of test_host_sanitizers.py: the library the
binding loaded is the instrumented build named by PA_LIBRARY.  Outside that
run (no PA_LIBRARY) this checks nothing."""
import os

import paged_kv_cache_302_amd as pa


def test_binding_loads_the_named_library():
    want = os.environ.get("PA_LIBRARY")
    lib = pa.load_library()
    if want:
        assert pa.LIB_PATH == want
        assert os.path.samefile(lib._name, want)
