import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_LIB = os.path.join(ROOT, "paged_kv_cache_83_amd", "libpa.so")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The library is normally built beforehand (__graft_entry__.build()); build it
    # here only when it is missing entirely, so CPU test runs are self-contained.
    if not os.path.exists(_LIB):
        import importlib.util
        path = os.path.join(ROOT, "paged_kv_cache_83_amd", "build.py")
        spec = importlib.util.spec_from_file_location("_pa_build", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
