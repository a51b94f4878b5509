import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_sessionstart(session):
    # Load what is built; build only if nothing is (the library is git-ignored).
    lib = os.path.join(ROOT, "linear_kernelized_attention_favor_amd", "libfavor.so")
    if not os.path.exists(lib):
        import importlib.util
        path = os.path.join(ROOT, "linear_kernelized_attention_favor_amd", "build_lib.py")
        spec = importlib.util.spec_from_file_location("favor_build_lib", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
