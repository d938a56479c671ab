import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # another build of the library under test (the host-sanitizer build of
    # tests/sanitize_host.py); CPU-only runs
    lib = os.environ.get("HW_TEST_LIB")
    if lib:
        from decode_attention_shared_hw_amd import hogwild_attn as hw
        hw.LIB_PATH = lib
