import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # the host-sanitizer test reruns the CPU boundary tests against a sanitized
    # host-only build of the library, named here
    lib = os.environ.get("LA_TEST_LIBRARY")
    if lib:
        import linear_attention_video_02_amd as la
        la.LIB_PATH = lib
