import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # Tests load what is built; they build only when nothing is there.
    import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build(force=False)
    from quantized_matmul_rmsnorm_amd import build as lib_build
    if not os.path.exists(lib_build.LIB):
        lib_build.build()
