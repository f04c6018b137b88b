"""MI355X (gfx950) q8-plane producers, q4_K / q6_K integer-dot matmuls and
q4_K / q5_K / q6_K one-token GEMVs.

The compute lives in libmmq.so (hand-written HIP kernels behind the C ABI of
include/mmq.h); ``_lib`` is its ctypes binding, re-exported here under the C
names (mmq_quant_rms, mmq_quant_swiglu, mmq_quant_f32, mmq_gemm_q4k,
mmq_gemm_q6k, mmvq_q6k, mmvq_q4k, mmvq_q5k, ...).  Loading happens on first
attribute access, so ``quantized_matmul_rmsnorm_amd.build`` can run before the
library exists; any
other access without a built library raises ImportError -- there is no
fallback implementation.
"""


import importlib


def __getattr__(name):
    if name.startswith("__") or name in ("_lib", "build"):
        raise AttributeError(name)
    lib = importlib.import_module(__name__ + "._lib")
    return getattr(lib, name)
