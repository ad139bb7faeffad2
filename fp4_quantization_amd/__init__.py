"""fp4_quantization_amd: fused normalization + FP8 / NVFP4 activation
quantization for AMD Instinct MI355X (gfx950).

The compute path is ``libnq.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/nq.h``); :mod:`fp4_quantization_amd.nq` is its thin
Python binding.  Importing that module loads the library and raises if it is
missing: there is no CPU fallback.

:mod:`fp4_quantization_amd.workloads` (seeded synthetic inputs) and
:mod:`fp4_quantization_amd.traffic` (the byte model) are plain Python and do
not load the library.
"""

__version__ = "0.1.0"


def __getattr__(name):
    # Lazy: `fp4_quantization_amd.nq_*` resolves through the binding, which
    # loads libnq.so (and fails loudly when it is absent).
    if name.startswith("nq_") or name in ("nq", "NQError"):
        import importlib
        _nq = importlib.import_module(__name__ + ".nq")
        return _nq if name == "nq" else getattr(_nq, name)
    raise AttributeError(name)
