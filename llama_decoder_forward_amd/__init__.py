"""MI355X (gfx950) Llama-2 decoder forward: prefill, static-KV decode and
sampling in hand-written HIP kernels behind the C ABI of include/llm.h.

``binding`` (the ctypes wrapper of libllm.so) is imported on first use so
that the workload tables and synthetic inputs stay importable on machines
without the built library; the binding itself raises if the library is
missing.
"""
from . import configs, synth  # noqa: F401


def __getattr__(name):
    if name == "binding":
        import importlib
        return importlib.import_module(".binding", __name__)
    raise AttributeError(name)
