"""MI355X (gfx950) KV-cache importance scoring and compaction after prefill.

The compute lives in libkvc.so (hand-written HIP, C ABI in include/kvc.h);
``binding`` exposes the same entry points over torch device tensors and
``pipeline`` chains them into InfoKV's and SelKV's paths.  ``configs`` and
``synth`` describe the synthetic Llama-shaped workloads.
"""
from .configs import ALL, BY_NAME, Workload, reduced  # noqa: F401

__all__ = ["ALL", "BY_NAME", "Workload", "reduced", "binding", "pipeline", "synth", "build"]


def __getattr__(name):
    # binding/pipeline load the HIP library on first use; configs/synth do not
    if name in ("binding", "pipeline", "synth", "build"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
