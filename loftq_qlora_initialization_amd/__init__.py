"""LoftQ initialisation on AMD Instinct MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in ``libloftq.so`` (see include/loftq.h); ``binding`` is its thin
ctypes wrapper and ``synth`` the seeded input generators.  Binding names are
resolved lazily, so importing ``synth`` alone does not load the library, while any
use of an entry point loads it and raises ImportError if it is not built.
"""
from __future__ import annotations

import importlib

_BINDING_NAMES = {
    "loftq_nf4_quantize", "loftq_double_quant", "loftq_nf4_dequantize", "loftq_nf4_merge", "loftq_nf4_unmerge",
    "loftq_lowrank_svd", "loftq_init", "loftq_qlora_forward", "qlora_forward_workspace_bytes",
    "default_config", "nf4_codebook", "nf_codebook", "exported_symbols", "workspace_bytes", "lowrank_workspace_bytes",
    "InitBuffers", "LoftqConfig", "LoftqError", "LIB_PATH", "EXPORTS", "profile_enable", "profile_collect", "profile_calibrate",
    "loftq_init_batch", "BatchRunner", "LoftqMatrix", "loftq_qlora_forward_noalloc", "qlora_forward_noalloc_max_bytes",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        return getattr(importlib.import_module(".binding", __name__), name)
    raise AttributeError(name)
