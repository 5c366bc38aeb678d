"""cross_model_kv_amd: closed-form cross-model KV-cache mapping on AMD Instinct MI355X.

The compute lives in libkvmap (HIP kernels for gfx950 behind the C-ABI declared in
include/kvmap.h); ``cross_model_kv_amd.kvmap`` is its ctypes binding.
"""

from . import kvmap  # noqa: F401
from .kvmap import Context, GramState, KvmapError  # noqa: F401

__all__ = ["kvmap", "Context", "GramState", "KvmapError"]
