"""MI355X-native sparse-KV decode step.

Importing the package loads nothing native.  ``sparse_kv_cache_block_amd.binding``
loads the compiled HIP library (``libsparsekv.so``) on first use and raises if
it is missing; there is no CPU fallback.
"""
from . import configs  # noqa: F401

__all__ = ["configs"]
