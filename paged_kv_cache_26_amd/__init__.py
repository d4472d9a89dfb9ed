"""MI355X-native paged decode attention: libpkv (HIP, gfx950) and its Python binding.

Importing the package loads nothing; the binding in ``paged_kv_cache_26_amd.pkv`` loads
libpkv.so on first use and raises if it has not been built.
"""

__all__ = ["pkv", "workload", "build"]
