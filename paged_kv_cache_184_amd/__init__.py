"""Paged KV-cache attention for MI355X (gfx950): a C-ABI HIP library plus a thin binding.

Importing the package loads nothing native; ``paged_kv_cache_184_amd.ops`` loads
``libpkv.so`` on first use and raises if it is missing.
"""
