"""Wave-index decode attention and segmented k-means index build for MI355X.

The compute lives in a HIP shared library (libwi.so, C ABI declared in
include/wi.h); `wi` is its thin ctypes binding. Importing the package does
not load the library; `wi.lib()` does, and raises if it is missing.
"""
from . import synth  # noqa: F401
