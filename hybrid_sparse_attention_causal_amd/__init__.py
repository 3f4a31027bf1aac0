"""HySparse hybrid-block attention hot path for AMD MI355X (gfx950).

The compute lives in a C-ABI HIP library (libhysparse.so, declared in
include/hysparse.h); `binding` marshals torch device tensors into it.  The
library is loaded lazily on first use and its absence is an error.
"""
__all__ = ["inputs", "binding"]
