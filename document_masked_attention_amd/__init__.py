"""Document-masked attention for MI355X (gfx950).

The compute path is the HIP library ``libdocmask.so`` (C ABI declared in
``include/docmask.h``); ``api`` holds the thin Python binding.  Importing this
package does not load the library; the first call does, and it raises if the
library has not been built.
"""
__all__ = ["api", "workloads"]
