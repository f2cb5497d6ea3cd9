"""Batch-1 FP16 decode as one persistent HIP kernel on MI355X (gfx950).

``persistent_runtime_amd.lf`` binds the C ABI of ``liblf.so`` (declared in
``include/lf.h``); ``roofline`` holds the algorithmic byte model.  Importing the
package loads nothing; the native library is loaded on first use of ``lf``.
"""
