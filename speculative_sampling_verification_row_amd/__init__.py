"""Batched speculative-sampling verification on AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libspecverify.so`` (sources in
``csrc/``, C ABI in ``include/spec_verify.h``); ``binding`` marshals torch
tensors onto it.  Importing this package loads nothing: the library is loaded
on the first call and a missing library raises an error instead of falling
back to any other implementation.
"""

__all__ = ["binding", "inputs"]
