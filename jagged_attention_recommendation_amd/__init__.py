"""Jagged attention (JFA softmax and GDPA activation attention) for MI355X (gfx950).

The compute lives in ``libgdpa.so`` (hand-written HIP kernels behind a C ABI, declared in
``include/gdpa.h``); :mod:`.gdpa` is the thin ctypes binding. :mod:`.inputs` draws seeded synthetic
problems and :mod:`.workload` counts useful flops and bytes.
"""
from . import inputs, workload  # noqa: F401

__all__ = ["inputs", "workload"]
