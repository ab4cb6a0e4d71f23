"""Activation-sparse ReLU feedforward layer for AMD MI355X (gfx950).

The compute lives in libsffn.so (HIP kernels behind the C ABI of
include/sffn.h); :mod:`.binding` marshals torch tensors into it and
:mod:`.workloads` draws the seeded synthetic inputs.
"""
from .binding import SparseFFN, SffnError, load_library  # noqa: F401
