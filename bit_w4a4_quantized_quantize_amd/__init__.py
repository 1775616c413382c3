"""MI355X (gfx950) SVDQuant W4A4 NVFP4 linear layer: HIP kernels behind a C ABI.

    y = scaled_mma(quant(x * smooth), qweight, ascales, wscales) * wtscale * wcscales
        + (x @ proj_down) @ proj_up^T + bias

The compute lives in libsvdq.so (csrc/*.hip, C ABI in include/svdq.h);
``ops`` is the PyTorch-facing binding. Importing this package does not load
the library; the first call does, and fails loudly if it is not built.
"""

from . import _lib  # noqa: F401

__all__ = ["ops", "build"]
