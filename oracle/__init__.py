"""CPU oracle for the SVDQuant W4A4 NVFP4 linear layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (no kernels, headers, tables or helpers) and never imports it.

It is a plain, slow, obviously correct restatement of what the pages define,
in NumPy with float64 / int64 arithmetic:

* ``formats``  - bf16, E2M1 (FP4) and float8_e4m3fn encode/decode, nibble pack.
* ``svdq``     - activation quantisation, weight quantisation (input
                 preparation), dequantisation, the main scaled GEMM, the
                 low-rank residual and the epilogue of the layer
                 y = scaled_mma(quant(x*smooth), qweight, ascales, wscales)
                     * wtscale * wcscales + (x @ proj_down) @ proj_up^T + bias
                 (model card "nunchaku-z-image-turbo-svdq", section
                 "What's stored on disk", runtime reconstruction formula).
* ``prep``     - SVDQuant weight preparation from a bf16 weight: smoothing,
                 the rank-R split (exact truncated SVD as the optimum, and the
                 randomized range finder the device runs), the residual, the
                 two-level scales and the residual's quantisation.
* ``mx``       - the MXFP4 datatype variant (E2M1 with power-of-two scales per
                 32 K, re-rounded from the NVFP4 operands): quantiser,
                 dequantiser and the variant layer.
* ``repack``   - the index map of the library's MFMA-order weight layout,
                 written independently from its definition, so the GPU repack
                 can be compared byte for byte.

Parity pins (tests/test_oracle_*.py) tie every function to something other
than itself: the E2M1 grid and bit structure, the e4m3fn range, exhaustive
decode tables, torch's float8_e4m3fn cast, exact rational brute force on tiny
shapes, the int64-exact form of the main term, and the formula's closed-form
special cases (R = 0, qweight = 0, lossless inputs).

Parity unpinned: agreement with third-party implementations of the layer
(nunchaku, vLLM, the CuTe kernels). The pages publish no checkpoint, kernel
output or test vector, so the activation quantiser is pinned only to the
readings stated in svdq.py, not to any published artifact.
"""

from . import formats, svdq, repack, prep, mx  # noqa: F401
