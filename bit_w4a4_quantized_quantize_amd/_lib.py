"""ctypes loader of libsvdq.so, the HIP library built from csrc/ (C ABI in include/svdq.h).

There is no fallback: if the library is missing or fails to load, every call
raises. Build it with ``python -m bit_w4a4_quantized_quantize_amd.build``.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvdq.so")

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_size = ctypes.c_size_t
_int = ctypes.c_int

# name -> (restype, argtypes); mirrors include/svdq.h
SIGNATURES = {
    "svdq_abi_version": (_int, []),
    "svdq_status_string": (ctypes.c_char_p, [_int]),
    "svdq_last_error": (ctypes.c_char_p, []),
    "svdq_debug_mode": (_int, []),
    "svdq_set_gemm_tile": (_int, [_int, ctypes.POINTER(_int)]),
    "svdq_quantize_act_workspace_bytes": (_size, [_i64, _i64, _i64]),
    "svdq_packed_act_bytes": (_size, [_i64, _i64]),
    "svdq_quantize_act": (_int, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _i64, _int,
                                 _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_repack_weight_bytes": (_size, [_i64, _i64]),
    "svdq_repack_weight": (_int, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _size, _c_void_p]),
    "svdq_unpack_weight": (_int, [_c_void_p, _size, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "svdq_gemm_w4a4": (_int, [_c_void_p, _c_void_p, _int, _c_void_p, _c_void_p, _c_void_p, _int,
                              _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                              _i64, _i64, _i64, _i64, _c_void_p, _c_void_p]),
    "svdq_linear_workspace_bytes": (_size, [_i64, _i64, _i64, _i64]),
    "svdq_linear_w4a4": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _int,
                                _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                _i64, _i64, _i64, _i64, _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_calibrate_workspace_bytes": (_size, [_i64, _i64]),
    "svdq_calibrate_act_gscale": (_int, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _size,
                                         _c_void_p]),
    "svdq_quantize_act_static": (_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _c_void_p, _i64, _int,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_linear_w4a4_static": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _int,
                                       _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _i64, _i64, _i64, _i64, _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_noalloc_scratch_bytes": (_size, []),
    "svdq_linear_w4a4_noalloc": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _int,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                        _i64, _i64, _i64, _i64, _c_void_p, _c_void_p]),
    "svdq_gemm_w4a4_gated": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _c_void_p, _i64, _i64, _i64, _i64, _c_void_p, _c_void_p]),
    "svdq_gemm_w4a4_gated_quant": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                          _c_void_p, _i64, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                          _size, _c_void_p]),
    "svdq_lowrank_down": (_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_linear_gated_workspace_bytes": (_size, [_i64, _i64, _i64, _i64]),
    "svdq_linear_w4a4_gated": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                      _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i64,
                                      _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_linear_bf16": (_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p]),
    "svdq_prepare_workspace_bytes": (_size, [_i64, _i64, _i64]),
    "svdq_prepare_weight": (_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _int,
                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p, _size, _c_void_p]),
    "svdq_prepare_residual": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64,
                                     _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_mx_codes_bytes": (_size, [_i64, _i64]),
    "svdq_mx_scales_bytes": (_size, [_i64, _i64]),
    "svdq_reround_weight_mxfp4": (_int, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "svdq_quantize_act_mxfp4": (_int, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "svdq_gemm_mxfp4": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                               _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _c_void_p, _c_void_p]),
    "svdq_linear_mxfp4_workspace_bytes": (_size, [_i64, _i64, _i64]),
    "svdq_linear_mxfp4": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                 _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _c_void_p, _c_void_p, _size,
                                 _c_void_p]),
    "svdq_calib_table_bytes": (_size, []),
    "svdq_calib_flop_per_iteration": (_i64, [_i64]),
    "svdq_calib_mfma": (_int, [_c_void_p, _size, _i64, _i64, _c_void_p, _size, _c_void_p, _size, _c_void_p]),
    "svdq_calib_scaled_flop_per_iteration": (_i64, [_i64]),
    "svdq_calib_mfma_scaled": (_int, [_c_void_p, _size, _i64, _i64, _int, _c_void_p, _size, _c_void_p, _size,
                                      _c_void_p]),
    "svdq_calib_lds_bytes_per_iteration": (_i64, [_i64]),
    "svdq_calib_lds": (_int, [_i64, _i64, _int, _c_void_p, _size, _c_void_p]),
    "svdq_calib_copy": (_int, [_c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_calib_wall_clock_khz": (_int, [ctypes.POINTER(_int)]),
}

STATUS = {
    0: "SVDQ_OK", 1: "SVDQ_ERR_NULL", 2: "SVDQ_ERR_SHAPE", 3: "SVDQ_ERR_UNSUPPORTED",
    4: "SVDQ_ERR_ALIGN", 5: "SVDQ_ERR_WORKSPACE", 6: "SVDQ_ERR_ALIAS", 7: "SVDQ_ERR_HIP",
    8: "SVDQ_ERR_INVALID",
}
WEIGHT_CANONICAL = 0
WEIGHT_PACKED = 1
ACT_CANONICAL = 0
ACT_PACKED = 1
ACT_MXFP4 = 2

_lib = None


def lib():
    """The loaded library (loaded once). Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m bit_w4a4_quantized_quantize_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class SvdqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        L = lib()
        msg = L.svdq_last_error().decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({L.svdq_status_string(status).decode()}): {msg}")


def check(fn, status):
    if status != 0:
        raise SvdqError(fn, status)
