"""C ABI host tests: the library loads without a GPU, exports every entry point
include/svdq.h declares, and rejects bad arguments on the host before any HIP call.

The error-path cases use fake device addresses that are never dereferenced; each
case is built to fail validation, so nothing is ever launched. They are skipped
where a GPU is visible, so a validation regression can never turn one of them
into a launch with fake pointers.
"""

import ctypes
import os
import re

import pytest
import torch

from bit_w4a4_quantized_quantize_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")

no_gpu_only = pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="fake-pointer validation cases run on CPU-only hosts")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svdq_\w+)\s*\(", text)))


def test_header_symbols_exported_and_bound():
    L = _lib.lib()
    names = header_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(L, name), name
        assert name in _lib.SIGNATURES, name
    assert L.svdq_abi_version() == 1
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings():
    L = _lib.lib()
    for code in range(9):
        assert L.svdq_status_string(code).decode()
    assert L.svdq_status_string(99).decode() == "unknown status"


def test_size_queries():
    L = _lib.lib()
    assert L.svdq_repack_weight_bytes(10240, 3840) == 10240 * 3840 // 2 + 10240 * 3840 // 16
    assert L.svdq_repack_weight_bytes(33, 80) == 2 * 2 * 1152
    assert L.svdq_repack_weight_bytes(10, 15) == 0
    ws = L.svdq_linear_workspace_bytes(4096, 10240, 3840, 128)
    assert ws >= 4096 * 1920 + 240 * 4096 + 4096 * 128 * 2
    assert L.svdq_quantize_act_workspace_bytes(4096, 3840, 0) == 0
    assert L.svdq_quantize_act_workspace_bytes(0, 3840, 128) == 0


A = 0x7F0000000000  # fake, 16-byte aligned device addresses, never dereferenced


def fake(i):
    return A + i * 0x10000000


def q(**kw):
    args = dict(x=fake(1), smooth=fake(2), M=64, K=256, proj_down=fake(3), R=16,
                qact=fake(4), ascales=fake(5), lora_act=fake(6), ws=fake(7), ws_bytes=1 << 30,
                layout=0, stream=None)
    args.update(kw)
    L = _lib.lib()
    return L.svdq_quantize_act(args["x"], args["smooth"], args["M"], args["K"], args["proj_down"],
                               args["R"], args["layout"], args["qact"], args["ascales"], args["lora_act"],
                               args["ws"], args["ws_bytes"], args["stream"])


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), 2), (dict(K=0), 2), (dict(K=24), 2), (dict(R=-16), 2),
    (dict(R=8), 3), (dict(K=1 << 25), 3), (dict(M=1 << 20, K=1 << 12), 3),
    (dict(x=None), 1), (dict(smooth=None), 1), (dict(qact=None), 1), (dict(ascales=None), 1),
    (dict(proj_down=None), 1), (dict(lora_act=None), 1),
    (dict(x=fake(1) + 8), 4), (dict(ascales=fake(5) + 4), 4),
    (dict(qact=fake(1) + 64), 6), (dict(lora_act=fake(3)), 6), (dict(ascales=fake(4)), 6),
    (dict(layout=3), 8), (dict(layout=1), 8),           # packed needs ascales NULL
    (dict(layout=2, K=192), 3),                         # the MXFP4 layout needs K % 128 == 0
    (dict(layout=2, ascales=None), 1), (dict(layout=2, ascales=fake(4) + 32 * 64), 6),
    (dict(layout=1, ascales=None, qact=fake(2) - 1024 * 4), 6),
])
def test_quantize_act_rejections(kw, code):
    assert q(**kw) == code
    assert _lib.lib().svdq_last_error().decode() != ""


def test_quantize_act_workspace_sizes():
    """Scratch is needed only when the down-projection splits K (R > 0, few 64-row blocks):
    fp32 partials [splits, M, R]; none for R = 0 or many rows."""
    L = _lib.lib()
    for M, K, R in [(65536, 10240, 128), (7, 16, 0), (4096, 3840, 0), (64, 64, 16)]:
        assert L.svdq_quantize_act_workspace_bytes(M, K, R) == 0
    ws = L.svdq_quantize_act_workspace_bytes(4096, 3840, 128)
    assert ws >= 2 * 4096 * 128 * 4 and ws % (4096 * 128 * 4) == 0
    assert L.svdq_linear_workspace_bytes(4096, 10240, 3840, 128) >= ws + 4096 * 128 * 2


@no_gpu_only
def test_quantize_act_workspace_rejections():
    big = dict(M=4096, K=3840, R=128)
    need = _lib.lib().svdq_quantize_act_workspace_bytes(4096, 3840, 128)
    assert q(ws_bytes=need - 1, **big) == 5
    assert q(ws=None, **big) == 1
    assert q(ws=fake(7) + 8, **big) == 4
    assert q(ws=fake(6), **big) == 6          # overlaps lora_act


@no_gpu_only
def test_empty_problem_is_ok_without_pointers():
    assert q(M=0, x=None, smooth=None, qact=None, ascales=None) == 0


def gemm(**kw):
    args = dict(qact=fake(1), ascales=fake(2), act_layout=0, lora=fake(3), weight=fake(4), wscales=fake(5),
                layout=0, wcscales=fake(6), wtscale=fake(7), proj_up=fake(8), bias=fake(9),
                M=64, N=128, K=256, R=16, y=fake(10), stream=None)
    args.update(kw)
    L = _lib.lib()
    return L.svdq_gemm_w4a4(args["qact"], args["ascales"], args["act_layout"], args["lora"], args["weight"],
                            args["wscales"],
                            args["layout"], args["wcscales"], args["wtscale"], args["proj_up"],
                            args["bias"], args["M"], args["N"], args["K"], args["R"], args["y"],
                            args["stream"])


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(N=-3), 2), (dict(K=40), 2), (dict(R=24), 3),
    (dict(layout=5), 8), (dict(layout=1), 8), (dict(wscales=None), 1),
    (dict(qact=None), 1), (dict(y=None), 1), (dict(wtscale=None), 1), (dict(proj_up=None), 1),
    (dict(lora=None), 1), (dict(bias=fake(9) + 2), 4), (dict(weight=fake(4) + 1), 4),
    (dict(y=fake(1)), 6), (dict(y=fake(6) - 64), 6),
    (dict(act_layout=3), 8), (dict(act_layout=1), 8),                         # ascales must be NULL
    (dict(act_layout=1, ascales=None, layout=1, wscales=None, qact=None), 1),
    (dict(act_layout=1, ascales=None, layout=1, wscales=None, M=1 << 20, K=1 << 12), 3),   # packed act > 2 GiB
    (dict(act_layout=1, ascales=None, layout=1, wscales=None, N=1 << 20, K=1 << 12), 3),   # packed weight > 2 GiB
])
def test_gemm_rejections(kw, code):
    assert gemm(**kw) == code


@no_gpu_only
def test_gemm_empty_and_optional_bias_and_r0():
    assert gemm(M=0) == 0
    assert gemm(N=0) == 0
    # R = 0 needs neither lora_act nor proj_up; these calls still fail later only on y=None
    assert gemm(R=0, lora=None, proj_up=None, y=None) == 1


def lin(**kw):
    args = dict(x=fake(1), smooth=fake(2), weight=fake(3), wscales=fake(4), layout=0,
                wcscales=fake(5), wtscale=fake(6), proj_down=fake(7), proj_up=fake(8), bias=None,
                M=64, N=128, K=256, R=16, y=fake(9), ws=fake(10), ws_bytes=1 << 30, stream=None)
    args.update(kw)
    L = _lib.lib()
    return L.svdq_linear_w4a4(args["x"], args["smooth"], args["weight"], args["wscales"], args["layout"],
                              args["wcscales"], args["wtscale"], args["proj_down"], args["proj_up"],
                              args["bias"], args["M"], args["N"], args["K"], args["R"], args["y"],
                              args["ws"], args["ws_bytes"], args["stream"])


@no_gpu_only
def test_linear_rejections():
    L = _lib.lib()
    need = L.svdq_linear_workspace_bytes(64, 128, 256, 16)
    assert lin(ws_bytes=need - 1) == 5
    assert lin(ws=None) == 1
    assert lin(proj_down=None) == 1
    assert lin(y=fake(10)) == 6          # y overlaps the workspace
    assert lin(K=17) == 2
    assert lin(M=0) == 0
    assert lin(layout=1, wscales=None, N=1 << 20, K=1 << 12) == 3   # packed weight > 2 GiB


@no_gpu_only
def test_repack_rejections():
    L = _lib.lib()
    need = L.svdq_repack_weight_bytes(128, 256)
    assert L.svdq_repack_weight(fake(1), fake(2), 128, 256, fake(3), need - 1, None) == 5
    assert L.svdq_repack_weight(None, fake(2), 128, 256, fake(3), need, None) == 1
    assert L.svdq_repack_weight(fake(1), fake(2), 128, 250, fake(3), need, None) == 2
    assert L.svdq_repack_weight(fake(1), fake(2), 128, 256, fake(1) + 16, need, None) == 6
    assert L.svdq_unpack_weight(fake(1), need, 128, 256, fake(1), fake(2), None) == 6
    assert L.svdq_unpack_weight(fake(1), need, 0, 256, None, None, None) == 0


def gated(**kw):
    args = dict(x=fake(1), smooth=fake(2), weight=fake(3), wcscales=fake(5), wtscale=fake(6),
                proj_down=fake(7), proj_up=fake(8), bias=None, M=64, F=128, K=256, R=16, h=fake(9),
                ws=fake(10), ws_bytes=1 << 30, stream=None)
    args.update(kw)
    L = _lib.lib()
    return L.svdq_linear_w4a4_gated(args["x"], args["smooth"], args["weight"], args["wcscales"],
                                    args["wtscale"], args["proj_down"], args["proj_up"], args["bias"],
                                    args["M"], args["F"], args["K"], args["R"], args["h"], args["ws"],
                                    args["ws_bytes"], args["stream"])


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(F=-32), 2), (dict(F=48), 3), (dict(K=40), 2), (dict(R=24), 3),
    (dict(weight=None), 1), (dict(h=None), 1), (dict(x=None), 1), (dict(wtscale=None), 1),
    (dict(proj_up=None), 1), (dict(h=fake(9) + 4), 4),
    (dict(h=fake(3)), 6),                                   # h overlaps the weight
    (dict(ws_bytes=0), 5),
    (dict(F=1 << 20, K=1 << 12), 3),                        # packed 2F-channel weight > 2 GiB
])
def test_linear_gated_rejections(kw, code):
    assert gated(**kw) == code


@no_gpu_only
def test_gated_empty_is_ok():
    assert gated(M=0) == 0
    assert gated(F=0) == 0
    L = _lib.lib()
    assert L.svdq_gemm_w4a4_gated(fake(1), fake(2), fake(3), fake(5), fake(6), fake(8), None,
                                  64, 48, 256, 16, fake(9), None) == 3


def bf16_linear(**kw):
    args = dict(x=fake(1), weight=fake(2), bias=None, M=64, N=128, K=256, y=fake(3), stream=None)
    args.update(kw)
    L = _lib.lib()
    return L.svdq_linear_bf16(args["x"], args["weight"], args["bias"], args["M"], args["N"], args["K"],
                              args["y"], args["stream"])


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), 2), (dict(N=-1), 2), (dict(K=0), 2), (dict(K=40), 2),
    (dict(x=None), 1), (dict(weight=None), 1), (dict(y=None), 1),
    (dict(y=fake(3) + 2), 4), (dict(bias=fake(4) + 8), 4),
    (dict(y=fake(1) + 64), 6),                              # y overlaps x
    (dict(bias=fake(3) + 16), 6),                           # y overlaps the bias
    (dict(N=(1 << 24) + 16), 3), (dict(M=(1 << 24) + 16), 3),
])
def test_linear_bf16_rejections(kw, code):
    assert bf16_linear(**kw) == code


@no_gpu_only
def test_linear_bf16_empty_is_ok():
    assert bf16_linear(M=0) == 0
    assert bf16_linear(N=0) == 0
    assert bf16_linear(M=0, x=None, weight=None, y=None) == 0


def prep(**kw):
    args = dict(weight=fake(1), smooth=fake(2), omega=fake(3), N=256, K=128, R=16, iters=2, qweight=fake(4),
                wscales=fake(5), wcscales=fake(6), wtscale=fake(7), pd=fake(8), pu=fake(9), ws=fake(10),
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    L = _lib.lib()
    return L.svdq_prepare_weight(args["weight"], args["smooth"], args["omega"], args["N"], args["K"], args["R"],
                                 args["iters"], args["qweight"], args["wscales"], args["wcscales"], args["wtscale"],
                                 args["pd"], args["pu"], args["ws"], args["ws_bytes"], args["stream"])


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), 2), (dict(K=40), 2), (dict(R=-16), 2), (dict(R=24), 3), (dict(R=144), 3),
    (dict(N=64, K=32, R=48), 3),                               # R above min(N, K)
    (dict(iters=-1), 8), (dict(iters=17), 8),
    (dict(weight=None), 1), (dict(omega=None), 1), (dict(pd=None), 1), (dict(ws=None), 1),
    (dict(wtscale=fake(7) + 2), 4),
    (dict(ws_bytes=0), 5),
    (dict(qweight=fake(1) + 32), 6),                           # qweight overlaps the weight
    (dict(pu=fake(10)), 6),                                    # proj_up overlaps the workspace
    (dict(N=1 << 20, K=1 << 11), 3),                           # weight of 4 GiB
])
def test_prepare_rejections(kw, code):
    assert prep(**kw) == code


@no_gpu_only
def test_prepare_empty_and_rank_zero_pointers():
    assert prep(N=0) == 0
    L = _lib.lib()
    # R = 0: omega and the factors may be NULL (rejected later only for a tiny workspace)
    assert prep(R=0, omega=None, pd=None, pu=None, ws_bytes=0) == 5
    assert L.svdq_prepare_workspace_bytes(10240, 3840, 128) >= 10240 * 3840 * 2
    assert L.svdq_prepare_workspace_bytes(0, 3840, 128) == 0


@no_gpu_only
def test_quantize_act_static_rejects_mx_layout():
    L = _lib.lib()
    assert L.svdq_quantize_act_static(fake(1), fake(2), fake(8), 64, 256, fake(3), 16, 2, fake(4), fake(5),
                                      fake(6), fake(7), 1 << 30, None) == 3
    assert "static" in L.svdq_last_error().decode()


@no_gpu_only
def test_mx_rejections_and_sizes():
    L = _lib.lib()
    assert L.svdq_mx_codes_bytes(33, 256) == 64 * 128
    assert L.svdq_mx_scales_bytes(33, 256) == 64 * 8
    assert L.svdq_mx_codes_bytes(32, 192) == 0          # K not a multiple of 128
    assert L.svdq_quantize_act_mxfp4(fake(1), fake(2), 64, 192, fake(3), fake(4), None) == 3
    assert L.svdq_quantize_act_mxfp4(fake(1), fake(2), 64, 200, fake(3), fake(4), None) == 2
    assert L.svdq_quantize_act_mxfp4(None, fake(2), 64, 256, fake(3), fake(4), None) == 1
    assert L.svdq_quantize_act_mxfp4(fake(1), fake(2), 0, 256, None, None, None) == 0
    assert L.svdq_reround_weight_mxfp4(fake(1), fake(2), 64, 256, fake(1) + 64, fake(4), None) == 6
    assert L.svdq_gemm_mxfp4(fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7), fake(8), None,
                             64, 64, 256, 24, fake(9), None) == 3
    assert L.svdq_linear_mxfp4(fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7), fake(8), None,
                               64, 64, 256, 16, fake(9), fake(10), 0, None) == 5


@pytest.mark.parametrize("value,on", [(None, 0), ("1", 1), ("true", 1), ("ON", 1), ("Yes", 1), ("0", 0),
                                      ("", 0), ("no", 0), ("off", 0), ("2", 0), ("1 ", 0), ("truetrue", 0)])
def test_debug_flag_parsing(value, on):
    """SVDQ_DEBUG is read once per process, so each value runs in a fresh interpreter."""
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("SVDQ_DEBUG", None)
    if value is not None:
        env["SVDQ_DEBUG"] = value
    code = ("import sys; sys.path.insert(0, %r); from bit_w4a4_quantized_quantize_amd import _lib; "
            "print(_lib.lib().svdq_debug_mode())" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert int(out.stdout.strip()) == on


@no_gpu_only
def test_noalloc_size_limit_and_empty():
    """The no-allocation entry point refuses a problem whose workspace exceeds its static
    scratch, on the host, before any pointer is used; empty problems succeed."""
    L = _lib.lib()
    cap = L.svdq_noalloc_scratch_bytes()
    assert cap == 64 << 20
    M, K, N, R = 16896, 10240, 3840, 128
    assert L.svdq_linear_workspace_bytes(M, N, K, R) > cap
    st = L.svdq_linear_w4a4_noalloc(fake(1), fake(2), fake(3), None, 1, fake(4), fake(5), fake(6), fake(7), None,
                                    M, N, K, R, fake(8), None)
    assert st == 5
    assert b"static scratch" in L.svdq_last_error()
    assert L.svdq_linear_w4a4_noalloc(None, None, None, None, 1, None, None, None, None, None, 0, N, K, R, None,
                                      None) == 0
    assert L.svdq_linear_w4a4_noalloc(None, None, None, None, 1, None, None, None, None, None, 64, N, 100, R, None,
                                      None) == 2   # K not a multiple of 16


@no_gpu_only
def test_calib_rejections_and_sizes():
    """The measurement helpers check their arguments on the host: sizes, formats, buffers."""
    L = _lib.lib()
    tb = L.svdq_calib_table_bytes()
    assert tb == 64 * 8 * 64 * 16
    assert L.svdq_calib_flop_per_iteration(256) == 256 * 8 * 20 * 2 * 32 * 32 * 16
    assert L.svdq_calib_scaled_flop_per_iteration(256) == 256 * 8 * 20 * 2 * 32 * 32 * 64
    assert L.svdq_calib_scaled_flop_per_iteration(0) == 0
    wg = 4
    out_b, clk_b = wg * 512 * 4, wg * 4 * 8
    args = (fake(1), tb, 10, wg)
    assert L.svdq_calib_mfma_scaled(*args, 7, fake(2), out_b, fake(3), clk_b, None) == 3    # format
    assert L.svdq_calib_mfma_scaled(*args, 4, fake(2), out_b - 4, fake(3), clk_b, None) == 5
    assert L.svdq_calib_mfma_scaled(fake(1), tb - 16, 10, wg, 0, fake(2), out_b, fake(3), clk_b, None) == 5
    assert L.svdq_calib_mfma_scaled(fake(1), tb, 0, wg, 4, fake(2), out_b, fake(3), clk_b, None) == 2
    assert L.svdq_calib_mfma_scaled(None, tb, 10, wg, 4, fake(2), out_b, fake(3), clk_b, None) == 1
    assert L.svdq_calib_mfma_scaled(*args, 4, fake(1) + 64, out_b, fake(3), clk_b, None) == 6   # overlaps table
    assert L.svdq_calib_mfma(fake(1), tb, 10, 0, fake(2), out_b, fake(3), clk_b, None) == 2
    assert L.svdq_calib_copy(fake(1), fake(2), 24, None) == 2
    assert L.svdq_calib_lds_bytes_per_iteration(256) == 256 * 512 * 8 * 16
    assert L.svdq_calib_lds(10, wg, 3, fake(2), out_b, None) == 3
    assert L.svdq_calib_lds(0, wg, 0, fake(2), out_b, None) == 2
    assert L.svdq_calib_lds(10, wg, 0, None, out_b, None) == 1
    assert L.svdq_calib_lds(10, wg, 1, fake(2), out_b - 4, None) == 5


def test_gemm_tile_override():
    """svdq_set_gemm_tile is host-only: 0..4 are taken and the previous value comes back;
    anything else is refused with SVDQ_ERR_INVALID and changes nothing."""
    L = _lib.lib()
    prev = ctypes.c_int(-1)
    assert L.svdq_set_gemm_tile(3, ctypes.byref(prev)) == 0
    try:
        assert prev.value == 0
        for bad in (-1, 5, 99):
            assert L.svdq_set_gemm_tile(bad, ctypes.byref(prev)) == 8
            assert "tile" in L.svdq_last_error().decode()
        assert L.svdq_set_gemm_tile(4, None) == 0
        assert L.svdq_set_gemm_tile(0, ctypes.byref(prev)) == 0
        assert prev.value == 4
    finally:
        L.svdq_set_gemm_tile(0, None)
