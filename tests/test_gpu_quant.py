"""GPU parity of the activation quantisation (qact, ascales): bit-exact against the oracle.

Cases: the tiny and DiT-shaped workloads (outlier channels, SwiGLU-like inputs),
the full 1024^2 activation shape, ragged M and K, exact E2M1 midpoints, signed
zeros, all-zero and underflowing blocks, saturating blocks, and sentinel-filled
outputs (every byte written, none beyond).
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import svdq as S
from tests.gpu_util import dev_bf16, host_bits, host_u8

pytestmark = pytest.mark.gpu


def run_quant(ops, x_bits, sm_bits, sentinel=True):
    M, K = x_bits.shape
    x = dev_bf16(x_bits)
    sm = dev_bf16(sm_bits)
    qbuf = torch.full((M * (K // 2) + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full(((K // 16) * M + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    qact = qbuf[: M * (K // 2)].view(M, K // 2)
    ascales = sbuf[: (K // 16) * M].view(K // 16, M)
    ops.quantize_act(x, sm, qact=qact, ascales=ascales)
    torch.cuda.synchronize()
    if sentinel:
        assert np.all(host_u8(qbuf[M * (K // 2):]) == 0xA5), "qact written past its end"
        assert np.all(host_u8(sbuf[(K // 16) * M:]) == 0x5A), "ascales written past its end"
    return host_u8(qact), host_u8(ascales)


def assert_exact(ops, x_bits, sm_bits):
    q_gpu, s_gpu = run_quant(ops, x_bits, sm_bits)
    q_ref, s_ref = S.quantize_act(x_bits, sm_bits)
    bad_s = np.argwhere(s_gpu != s_ref)
    assert bad_s.size == 0, f"ascales mismatch at {bad_s[:5].tolist()}"
    bad_q = np.argwhere(q_gpu != q_ref)
    assert bad_q.size == 0, f"qact mismatch at {bad_q[:5].tolist()}: gpu {q_gpu[tuple(bad_q[0])]:#x} ref {q_ref[tuple(bad_q[0])]:#x}"


@pytest.mark.parametrize("M,K,kind,seed", [
    (64, 256, "tiny", 1001),
    (256, 3840, "dit", 1002),
    (96, 10240, "swiglu", 1023),
    (1, 3840, "dit", 3),
    (63, 272, "dit", 4),       # K not a multiple of the 256-wide chunk
    (33, 48, "tiny", 5),       # K = 3 blocks
    (4097, 256, "dit", 6),     # ragged M beyond a tile
])
def test_quant_bit_exact(gpu_lib, M, K, kind, seed):
    x, sm = workloads.make_activation(M, K, kind=kind, seed=seed)
    assert_exact(gpu_lib, x, sm)


def test_quant_full_1024_shape(gpu_lib):
    """The 1024^2 activation (M=4096, K=3840) with outlier channels, every element."""
    cfg = workloads.FFN_W1_1024
    x, sm = workloads.make_activation(cfg["M"], cfg["K"], kind=cfg["kind"], seed=cfg["seed"])
    assert_exact(gpu_lib, x, sm)


def test_quant_exact_ties_signed_zeros_and_special_blocks(gpu_lib):
    rng = np.random.default_rng(17)
    M, K = 64, 512
    vals = np.zeros((M, K))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for m in range(M):
        for b in range(K // 16):
            kind = (m + b) % 6
            sc = F.e4m3_decode(np.array([rng.integers(0x08, 0x70)]))[0]
            blk = np.zeros(16)
            if kind == 0:      # exact midpoints times a normal scale, amax = 6 s
                blk[0] = 6 * sc
                blk[1:8] = mids * sc * np.where(rng.random(7) < 0.5, 1, -1)
                blk[8:15] = mids[::-1] * sc
            elif kind == 1:    # all zero with some negative zeros
                blk[:] = 0.0
            elif kind == 2:    # underflowing block: scale rounds to 0, signs kept
                blk[:] = rng.standard_normal(16) * 2.0 ** -24
            elif kind == 3:    # subnormal e4m3 scales
                blk[:] = rng.standard_normal(16) * 2.0 ** -7
            elif kind == 4:    # saturating: amax/6 > 448
                blk[:] = rng.standard_normal(16) * 5000
            else:              # ordinary
                blk[:] = rng.standard_normal(16)
            vals[m, 16 * b:16 * b + 16] = blk
    x = F.f64_to_bf16(vals)
    # negative zeros in the all-zero blocks
    zero_blocks = np.zeros_like(x, dtype=bool)
    for m in range(M):
        for b in range(K // 16):
            if (m + b) % 6 == 1:
                zero_blocks[m, 16 * b:16 * b + 16:3] = True
    x[zero_blocks] = 0x8000
    ones = F.f64_to_bf16(np.ones(K))
    # the tie cases must really be exact midpoints after bf16 rounding
    xv = F.bf16_to_f64(x)
    assert np.array_equal(np.abs(xv[vals != 0]), np.abs(F.bf16_to_f64(F.f64_to_bf16(vals[vals != 0]))))
    assert_exact(gpu_lib, x, ones)
    # also with a non-trivial smooth (bf16 x bf16 products, exact in fp32)
    sm = F.f64_to_bf16(np.where(np.arange(K) % 2 == 0, 0.5, 2.0))
    assert_exact(gpu_lib, x, sm)


def _special_blocks(M, K, seed):
    """x [M, K] (bf16 bits) whose 16-blocks cycle through six kinds: exact E2M1 midpoints
    times a normal e4m3 scale with amax = 6 s (ties), all zero with negative zeros, values
    whose scale underflows to 0 (signs kept), subnormal scales, saturating (amax/6 > 448), and
    ordinary normal values."""
    rng = np.random.default_rng(seed)
    nb = K // 16
    mi, bi = np.meshgrid(np.arange(M), np.arange(nb), indexing="ij")
    kind = (mi + bi) % 6
    sc = F.e4m3_decode(rng.integers(0x08, 0x70, size=(M, nb)).astype(np.uint8))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    blk = np.zeros((M, nb, 16))
    k0 = (kind == 0)[..., None]
    signs = np.where(rng.random((M, nb, 7)) < 0.5, 1.0, -1.0)
    blk[..., 0:1] = np.where(k0, 6 * sc[..., None], 0.0)
    blk[..., 1:8] = np.where(k0, mids * sc[..., None] * signs, 0.0)
    blk[..., 8:15] = np.where(k0, mids[::-1] * sc[..., None], 0.0)
    noise = rng.standard_normal((M, nb, 16))
    for k, factor in ((2, 2.0 ** -24), (3, 2.0 ** -7), (4, 5000.0), (5, 1.0)):
        blk = np.where((kind == k)[..., None], noise * factor, blk)
    x = F.f64_to_bf16(blk.reshape(M, K))
    neg0 = np.zeros((M, nb, 16), dtype=bool)
    neg0[..., 0::3] = True
    x[(neg0 & (kind == 1)[..., None]).reshape(M, K)] = 0x8000
    return x


@pytest.mark.parametrize("K", [1280, 3840])
@pytest.mark.parametrize("packed", [True, False])
def test_fused_quant_special_blocks_bit_exact(gpu_lib, K, packed):
    """The special blocks above through the fused quantise + down-projection kernels (R = 128,
    M = 2048): the split-free form at K = 1280 and the K-split form at K = 3840, in both
    output layouts. Codes and scales equal the oracle's bit for bit; each fused kernel has its
    own copy of the quantisation, so the tie, zero and saturation rules are pinned in each."""
    from oracle import repack as P
    M, R = 2048, 128
    x = _special_blocks(M, K, 31 + K)
    sm = F.f64_to_bf16(np.where(np.arange(K) % 3 == 0, 0.5, 1.0))
    pd = F.f64_to_bf16(np.random.default_rng(32).standard_normal((K, R)) * 0.02)
    q_ref, s_ref = S.quantize_act(x, sm)
    if packed:
        buf, _, _ = gpu_lib.quantize_act(dev_bf16(x), dev_bf16(sm), dev_bf16(pd), packed=True)
        torch.cuda.synchronize()
        q, s = P.unpack(host_u8(buf), M, K)
    else:
        qt, st, _ = gpu_lib.quantize_act(dev_bf16(x), dev_bf16(sm), dev_bf16(pd))
        torch.cuda.synchronize()
        q, s = host_u8(qt), host_u8(st)
    assert np.array_equal(s, s_ref), f"scales differ at {np.argwhere(s != s_ref)[:4].tolist()}"
    assert np.array_equal(q, q_ref), f"codes differ at {np.argwhere(q != q_ref)[:4].tolist()}"


def test_quant_random_bit_patterns(gpu_lib):
    """Arbitrary finite bf16 bit patterns (wide exponent range) times a random smooth."""
    rng = np.random.default_rng(23)
    M, K = 128, 1024
    x = rng.integers(0, 1 << 16, size=(M, K), dtype=np.uint64).astype(np.uint16)
    exp = (x >> 7) & 0xFF
    x = np.where((exp > 100) & (exp < 150), x, x & 0x807F | (127 << 7)).astype(np.uint16)
    sm = workloads.f32_to_bf16_bits(rng.uniform(0.25, 4.0, size=K))
    assert_exact(gpu_lib, x, sm)


def test_quant_deterministic(gpu_lib):
    x, sm = workloads.make_activation(512, 3840, kind="dit", seed=8)
    a = run_quant(gpu_lib, x, sm)
    b = run_quant(gpu_lib, x, sm)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_quant_empty(gpu_lib):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    sm = torch.ones(256, dtype=torch.bfloat16, device="cuda")
    qact, ascales, lora = gpu_lib.quantize_act(x, sm)
    assert qact.shape == (0, 128) and ascales.shape == (16, 0) and lora is None


def _unspecified_rows_mask(M, K):
    """Bytes of a packed activation buffer that belong to rows >= M (left unspecified)."""
    from oracle import repack as P
    MP, KP = -(-M // 32), -(-K // 64)
    total = P.packed_bytes(M, K)
    mask = np.zeros(total, dtype=bool)
    d = np.arange(256)
    c_of_dword = (d // 4) % 32
    for q in range(MP):
        bad_c = 32 * q + np.arange(32) >= M
        if not bad_c.any():
            continue
        for p in range(KP):
            base = 1024 * (p * MP + q)
            rows_bad = bad_c[c_of_dword]
            for k in range(4):
                mask[base + 4 * d[rows_bad] + k] = True
            sbase = 1024 * KP * MP + 128 * (p * MP + q)
            for b in range(128):
                if bad_c[b // 4]:
                    mask[sbase + b] = True
    return mask


@pytest.mark.parametrize("M,K,R,kind,seed", [
    (64, 256, 16, "tiny", 1001),
    (77, 336, 32, "dit", 51),        # ragged M, K % 64 == 16
    (600, 3840, 128, "dit", 52),
    (96, 10240, 128, "swiglu", 53),
    (130, 1024, 0, "dit", 54),       # quantisation alone into the packed layout
    (4096, 1280, 128, "swiglu", 57), # short K: the split-free fused kernel
    (2049, 1280, 96, "dit", 58),     # split-free, ragged M, a half-empty second column half
    (1000, 1040, 128, "dit", 59),    # split-free, K neither a multiple of 64 nor of 256
])
def test_quant_packed_layout_bit_exact(gpu_lib, M, K, R, kind, seed):
    """Packed activation output == the oracle's codes/scales placed by the oracle's
    own statement of the packed layout (zero beyond K; rows beyond M unspecified)."""
    from oracle import repack as P
    d = workloads.make_linear(M, K, 16, R, kind=kind, seed=seed, with_bias=False)
    buf, asc, lora = gpu_lib.quantize_act(dev_bf16(d["x"]), dev_bf16(d["smooth"]),
                                          dev_bf16(d["proj_down"]) if R > 0 else None, packed=True)
    torch.cuda.synchronize()
    assert asc is None
    got = host_u8(buf)
    q_ref, s_ref = S.quantize_act(d["x"], d["smooth"])
    expect = P.repack(q_ref, s_ref)
    assert got.size == expect.size
    keep = ~_unspecified_rows_mask(M, K)
    bad = np.argwhere((got != expect) & keep)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:4].ravel().tolist()}"
    q2, s2 = P.unpack(got, M, K)
    assert np.array_equal(q2, q_ref) and np.array_equal(s2, s_ref)


def test_quant_every_scale_with_ties_at_every_midpoint(gpu_lib):
    """For each of the 126 nonzero e4m3 scales s: a block with amax = 6 s (so the
    scale code is exactly s) holding the 7 E2M1 midpoints times s, both signs, and
    their bf16 neighbours just below and above. Exercises the exact tie handling
    (scale rule, reciprocal, 21-bit rounding) for every scale the format has."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    for code in range(1, 0x7F):
        s = F.e4m3_decode(np.array([code]))[0]
        if 6 * s > 3.0e38:
            continue
        for variant in range(3):
            blk = np.zeros(16)
            blk[0] = 6 * s
            vals = mids * s
            if variant == 1:      # next bf16 value below each midpoint
                vals = F.bf16_to_f64(F.f64_to_bf16(vals)) - F.bf16_to_f64(F.f64_to_bf16(vals)) * 2.0 ** -8
            if variant == 2:      # next bf16 value above
                vals = vals + vals * 2.0 ** -7
            blk[1:8] = vals
            blk[8:15] = -vals
            blk[15] = -6 * s
            rows.append(blk)
    vals = np.array(rows)
    x = F.f64_to_bf16(vals)
    ones = F.f64_to_bf16(np.ones(16))
    assert_exact(gpu_lib, x, ones)
    q_ref, s_ref = S.quantize_act(x, ones)
    # the tie rows really produce the intended scale codes
    assert set(np.unique(s_ref)) >= set(range(0x20, 0x7F))


def test_quant_packed_2048px_sampled_rows(gpu_lib):
    """The 2048px activation (M = 16384 + 512 tokens, K = 3840, R = 128), packed output with
    the down-projection, in the configuration the whole layer launches: codes and scales of
    48 sampled rows bit-exact (through the oracle's unpack of the whole buffer), lora_act
    of the same rows within bf16 rounding plus fp32 accumulation."""
    from oracle import repack as P
    cfg = workloads.LAYERS_2048["w1"]
    M, K, R = cfg["M"], cfg["K"], cfg["R"]
    d = workloads.make_linear(M, K, 16, R, kind=cfg["kind"], seed=cfg["seed"], with_bias=False)
    buf, _, lora = gpu_lib.quantize_act(dev_bf16(d["x"]), dev_bf16(d["smooth"]), dev_bf16(d["proj_down"]),
                                        packed=True)
    torch.cuda.synchronize()
    q_all, s_all = P.unpack(host_u8(buf), M, K)
    rows = np.sort(np.random.default_rng(61).choice(M, size=48, replace=False))
    rows[0], rows[-1] = 0, M - 1
    q_ref, s_ref = S.quantize_act(d["x"][rows], d["smooth"])
    assert np.array_equal(q_all[rows], q_ref)
    assert np.array_equal(s_all[:, rows], s_ref)
    got = F.bf16_to_f64(host_bits(lora)[rows])
    ref = S.lowrank_down(d["x"][rows], d["proj_down"])
    scale = np.abs(F.bf16_to_f64(d["x"][rows])) @ np.abs(F.bf16_to_f64(d["proj_down"]))
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + scale * K * 2.0 ** -23 + 1e-30)


@pytest.mark.parametrize("M,K,R,kind,seed", [
    (64, 256, 16, "tiny", 1001),
    (77, 336, 32, "dit", 55),        # ragged M, K % 64 == 16
    (4096, 3840, 128, "dit", 1003),  # the 1024^2 activation, K split over workgroups
    (40, 10240, 256, "swiglu", 56),  # long K, two 128-wide R chunks
    (4096, 1280, 128, "swiglu", 60), # short K: the split-free fused kernel
    (2049, 1040, 96, "dit", 61),     # split-free, ragged M and K
])
def test_quant_canonical_with_down_projection_bit_exact(gpu_lib, M, K, R, kind, seed):
    """Canonical qact/ascales written by the fused quantisation + down-projection
    kernel (R > 0) equal the oracle bit for bit; no byte past either output."""
    d = workloads.make_linear(M, K, 16, R, kind=kind, seed=seed, with_bias=False)
    qbuf = torch.full((M * (K // 2) + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full(((K // 16) * M + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    qact = qbuf[: M * (K // 2)].view(M, K // 2)
    ascales = sbuf[: (K // 16) * M].view(K // 16, M)
    gpu_lib.quantize_act(dev_bf16(d["x"]), dev_bf16(d["smooth"]), dev_bf16(d["proj_down"]),
                         qact=qact, ascales=ascales)
    torch.cuda.synchronize()
    assert np.all(host_u8(qbuf[M * (K // 2):]) == 0xA5), "qact written past its end"
    assert np.all(host_u8(sbuf[(K // 16) * M:]) == 0x5A), "ascales written past its end"
    q_ref, s_ref = S.quantize_act(d["x"], d["smooth"])
    assert np.array_equal(host_u8(ascales), s_ref)
    assert np.array_equal(host_u8(qact), q_ref)
